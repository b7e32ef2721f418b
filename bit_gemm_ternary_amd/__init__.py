"""bit_gemm_ternary_amd: BitNet b1.58 BitLinear forward on MI355X (gfx950)."""
