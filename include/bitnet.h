/*
 * bitnet.h - C ABI of the MI355X (gfx950) BitNet b1.58 BitLinear forward pass
 * and of its straight-through-estimator backward.
 *
 * A BitLinear layer replaces a bias-free linear layer y = W x.  Its weights are
 * quantised once to the three values {-1, 0, +1} with one per-tensor scale and
 * stored packed, four weights per byte; at every forward the activations are
 * RMS-normalised and quantised per token (int8 absmax, or, for the BitNet v2
 * H-BitLinear variant, Walsh-Hadamard transform + int4 absmax), contracted
 * against the ternary weights with integer arithmetic accumulated in int32,
 * and dequantised by both scales into float32.
 *
 * Pages this follows (titles as printed on them):
 *   [FT] "LLM을 1.58비트로 파인튜닝: BitNet을 이용한 극단적인 양자화"
 *        (Hugging Face fine-tuning write-up): section "양자화 메커니즘"
 *        (per-tensor absmean weight scale, round, clamp to [-1, 1], rescale;
 *        per-token absmax int8 activations after normalisation), "계산 패러다임"
 *        (the matmul becomes integer additions), "주요 결과" (weights packed in
 *        int8 tensors), "추론 최적화 및 커스텀 커널" (weights unpacked on the fly
 *        inside the matmul), "Transformers와의 통합" (drop-in linear layer).
 *   [V2] "초저용량 LLM의 진화: BitNet v2 파헤치기 (1비트 LLM을 위한 4비트 활성화)",
 *        section "방법론" (Hadamard transform of the activations before 4-bit
 *        quantisation).
 *   [2B] "AI 혁신의 선두: 마이크로소프트의 1비트 LLM, BitNet b1.58 2B4T", section
 *        "주요 아키텍처 혁신" (ternary weights by absmean; no bias term).
 *   [QP] endplan.ai primer "양자화(quantization) 1.58bit", section
 *        "그러면 크기를 더 못줄이나요?" (absmax factor 127/absmax; dequantise by
 *        dividing by it).
 *
 * Conventions shared by every call:
 *   - All array arguments are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or keeps them after the call returns.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *     default stream) and the call returns before it completes.  Outputs are
 *     valid, and inputs may be released, once the stream has been synchronised.
 *   - Outputs must not alias inputs.
 *   - Every argument is validated on the host before anything is enqueued; on
 *     a non-OK status nothing was launched and no output was touched.  A HIP
 *     launch failure returns BITNET_ERR_HIP.  Device faults surface at the
 *     caller's next synchronising HIP call.
 *   - bitnet_last_error() returns a thread-local description of the last
 *     non-OK status returned on the calling thread.
 *   - Calls are re-entrant; concurrent calls on different streams are allowed.
 *   - Matrices are row-major.  Weights are [N][K] (out features x in
 *     features); activations and outputs are [M][K] and [M][N] (tokens first).
 *   - Shape limits: 0 <= M, N <= 2^31 - 1; 64 <= K <= 65536 with K % 64 == 0.
 *     The Hadamard calls need K to be a power of two with 256 <= K <= 32768.
 */
#ifndef BITNET_H
#define BITNET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITNET_ABI_VERSION 1

typedef enum {
    BITNET_OK = 0,
    BITNET_ERR_NULL = 1,         /* a required pointer is NULL */
    BITNET_ERR_SHAPE = 2,        /* M, N or K out of range, or K % 64 != 0 */
    BITNET_ERR_UNSUPPORTED = 3,  /* valid request the library does not implement
                                    (Hadamard with K not a power of two in [256, 32768]) */
    BITNET_ERR_ALIGN = 4,        /* a device pointer is not aligned as documented */
    BITNET_ERR_WORKSPACE = 5,    /* a workspace is missing or too small */
    BITNET_ERR_HIP = 6,          /* a HIP launch or runtime call failed */
    BITNET_ERR_VALUE = 7         /* a scalar argument is invalid (eps < 0 or not finite,
                                    hadamard not 0 or 1) */
} bitnet_status;

/*
 * Packed weight layout (a format of this library; the pages only say that the
 * ternary weights are stored packed in int8 tensors, [FT] "주요 결과"):
 *   packed is uint8 [N][K/4]; row n holds the K weights of output feature n.
 *   Read as little-endian 32-bit words, word g of a row holds weights
 *   16g .. 16g+15, weight 16g + 4i + b in bits 2i..2i+1 of byte b of the word.
 *   The 2-bit field is q + 1 (0, 1 or 2 for q = -1, 0, +1; 3 is never written).
 *   So (word >> 2i) & 0x03030303 gives the fields of weights 16g+4i .. 16g+4i+3
 *   as four bytes in order, ready for byte-wise dot products.
 */

/* Bytes of device workspace bitnet_pack_weights needs for an N x K matrix. */
size_t bitnet_pack_weights_workspace_bytes(int64_t N, int64_t K, int hadamard);

/*
 * Weight quantisation and packing ([FT] "양자화 메커니즘", weights;
 * [2B] "주요 아키텍처 혁신"; [FT] "주요 결과").  Run once per layer.
 *
 *   W          in   float32 [N][K], 16-byte aligned.
 *   N, K            N >= 1; K as in the shape limits.
 *   hadamard        0: quantise W.  1: first replace every row of W by its
 *                   unnormalised Walsh-Hadamard transform (Sylvester order),
 *                   so the layer can take Hadamard-transformed activations
 *                   (bitnet_hadamard_quant_act); needs K a power of two.
 *   packed     out  uint8 [N][K/4] in the layout above, 16-byte aligned.
 *   w_scale    out  float32 [2]: w_scale[0] = d_w, the dequantisation
 *                   multiplier: gamma = mean |W| over all N*K entries
 *                   (accumulated in float64, each row left to right then the
 *                   rows in order), rounded to float32 (hadamard = 1: gamma of
 *                   the transformed rows divided by sqrt(K));
 *                   w_scale[1] = s_w = float32(1 / gamma), the quantisation
 *                   factor.  Codes are q = clamp(rint(w * s_w), -1, 1) with
 *                   w * s_w one float32 multiply and rint round-half-to-even.
 *                   An all-zero W gives d_w = s_w = 0 and every q = 0.
 *   workspace       device scratch of at least
 *                   bitnet_pack_weights_workspace_bytes(N, K, hadamard) bytes,
 *                   16-byte aligned; contents undefined afterwards.
 */
int bitnet_pack_weights(const float* W, int64_t N, int64_t K, int hadamard, uint8_t* packed,
                        float* w_scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * bitnet_pack_weights without a caller workspace and without any allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture (weights re-packed every step of quantisation-aware training),
 * tight serving loops, harnesses that forbid hipMalloc.  It calls no hipMalloc,
 * hipFree or allocating library routine; the caller still passes W, packed and
 * w_scale, with the same meaning, layout and rules as bitnet_pack_weights.
 *
 * In place of the workspace it uses a scratch array that the library owns: a
 * static device array of BITNET_NOALLOC_SCRATCH_BYTES bytes, one per GPU the
 * library runs on, held until the process ends.  Its address on a GPU is
 * looked up on the first call on that GPU (hipGetSymbolAddress, with that GPU
 * current) and kept.  A request whose workspace would exceed the array,
 * bitnet_pack_weights_workspace_bytes(N, K, hadamard) >
 * BITNET_NOALLOC_SCRATCH_BYTES (about 524,000 rows without the rotation; N*K
 * up to about a million weights with it), returns BITNET_ERR_WORKSPACE before
 * anything is launched.
 *
 * `stream` must belong to the calling thread's current device
 * (BITNET_ERR_VALUE otherwise).  Every call on one GPU shares that GPU's
 * array and leaves its contents behind (nothing in it needs clearing: each
 * call writes every scratch word it reads): calls whose work overlaps on one
 * GPU (different streams, or threads without ordering) race on the array and
 * must be serialised by the caller.
 */
#define BITNET_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

int bitnet_pack_weights_noalloc(const float* W, int64_t N, int64_t K, int hadamard, uint8_t* packed,
                                float* w_scale, void* stream);

/*
 * Fused RMSNorm + per-token absmax int8 activation quantisation
 * ([FT] "양자화 메커니즘", activations; [QP] absmax factor 127/absmax).
 *
 *   x          in   bf16 [M][K] (raw uint16 bit patterns), 16-byte aligned.
 *   gain       in   float32 [K] RMSNorm gain, or NULL for none; 16-byte aligned.
 *   eps             RMSNorm epsilon (finite, >= 0).
 *   xq         out  int8 [M][K] codes, 16-byte aligned.
 *   x_scale    out  float32 [M]: d_x[m] = absmax * rstd / 127 (float64, then
 *                   rounded to float32), the dequantisation multiplier.
 *   x_qsum     out  int32 [M]: sum of the token's codes (needed by
 *                   bitnet_linear_forward).
 * Per token: u = x * gain (float32), a = max |u|, rstd = 1/sqrt(mean(x^2) + eps)
 * (float64).  Codes q = clamp(rint(u * float32(127 / a)), -128, 127); the
 * positive factor rstd multiplies all of a token's values, so it does not
 * change the codes and is applied only in d_x.  A token with a < 2^-120 gets
 * all-zero codes and d_x = 0.  M = 0 is a no-op.
 */
int bitnet_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M, int64_t K,
                     int8_t* xq, float* x_scale, int32_t* x_qsum, void* stream);

/*
 * H-BitLinear activations: RMSNorm + Walsh-Hadamard transform + per-token
 * absmax int4 quantisation ([V2] "방법론").
 *
 * Same arguments as bitnet_quant_act; K must be a power of two in
 * [256, 32768].  Per token: u = x * gain, t = H u with H the unnormalised
 * Sylvester Hadamard matrix (float32 butterflies, stage distance ascending
 * 1, 2, 4, ...), a = max |t|, codes q = clamp(rint(t * float32(7 / a)), -8, 7)
 * stored one per int8, d_x = a * rstd / (7 sqrt(K)) (the transform's 1/sqrt(K)
 * normalisation is folded in here).  Weights for this path are packed with
 * hadamard = 1.
 */
int bitnet_hadamard_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M,
                              int64_t K, int8_t* xq, float* x_scale, int32_t* x_qsum,
                              void* stream);

/*
 * H-BitLinear activations as true 4-bit-range floats ([V2] "방법론": 4-bit
 * activations for hardware with low-bit arithmetic).  Same computation and
 * codes as bitnet_hadamard_quant_act, written as 6-bit E3M2 floats (sign,
 * 3 exponent bits with bias 3, 2 mantissa bits), which hold every integer in
 * [-8, 8] exactly:
 *
 *   xq6   out  uint8 [M][K/4*3], 16-byte aligned (x_scale, x_qsum as before).
 *              Each group of 32 consecutive K values takes 24 bytes; value p of
 *              the group (bits 6p .. 6p+5 of its little-endian 192-bit word) is
 *              the code at K offset 16 (p % 2) + 4 (p / 8) + (p % 8) / 2.
 *
 * Consumed by bitnet_linear_forward_f6.  K a power of two in [256, 32768].
 */
int bitnet_hadamard_quant_act_f6(const uint16_t* x, const float* gain, float eps, int64_t M,
                                 int64_t K, uint8_t* xq6, float* x_scale, int32_t* x_qsum,
                                 void* stream);

/*
 * H-BitLinear activations stored at half a byte per value ([V2] "방법론":
 * 4-bit activations).  Same computation and codes as bitnet_hadamard_quant_act,
 * packed two per byte in 4-bit two's complement:
 *
 *   xq4   out  uint8 [M][K/2], 16-byte aligned (x_scale, x_qsum as before).
 *              In each group g of 16 consecutive codes, byte 8g + j holds code
 *              16g + j in its low nibble and code 16g + 8 + j in its high
 *              nibble (j = 0..7), the slot order of the packed weights.
 *
 * Consumed by bitnet_linear_forward_i4.  K a power of two in [256, 32768].
 */
int bitnet_hadamard_quant_act_i4(const uint16_t* x, const float* gain, float eps, int64_t M,
                                 int64_t K, uint8_t* xq4, float* x_scale, int32_t* x_qsum,
                                 void* stream);

/*
 * Contraction + dequantisation reading the packed 4-bit codes of
 * bitnet_hadamard_quant_act_i4 directly ([V2] "방법론"; [FT] "계산 패러다임").
 * M <= 4 tokens run a GEMV on signed 4-bit dot products (the fields of two
 * weight slots per nibble lane against the code dwords, no unpacking of the
 * codes); larger M run the int8 matrix-core GEMM with the codes expanded to
 * 16 q in registers and the sums divided by 16.  acc and y are bit-identical
 * to bitnet_linear_forward on the same codes stored one per int8.
 *
 *   xq4, x_scale, x_qsum  in  outputs of bitnet_hadamard_quant_act_i4; xq4
 *                             [M][K/2], 16-byte aligned.
 *   other arguments           as bitnet_linear_forward (K a multiple of 64).
 */
int bitnet_linear_forward_i4(const uint8_t* xq4, const float* x_scale, const int32_t* x_qsum,
                             const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                             int64_t K, float* y, int32_t* acc, void* stream);

/*
 * Ternary integer contraction + dequantisation ([FT] "계산 패러다임",
 * "추론 최적화 및 커스텀 커널", "양자화 메커니즘" rescale; [QP] dequantise).
 *
 *   xq, x_scale, x_qsum  in  outputs of bitnet_quant_act or
 *                            bitnet_hadamard_quant_act ([M][K], [M], [M]);
 *                            xq 16-byte aligned.
 *   packed, w_scale      in  outputs of bitnet_pack_weights ([N][K/4], [2]);
 *                            packed 16-byte aligned.
 *   y                    out float32 [M][N]: y = acc * d_x[m] * d_w.
 *   acc                  out int32 [M][N] accumulators, or NULL to skip.
 * acc[m][n] = sum_k q_x[m][k] * q_w[n][k], exact in int32.  y and acc need
 * 4-byte alignment.  M = 0 or N = 0 is a no-op.  Token counts M <= 4 run a
 * bandwidth-bound GEMV; larger M run an int8 matrix-core GEMM.
 */
int bitnet_linear_forward(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                          const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                          int64_t K, float* y, int32_t* acc, void* stream);

/*
 * Contraction + dequantisation with 6-bit activation codes (the xq6 layout of
 * bitnet_hadamard_quant_act_f6) on the FP4 x FP6 matrix cores ([V2] "방법론";
 * [FT] "계산 패러다임").  The offset weight codes q + 1 (0, 1, 2) are exact in
 * FP4 E2M1, the activation codes in E3M2, and every partial sum is an integer
 * below 2^24 in magnitude, so the float32 accumulation is exact: acc and y are
 * bit-identical to bitnet_linear_forward on the int8 codes.
 *
 *   xq6, x_scale, x_qsum  in  outputs of bitnet_hadamard_quant_act_f6.
 *   other arguments           as bitnet_linear_forward (K a multiple of 64).
 */
int bitnet_linear_forward_f6(const uint8_t* xq6, const float* x_scale, const int32_t* x_qsum,
                             const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                             int64_t K, float* y, int32_t* acc, void* stream);

/*
 * Fused BitLinear forward: bitnet_quant_act followed by bitnet_linear_forward
 * in one call, with the same outputs ([FT] "양자화 메커니즘", "계산 패러다임").
 *
 *   x, gain, eps         in   as bitnet_quant_act.
 *   packed, w_scale      in   as bitnet_linear_forward.
 *   xq, x_scale, x_qsum  out  as bitnet_quant_act (the codes the contraction used).
 *   y, acc               out  as bitnet_linear_forward (acc may be NULL).
 * For decode (M <= 4 tokens, and K <= 32768 / M * 4 bytes of codes per lane as
 * in the GEMV) the normalisation and quantisation run inside the contraction
 * kernel, one launch in all; larger M run the two kernels back to back.
 * N = 0 only quantises; M = 0 is a no-op.
 */
int bitnet_bitlinear_forward(const uint16_t* x, const float* gain, float eps,
                             const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                             int64_t K, int8_t* xq, float* x_scale, int32_t* x_qsum, float* y,
                             int32_t* acc, void* stream);

/*
 * Grouped BitLinear forward: several projections that read the same input
 * (q|k|v, gate|up) contracted in one launch after one quantisation of x
 * ([FT] "양자화 메커니즘", "계산 패러다임"; the activation scale is per token, so
 * the codes are shared by every projection of the token).
 *
 *   x, gain, eps         in   as bitnet_quant_act.
 *   packed               in   uint8 [N][K/4], N = sum of group_rows: the
 *                             projections' packed weights (each produced by
 *                             bitnet_pack_weights) stacked row-wise in group
 *                             order; 16-byte aligned.
 *   w_scales             in   float32 [groups][2]: each group's (d_w, s_w) as
 *                             bitnet_pack_weights wrote it (device, 4-byte aligned).
 *   group_rows           in   int64 [groups] (host): rows of each group, >= 1.
 *   groups                    1 .. 8.
 *   xq, x_scale, x_qsum  out  as bitnet_quant_act.
 *   y                    out  float32 [M][N]: for n in group g,
 *                             y[m][n] = acc[m][n] * d_x[m] * d_w[g].
 *   acc                  out  int32 [M][N], or NULL.
 * Results are bit-identical to calling bitnet_bitlinear_forward once per
 * group with that group's rows.  M = 0 is a no-op (after the shape checks);
 * errors as bitnet_bitlinear_forward, plus BITNET_ERR_SHAPE for a bad group
 * count or size.
 */
int bitnet_bitlinear_forward_grouped(const uint16_t* x, const float* gain, float eps,
                                     const uint8_t* packed, const float* w_scales,
                                     const int64_t* group_rows, int groups, int64_t M, int64_t K,
                                     int8_t* xq, float* x_scale, int32_t* x_qsum, float* y,
                                     int32_t* acc, void* stream);

/*
 * Fused H-BitLinear forward ([V2] "방법론": the layer's input is Hadamard
 * transformed and quantised to 4-bit per-token absmax codes, then contracted
 * with the ternary weights packed with hadamard = 1):
 * bitnet_hadamard_quant_act_i4 followed by bitnet_linear_forward_i4, with the
 * same outputs.
 *
 *   x, gain, eps            in   as bitnet_hadamard_quant_act_i4 (K a power of
 *                                two in [256, 32768]).
 *   packed, w_scale         in   as bitnet_linear_forward_i4 (packed with
 *                                hadamard = 1 for the layer to mean y = x W^T).
 *   xq4, x_scale, x_qsum    out  as bitnet_hadamard_quant_act_i4 (the codes the
 *                                contraction used).
 *   y, acc                  out  as bitnet_linear_forward_i4 (acc may be NULL).
 * One token (M = 1) with K in [1024, 16384] and N up to 16384 (8192 at
 * K = 16384) runs in one launch: every workgroup
 * transforms and quantises the token while its weight loads are in flight,
 * then contracts on 4-bit dot products.  Other shapes run the two kernels back
 * to back.  Codes, x_qsum and acc are bit-identical either way; x_scale (and
 * so y) may differ from the two-launch path in the last float32 bits, since
 * the float64 sum of x^2 is added in another order.  N = 0 only quantises;
 * M = 0 is a no-op; errors as bitnet_bitlinear_forward.
 */
int bitnet_hadamard_bitlinear_forward(const uint16_t* x, const float* gain, float eps,
                                      const uint8_t* packed, const float* w_scale, int64_t M,
                                      int64_t N, int64_t K, uint8_t* xq4, float* x_scale,
                                      int32_t* x_qsum, float* y, int32_t* acc, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Row-parallel shards.  When the input features K of a layer are split over G
 * devices, each holds a K slice of every token and of the packed weights
 * (columns k0/4 .. (k0 + Ks)/4 of each packed row: slices start at multiples
 * of 64).  The per-token absmax and mean of x^2 of [FT] "양자화 메커니즘" are
 * over the whole token, so a shard computes its slice's part, the parts are
 * combined across devices (a maximum and a sum; the collective itself is the
 * caller's), and the slice is quantised with the combined values: its codes
 * are then exactly those an unsharded call writes for those positions.  The
 * contraction of a slice (bitnet_linear_forward with acc) gives int32 partial
 * sums whose sum over the shards is the unsharded acc exactly ([FT]
 * "계산 패러다임": integer additions), and bitnet_dequant applies the scales.
 * ---------------------------------------------------------------------------
 */

/*
 * Per-token statistics of a K slice.
 *   x       in   bf16 [M][K] slice (its own row stride K), 16-byte aligned.
 *   gain    in   float32 [K] (this slice's part of the gain) or NULL; 16-byte aligned.
 *   amax    out  float32 [M]: max_k |x * gain| over the slice (exact).
 *   sumsq   out  float64 [M]: sum_k x^2 over the slice (squares exact in
 *                float32, summed in float32 chains and float64); 8-byte aligned.
 * K as bitnet_quant_act.  M = 0 is a no-op.
 */
int bitnet_token_stats(const uint16_t* x, const float* gain, int64_t M, int64_t K, float* amax,
                       double* sumsq, void* stream);

/*
 * Codes of a K slice from the whole token's statistics.
 *   x, gain, eps, xq    as bitnet_quant_act, for the slice (K values per token).
 *   K_total             the whole token's K (K <= K_total <= 2^24): the mean of
 *                       x^2 divides by it.
 *   amax, sumsq   in    float32 [M], float64 [M]: the maxima and sums of the
 *                       bitnet_token_stats outputs over all shards.
 *   x_scale       out   float32 [M]: d_x of the whole token (equal on every
 *                       shard; equal to the unsharded d_x up to the order of
 *                       the float64 sum of x^2).
 *   x_qsum        out   int32 [M]: the sum of this slice's codes (what the
 *                       slice's contraction subtracts).
 * Codes q = clamp(rint(u * float32(127 / amax)), -128, 127); with amax the
 * maximum over all shards the clamp never acts and the codes equal the
 * unsharded ones.  A token with amax < 2^-120 gets zero codes and d_x = 0.
 */
int bitnet_quant_act_with_stats(const uint16_t* x, const float* gain, float eps, int64_t M,
                                int64_t K, int64_t K_total, const float* amax, const double* sumsq,
                                int8_t* xq, float* x_scale, int32_t* x_qsum, void* stream);

/*
 * Dequantisation of int32 accumulators ([FT] "양자화 메커니즘" rescale; [QP]
 * dequantise): y[m][n] = (acc[m][n] * d_x[m]) * d_w, float32, in the order of
 * the contraction calls' own epilogue.
 *   acc      in   int32 [M][N] (e.g. the shards' partial sums added up),
 *                 4-byte aligned.
 *   x_scale  in   float32 [M]; w_scale in float32 [2] (d_w at [0]).
 *   y        out  float32 [M][N], 4-byte aligned.
 * M = 0 or N = 0 is a no-op.
 */
int bitnet_dequant(const int32_t* acc, const float* x_scale, const float* w_scale, int64_t M, int64_t N,
                   float* y, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Backward pass under the straight-through estimator ([FT] "Straight-Through
 * Estimator (STE)를 이용한 학습": round() is given the gradient 1, so both
 * quantisers pass the gradient through).  Seen by the estimator the forward is
 * y = n~ W~^T with n~[m][k] = d_x[m] q_x[m][k] (standing for the normalised
 * activation n = x * gain * r, r = 1 / sqrt(mean(x^2) + eps), [FT]
 * "양자화 메커니즘": normalisation before quantisation) and W~ = d_w q_w
 * (standing for the latent weights W).  These calls compute, for a loss L,
 *   dL/dn = dL/dy W~,   dL/dW = (dL/dy)^T n~,   dL/dx, dL/dgain from dL/dn.
 * They cover the end of the [FT] "동적 워밍업 양자화" schedule (lambda = 1, fully
 * quantised); with lambda < 1 the forward operands are blends of the
 * full-precision and quantised values, which is a dense float contraction and
 * not a ternary one.  Gradients are bf16 [M][N] (uint16 bit patterns); shapes
 * need N and K multiples of 64 in [64, 65536] and 0 <= M <= 2^31 - 1.
 * ---------------------------------------------------------------------------
 */

/*
 * The packed weights with the roles of N and K exchanged, for dL/dn:
 *   packed    in  uint8 [N][K/4] (bitnet_pack_weights), 16-byte aligned;
 *   packed_t  out uint8 [K][N/4], 16-byte aligned, in the packed layout along
 *                 its rows (row k, word g holds the fields of n = 16g ..
 *                 16g+15, n = 16g + 4i + b in bits 2i..2i+1 of byte b).
 * Pack once per weight update, like the forward's packing.
 */
int bitnet_transpose_packed(const uint8_t* packed, int64_t N, int64_t K, uint8_t* packed_t,
                            void* stream);

/*
 * Gradient with respect to the normalised activations (the STE input side):
 *   grad_y    in  bf16 [M][N], 16-byte aligned;
 *   packed_t  in  bitnet_transpose_packed output [K][N/4], 16-byte aligned;
 *   w_scale   in  float32 [2] from bitnet_pack_weights (d_w is w_scale[0]);
 *   grad_n    out float32 [M][K]:  grad_n[m][k] = d_w * sum_n grad_y[m][n] q_w[n][k].
 * The products grad_y * q_w (q_w in {-1, 0, 1}) are exact; the sum is
 * accumulated in float32 on the bf16 matrix cores.  M = 0 is a no-op.
 */
int bitnet_linear_backward_input(const uint16_t* grad_y, const uint8_t* packed_t,
                                 const float* w_scale, int64_t M, int64_t N, int64_t K,
                                 float* grad_n, void* stream);

/* Workspace bytes of bitnet_linear_backward_weight (0 for an invalid shape or M = 0). */
size_t bitnet_linear_backward_weight_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Gradient with respect to the latent weights (the STE weight side):
 *   grad_y     in  bf16 [M][N], 16-byte aligned;
 *   xq         in  int8 codes [M][K] of the forward (bitnet_quant_act), 16-byte aligned;
 *   x_scale    in  float32 [M], d_x of the forward;
 *   grad_w     out float32 [N][K]:  grad_w[n][k] = sum_m grad_y[m][n] d_x[m] q_x[m][k];
 *   workspace  caller-owned device scratch of
 *              bitnet_linear_backward_weight_workspace_bytes(M, N, K) bytes,
 *              16-byte aligned (transposed operands; contents undefined after).
 * grad_y * d_x is rounded once to float32 and carried as two bf16 halves
 * (relative error <= 2^-16 per term); the codes are exact; the sum over m is
 * accumulated in float32 on the bf16 matrix cores.  M = 0 writes zeros; M
 * above 2^21 is rejected with BITNET_ERR_SHAPE.
 */
int bitnet_linear_backward_weight(const uint16_t* grad_y, const int8_t* xq, const float* x_scale,
                                  int64_t M, int64_t N, int64_t K, float* grad_w,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of bitnet_rmsnorm_backward with a gain gradient (0 if invalid or M = 0). */
size_t bitnet_rmsnorm_backward_workspace_bytes(int64_t M, int64_t K);

/*
 * Backward of the RMSNorm in front of the quantiser, n = x * gain * r:
 *   x          in  bf16 [M][K] (the forward's input), gain in float32 [K] or NULL (1);
 *   grad_n     in  float32 [M][K] (bitnet_linear_backward_input);
 *   grad_x     out float32 [M][K]:
 *              grad_x[m][j] = gain[j] r grad_n[m][j] - x[m][j] r^3 / K * sum_k grad_n[m][k] x[m][k] gain[k];
 *   grad_gain  out float32 [K] or NULL:  grad_gain[k] = sum_m grad_n[m][k] x[m][k] r[m];
 *   workspace  needed only with grad_gain: bitnet_rmsnorm_backward_workspace_bytes(M, K)
 *              bytes, 16-byte aligned.
 * r and both sums in float64, results rounded to float32.  Arrays 4-byte aligned.
 * M = 0 writes zeros to grad_gain (if given).
 */
int bitnet_rmsnorm_backward(const uint16_t* x, const float* gain, float eps, const float* grad_n,
                            int64_t M, int64_t K, float* grad_x, float* grad_gain, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Base-3 packing ("1.58 bits" per weight: a ternary weight carries log2 3 bits,
 * primer on 1.58-bit quantisation, section "1.58비트는 어디서 나온거에요?"):
 * five weights per byte, byte j of a row = c_0 + 3 c_1 + 9 c_2 + 27 c_3 + 81 c_4
 * with c_i = q[5j + i] + 1 (weights past K count as 0), rows padded with zero
 * bytes to bitnet_base3_row_bytes(K) = ceil(ceil(K / 5) / 16) * 16 bytes
 * (0 for an invalid K): 1.6 bits per weight.
 */
size_t bitnet_base3_row_bytes(int64_t K);

/*
 * Repack 2-bit packed weights (bitnet_pack_weights, [N][K/4], 16-byte aligned)
 * into the base-3 layout packed3 [N][bitnet_base3_row_bytes(K)] (16-byte
 * aligned); d_w and s_w are unchanged.  Same N and K rules as the packing.
 */
int bitnet_pack_base3(const uint8_t* packed, int64_t N, int64_t K, uint8_t* packed3, void* stream);

/*
 * bitnet_linear_forward for one token on base-3 packed weights: the same
 * codes, int32 accumulators and outputs as bitnet_linear_forward on the 2-bit
 * packing they came from.  M must be 0 or 1 and K at most 20480
 * (BITNET_ERR_UNSUPPORTED otherwise); xq and packed3 16-byte aligned.
 */
int bitnet_linear_forward_base3(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                                const uint8_t* packed3, const float* w_scale, int64_t M, int64_t N,
                                int64_t K, float* y, int32_t* acc, void* stream);

/*
 * The layer during the warm-up of quantisation ([FT] "동적 워밍업 양자화"):
 * with lambda = min(step / total_steps, 1), each operand is moved from its
 * full-precision value toward its quantised value by lambda, v + lambda
 * (Q(v) - v), so lambda = 0 is the dense layer and lambda = 1 the BitLinear
 * layer:
 *   a[m][k] = n + lambda (d_x[m] q_x[m][k] - n),  n = x[m][k] gain[k] rstd[m]
 *             (RMSNorm output; q_x, d_x the int8 codes and scale of
 *             bitnet_quant_act, rstd = 1 / sqrt(mean_k x^2 + eps))
 *   b[o][k] = W[o][k] + lambda (d_w q_w[o][k] - W[o][k])
 *   y[m][o] = sum_k a[m][k] b[o][k]
 * computed in float32 (operands blended in float32, float32 matrix-core sums).
 *
 *   x        in   bf16 [M][K], 16-byte aligned; gain [K] or NULL, eps >= 0.
 *   W        in   float32 [N][K] full-precision weights, 16-byte aligned.
 *   packed, w_scale  in  bitnet_pack_weights(W) outputs (hadamard = 0).
 *   lambda        in [0, 1] (BITNET_ERR_VALUE otherwise).
 *   y        out  float32 [M][N], 4-byte aligned.
 *   workspace     at least bitnet_linear_forward_blend_workspace_bytes(M, K)
 *                 bytes, 16-byte aligned (blended activations, int8 codes,
 *                 scales); contents undefined afterwards.
 * M = 0 or N = 0 is a no-op.
 */
size_t bitnet_linear_forward_blend_workspace_bytes(int64_t M, int64_t K);
int bitnet_linear_forward_blend(const uint16_t* x, const float* gain, float eps, const float* W,
                                const uint8_t* packed, const float* w_scale, float lambda, int64_t M, int64_t N,
                                int64_t K, float* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement reference, no passage of the pages: one plain read of `bytes`
 * bytes of device memory at `buf` (16-byte aligned, bytes a multiple of 16 and
 * >= 16), each byte once with 16-byte loads over the whole chip.  Its rate is
 * what a simple streaming kernel reaches on this GPU, against which the
 * bandwidth-bound kernels are also stated.  `sink` (device, 4 bytes, 4-byte
 * aligned) receives a word only on a data pattern that does not occur in
 * practice; its contents are otherwise left as they are.
 */
int bitnet_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/*
 * Profiling hook: arm two hipEvent_t (passed as void*; either may be NULL) for
 * the first kernel the next bitnet_* call on this thread launches (the
 * contraction kernel of bitnet_linear_forward, the quantisation kernel of the
 * quantisation calls and of bitnet_bitlinear_forward when M > 4, the fused
 * kernel of bitnet_bitlinear_forward when M <= 4).  That kernel is then launched with
 * hipExtLaunchKernelGGL, which records `start_event` / `stop_event` at the
 * start and end of its execution, so hipEventElapsedTime gives the kernel's
 * duration without dispatch gaps.  The events are disarmed when that call
 * returns, whether it launched or not.  Always returns BITNET_OK.
 */
int bitnet_set_kernel_events(void* start_event, void* stop_event);

/* Static text for a status code. */
const char* bitnet_status_string(int status);

/* Thread-local detail of the last non-OK status on this thread ("" if none). */
const char* bitnet_last_error(void);

/* BITNET_ABI_VERSION of the loaded library. */
int bitnet_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_H */
