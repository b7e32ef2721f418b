"""The oracle's pins catch plausible mistakes.

Each case copies ``oracle/oracle.c`` to a temporary directory, plants one
mistake by text substitution (a wrong rounding, a dropped term, a wrong
constant, a transposed index, a swapped sign), builds the copy with gcc and runs
the pin suite against it.  At least one pin must fail for every mutant.  CPU
only; the planted mistakes never touch the real oracle.
"""
import os

import pytest

import oracle
from oracle import build as oracle_build
import test_oracle_backward_pins as bpins
import test_oracle_base3_pins as b3pins
import test_oracle_blend_pins as blpins
import test_oracle_nibble_pins as nbpins
import test_oracle_pins as pins

MUTANTS = {
    "weights: round half away from zero": ("float r = rintf(v);", "float r = roundf(v);"),
    "weights: scale by the mean instead of its reciprocal":
        ("s_w = (float)(1.0 / gamma);", "s_w = (float)(gamma);"),
    "weights: no clamp": ("int q = (r > 1.0f) ? 1 : (r < -1.0f ? -1 : (int)r);", "int q = (int)r;"),
    "weights: signed sum instead of absolute":
        ("r += fabs((double)R[n * K + k]);", "r += (double)R[n * K + k];"),
    "weights: natural (untransposed) bit layout":
        ("return (int)(2 * ((k % 16) / 4));", "return (int)(2 * (k % 4));"),
    "weights: byte index of the natural layout":
        ("return 4 * (k / 16) + (k % 4);", "return k / 4;"),
    "weights: unpack without the -1 offset": ("q[n * K + k] = (int8_t)(field - 1);",
                                              "q[n * K + k] = (int8_t)(field);"),
    "weights: Hadamard scale not divided by sqrt(K)":
        ("d_w = hadamard ? (float)(gamma / sqrt((double)K)) : (float)gamma;", "d_w = (float)gamma;"),
    "transform: swapped butterfly sign": ("v[i + h] = a - b;", "v[i + h] = b - a;"),
    "int8: factor 128/absmax": ("const float c = 127.0f / a;", "const float c = 128.0f / a;"),
    "int8: truncation instead of rounding": ("float r = rintf(u[k] * c);", "float r = truncf(u[k] * c);"),
    "int8: scale divided by 128": ("d_x[m] = (float)(((double)a * rstd) / 127.0);",
                                   "d_x[m] = (float)(((double)a * rstd) / 128.0);"),
    "int8: gain dropped": ("u[k] = gain ? xk * gain[k] : xk;", "u[k] = xk;"),
    "int8: absmax taken before the gain": ("if (fabsf(u[k]) > a) a = fabsf(u[k]);",
                                           "if (fabsf(xk) > a) a = fabsf(xk);"),
    "rmsnorm: eps dropped": ("const double rstd = 1.0 / sqrt(sum_sq / (double)K + (double)eps);\n"
                             "        int64_t s = 0;",
                             "const double rstd = 1.0 / sqrt(sum_sq / (double)K);\n"
                             "        int64_t s = 0;"),
    "rmsnorm: mean of squares over K-1": ("sqrt(sum_sq / (double)K + (double)eps);\n        int64_t s",
                                          "sqrt(sum_sq / (double)(K - 1) + (double)eps);\n        int64_t s"),
    "int4: factor 8/absmax": ("const float c = 7.0f / a;", "const float c = 8.0f / a;"),
    "int4: scale without sqrt(K)": ("(7.0 * sqrt_k)", "(7.0 * (double)K)"),
    "int4: transform skipped": ("oracle_fwht_f32(t, K);\n", "\n"),
    "contraction: transposed weight index": ("(int64_t)qw[n * K + k]", "(int64_t)qw[k * N + n]"),
    "contraction: sampled path ignores the offset": ("s += (int64_t)xq[m * K + k] * (int64_t)(field - 1);",
                                                     "s += (int64_t)xq[m * K + k] * (int64_t)(field);"),
    "dequant: weight scale dropped": ("* (double)d_x[m] * (double)d_w;", "* (double)d_x[m];"),
    "transpose: shift of the old column": ("(uint8_t)(field << packed_shift_of(n));",
                                           "(uint8_t)(field << packed_shift_of(k));"),
    "backward input: transposed weight index": ("* (double)qw[n * K + k];", "* (double)qw[k * N + n];"),
    "backward input: weight scale dropped": ("grad_n[m * K + k] = s * (double)d_w;", "grad_n[m * K + k] = s;"),
    "backward weight: activation scale dropped": ("(double)bf16_bits_to_float(grad_y[m * N + n]) * (double)d_x[m] *",
                                                  "(double)bf16_bits_to_float(grad_y[m * N + n]) *"),
    "backward weight: codes of the wrong token": ("(double)xq[m * K + k];", "(double)xq[k];"),
    "rmsnorm backward: r^2 in the projection": ("const double r3 = r[m] * r[m] * r[m];",
                                                "const double r3 = r[m] * r[m];"),
    "rmsnorm backward: gain missing from the direct term": ("grad_x[m * K + k] = g * r[m] * (double)grad_n",
                                                            "grad_x[m * K + k] = r[m] * (double)grad_n"),
    "rmsnorm backward: projection not divided by K": ("- xv * r3 / (double)K * dot;", "- xv * r3 * dot;"),
    "rmsnorm backward: gain gradient without r": ("(double)bf16_bits_to_float(x[m * K + k]) * r[m];",
                                                  "(double)bf16_bits_to_float(x[m * K + k]);"),
    "rmsnorm backward: eps dropped": ("r[m] = 1.0 / sqrt(ss / (double)K + (double)eps);",
                                      "r[m] = 1.0 / sqrt(ss / (double)K);"),
    "base3: offset code not added": ("c = v + 1;", "c = v;"),
    "base3: base 4 places": ("place *= 3;", "place *= 4;"),
    "base3: padding weights as digit 1": ("int c = 0;\n                if (k < K) {", "int c = 1;\n                if (k < K) {"),
    "base3 unpack: offset not removed": ("q[n * K + k] = (int8_t)(byte % 3 - 1);", "q[n * K + k] = (int8_t)(byte % 3);"),
    "base3 unpack: wrong digit divisor": ("byte /= 3;", "byte /= 4;"),
    "blend: weights not blended": ("b[k] = w + lambda * (wt - w);", "b[k] = wt;"),
    "blend: activations not blended": ("a[m * K + k] = n + lambda * (nt - n);", "a[m * K + k] = n;"),
    "blend: lambda and 1 - lambda swapped": ("a[m * K + k] = n + lambda * (nt - n);",
                                             "a[m * K + k] = nt + lambda * (n - nt);"),
    "blend: RMSNorm factor dropped": ("const double n = (double)u * rstd;", "const double n = (double)u;"),
    "blend: dequantised weights without d_w": ("const double wt = d_w * (double)qw[o * K + k];",
                                               "const double wt = (double)qw[o * K + k];"),
    "schedule: no clamp at 1": ("if (step >= total) return 1.0;\n", "\n"),
    "nibbles: code pair swapped": ("out[m * (K / 2) + 8 * g + j] = (uint8_t)((lo & 15) | ((hi & 15) << 4));",
                                   "out[m * (K / 2) + 8 * g + j] = (uint8_t)((hi & 15) | ((lo & 15) << 4));"),
    "nibbles: high nibble from the next code": ("const int hi = q[m * K + 16 * g + 8 + j];",
                                                "const int hi = q[m * K + 16 * g + 2 * j + 1];"),
    "nibbles: unpack without sign extension": ("q[m * K + 16 * g + j] = (int8_t)(lo >= 8 ? lo - 16 : lo);",
                                               "q[m * K + 16 * g + j] = (int8_t)(lo);"),
    "nibbles: range check dropped": ("if (lo < -8 || lo > 7 || hi < -8 || hi > 7) bad = 1;", ""),
    "nibbles: high nibble taken from the low bits": ("const int lo = b & 15, hi = b >> 4;",
                                                     "const int lo = b & 15, hi = b & 15;"),
}

# Pins run against every mutant (the parametrised ones at a representative size).
PIN_CALLS = [
    (pins.test_weight_codes_are_ternary_and_fields_valid, {}),
    (pins.test_packed_bytes_by_hand, {}),
    (pins.test_shift_mask_unpacks_in_natural_order, {}),
    (pins.test_pack_unpack_round_trip, {}),
    (pins.test_round_half_even_and_clamp, {}),
    (pins.test_absmean_scale_against_exact_sum, {}),
    (pins.test_zero_code_fraction_of_gaussian_weights, {}),
    (pins.test_hadamard_prerotation_of_scaled_identity, {}),
    (pins.test_fwht_equals_explicit_sylvester_matrix, {"n": 64}),
    (pins.test_fwht_is_a_hadamard_matrix, {"n": 16}),
    (pins.test_fwht_involution_and_parseval, {}),
    (pins.test_int8_codes_invariants, {}),
    (pins.test_int8_codes_power_of_two_invariance, {}),
    (pins.test_int8_codes_ties_round_to_even, {}),
    (pins.test_int8_gain_is_per_channel, {}),
    (pins.test_absmax_worked_example, {}),
    (pins.test_zero_and_tiny_tokens, {}),
    (pins.test_int4_codes_invariants, {}),
    (pins.test_int4_codes_exact_on_small_integers, {}),
    (pins.test_int_gemm_matches_integer_matmul, {}),
    (pins.test_int_gemm_all_ones_and_extremes, {}),
    (pins.test_dequant_closed_form, {}),
    (pins.test_int8_path_end_to_end_scale, {}),
    (pins.test_hadamard_path_end_to_end_scale, {}),
    (bpins.test_transpose_packed_moves_every_field, {}),
    (bpins.test_backward_input_is_the_adjoint_of_the_forward, {}),
    (bpins.test_backward_input_closed_forms, {}),
    (bpins.test_backward_weight_is_the_adjoint_of_the_forward, {}),
    (bpins.test_backward_weight_single_token_is_an_outer_product, {}),
    (bpins.test_rmsnorm_backward_matches_finite_differences, {}),
    (bpins.test_rmsnorm_backward_is_orthogonal_to_x_without_eps, {}),
    (b3pins.test_hand_computed_bytes, {}),
    (b3pins.test_five_digits_to_a_byte_is_a_bijection, {}),
    (b3pins.test_round_trip_and_padding, {"N": 4, "K": 333, "row_bytes": 80}),
    (b3pins.test_same_codes_as_the_two_bit_packing, {}),
    (blpins.test_lambda_schedule, {}),
    (blpins.test_lambda_one_is_the_bitlinear_layer, {"gain": True}),
    (blpins.test_lambda_zero_is_the_dense_layer, {"gain": True}),
    (blpins.test_blend_is_quadratic_in_lambda_over_both_operands, {"lam": 0.5}),
    (nbpins.test_hand_computed_bytes, {}),
    (nbpins.test_single_code_positions, {}),
    (nbpins.test_code_pairs_to_a_byte_is_a_bijection, {}),
    (nbpins.test_unpack_against_a_sign_extension_formula, {}),
    (nbpins.test_codes_outside_int4_are_rejected, {}),
    (nbpins.test_hadamard_codes_round_trip, {}),
]


def _failures(orc):
    failed = []
    for fn, kwargs in PIN_CALLS:
        try:
            fn(orc, **kwargs)
        except (AssertionError, ValueError):
            failed.append(fn.__name__)
    return failed


def test_unmutated_copy_passes_every_pin(tmp_path):
    lib = oracle_build.build_oracle(src=oracle_build.SRC, out=str(tmp_path / "liboracle_copy.so"))
    assert _failures(oracle.Oracle(oracle.load(lib))) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name):
    old, new = MUTANTS[name]
    with open(oracle_build.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    src_path = tmp_path / "oracle_mutant.c"
    src_path.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "liboracle_mutant.so")
    # -Wno-error: some mutants leave a variable unused
    oracle_build.build_oracle(src=str(src_path), out=lib_path, extra_flags=["-Wno-error"])
    failed = _failures(oracle.Oracle(oracle.load(lib_path)))
    assert failed, f"no pin caught the mutant '{name}'"
    os.remove(lib_path)
