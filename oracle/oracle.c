/*
 * oracle.c - plain, slow CPU oracle of the BitNet b1.58 BitLinear forward pass
 * and of its BitNet v2 H-BitLinear variant.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The GPU library never
 * links, includes or calls it, and it shares no code with the GPU library.
 *
 * Every function below is the literal definition of one step, written as
 * nested loops in IEEE float32 / float64 with no blocking, fusion or
 * reordering.  Build with `-O2 -ffp-contract=off` (no FMA contraction, no
 * fast-math) so that each float operation written here is one IEEE rounding.
 *
 * Pages cited (titles as they appear on the pages):
 *   [FT]  "LLM을 1.58비트로 파인튜닝: BitNet을 이용한 극단적인 양자화"
 *         (Hugging Face fine-tuning write-up), sections
 *         "양자화 메커니즘" (quantization mechanism), "계산 패러다임"
 *         (computation paradigm), "주요 결과" (main results).
 *   [V2]  "초저용량 LLM의 진화: BitNet v2 파헤치기 (1비트 LLM을 위한 4비트 활성화)",
 *         section "방법론" (method).
 *   [2B]  "AI 혁신의 선두: 마이크로소프트의 1비트 LLM, BitNet b1.58 2B4T",
 *         sections "주요 아키텍처 혁신" (architecture) and
 *         "훈련 안정성 및 효율성 향상" (normalisation before quantisation).
 *   [FT]  also sections "Straight-Through Estimator (STE)를 이용한 학습"
 *         (training through round() with the gradient taken as 1) and
 *         "동적 워밍업 양자화" (the lambda warm-up blend).
 *   [QP]  endplan.ai quantization primer "양자화(quantization) 1.58bit",
 *         sections "그러면 크기를 더 못줄이나요?" (absmax example) and
 *         "1.58비트는 어디서 나온거에요?" (three weight values).
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *   - "round" is round-half-to-even (rintf under the default rounding mode).
 *   - The weight absmean is accumulated in float64: each row left to right,
 *     then the row sums top to bottom.
 *   - The normalisation is RMSNorm without mean subtraction.  Its positive
 *     per-token factor 1/rms is folded into the dequantisation scale, so the
 *     activation codes are computed from u = x * gain alone (absmax
 *     quantisation is invariant to a positive per-token factor).
 *   - int8 codes use the factor 127/absmax; int4 codes use 7/absmax and the
 *     range [-8, 7].
 *   - The Hadamard transform is the unnormalised Sylvester-order transform,
 *     computed by butterflies with the stage distance ascending 1, 2, 4, ...;
 *     its 1/sqrt(K) normalisation is folded into the float scales.
 *   - Packed int4 storage: two codes per byte, 4-bit two's complement; in
 *     each group of 16 codes, byte j holds code j in its low nibble and code
 *     8 + j in its high nibble (the slot order of the 2-bit weight packing).
 *   - Packed layout: row n of the [N][K] weight matrix owns K/4 bytes; the
 *     32-bit little-endian word g of the row holds weights 16g .. 16g+15, and
 *     weight 16g + 4i + b lives in bits 2i..2i+1 of byte b of that word.  The
 *     stored 2-bit field is q + 1, so it takes the values 0, 1 and 2.
 *
 * Parity pins for every function live in the oracle self-tests.  Nothing here
 * is "parity unpinned".
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_VERSION 4

int oracle_version(void) { return ORACLE_VERSION; }

/* Threads the OpenMP loops below use (for reporting CPU timings). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Sets the thread count of later calls (n >= 1), for one-core timings. */
void oracle_set_num_threads(int n) { omp_set_num_threads(n < 1 ? 1 : n); }

/* bfloat16 bits -> float32 (exact: bf16 is the top half of a float32). */
static float bf16_bits_to_float(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ------------------------------------------------------------------------- */
/* Packed-weight layout helpers.                                             */
/* ------------------------------------------------------------------------- */

/* Byte offset (inside one packed row) and bit shift of weight k. */
static int64_t packed_byte_of(int64_t k) { return 4 * (k / 16) + (k % 4); }
static int packed_shift_of(int64_t k) { return (int)(2 * ((k % 16) / 4)); }

/*
 * Unpack a packed [N][K/4] matrix into ternary values q in {-1, 0, +1}.
 * Returns the number of 2-bit fields equal to 3 (an invalid code; 0 for any
 * matrix written by oracle_pack_weights).  Invalid fields are stored as 0.
 */
int64_t oracle_unpack_weights(const uint8_t* packed, int64_t N, int64_t K, int8_t* q) {
    int64_t bad = 0;
    const int64_t row_bytes = K / 4;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            int field = (packed[n * row_bytes + packed_byte_of(k)] >> packed_shift_of(k)) & 3;
            if (field == 3) {
                bad++;
                q[n * K + k] = 0;
            } else {
                q[n * K + k] = (int8_t)(field - 1);
            }
        }
    }
    return bad;
}

/* ------------------------------------------------------------------------- */
/* Walsh-Hadamard transform ([V2] "방법론": Hadamard transform of the        */
/* activations before 4-bit quantisation).                                   */
/* ------------------------------------------------------------------------- */

/*
 * In-place unnormalised Walsh-Hadamard transform of v[0..n) in float32,
 * Sylvester (natural) order: the result is H v with H[i][j] = (-1)^popcount(i&j).
 * n must be a power of two.  Stages run with the butterfly distance h
 * ascending; each butterfly replaces (a, b) by (a + b, a - b), one float32
 * rounding each.
 */
void oracle_fwht_f32(float* v, int64_t n) {
    for (int64_t h = 1; h < n; h *= 2) {
        for (int64_t i = 0; i < n; i++) {
            if ((i & h) == 0) {
                float a = v[i];
                float b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* O1: weight quantisation and packing ([FT] "양자화 메커니즘", Weights;     */
/* [2B] "주요 아키텍처 혁신": absmean mapping to {-1, 0, +1};                 */
/* [FT] "주요 결과": weights stored packed in int8 tensors).                  */
/* ------------------------------------------------------------------------- */

/*
 * W: float32 [N][K] row-major (out features x in features).
 * hadamard = 1: first replace every row by its Walsh-Hadamard transform
 *   (weights pre-rotated by the same transform the H-BitLinear activations
 *   get), then quantise the rotated rows.
 * Outputs:
 *   packed  [N][K/4] bytes in the layout described at the top of this file.
 *   w_scale [2]: w_scale[0] = d_w, the dequantisation multiplier
 *                (mean |W|, divided by sqrt(K) when hadamard = 1);
 *                w_scale[1] = s_w, the quantisation factor 1 / mean |W|.
 *   q_out   [N][K] ternary values (may be NULL).
 * Requires K % 16 == 0 (and K a power of two when hadamard = 1).
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int oracle_pack_weights(const float* W, int64_t N, int64_t K, int hadamard,
                        uint8_t* packed, float* w_scale, int8_t* q_out) {
    if (N < 1 || K < 16 || K % 16 != 0) return -1;
    if (hadamard && (K & (K - 1)) != 0) return -1;

    float* R = (float*)malloc((size_t)N * (size_t)K * sizeof(float));
    if (!R) return -1;
    memcpy(R, W, (size_t)N * (size_t)K * sizeof(float));
    if (hadamard) {
        for (int64_t n = 0; n < N; n++) oracle_fwht_f32(R + n * K, K);
    }

    /* Mean absolute value in float64: rows left to right, then rows in order. */
    double* row_sum = (double*)malloc((size_t)N * sizeof(double));
    if (!row_sum) {
        free(R);
        return -1;
    }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        double r = 0.0;
        for (int64_t k = 0; k < K; k++) r += fabs((double)R[n * K + k]);
        row_sum[n] = r;
    }
    double S = 0.0;
    for (int64_t n = 0; n < N; n++) S += row_sum[n];
    free(row_sum);

    const double gamma = S / ((double)N * (double)K);
    float s_w, d_w;
    if (gamma == 0.0) {
        s_w = 0.0f; /* all-zero matrix: every code is 0 */
        d_w = 0.0f;
    } else {
        s_w = (float)(1.0 / gamma);
        d_w = hadamard ? (float)(gamma / sqrt((double)K)) : (float)gamma;
    }
    w_scale[0] = d_w;
    w_scale[1] = s_w;

    /* Scale, round half to even, clamp to [-1, 1]; store q + 1 in 2 bits. */
    const int64_t row_bytes = K / 4;
    memset(packed, 0, (size_t)N * (size_t)row_bytes);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            float v = R[n * K + k] * s_w;
            float r = rintf(v);
            int q = (r > 1.0f) ? 1 : (r < -1.0f ? -1 : (int)r);
            if (q_out) q_out[n * K + k] = (int8_t)q;
            packed[n * row_bytes + packed_byte_of(k)] |= (uint8_t)((q + 1) << packed_shift_of(k));
        }
    }
    free(R);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O2: RMSNorm + per-token absmax int8 quantisation ([FT] "양자화 메커니즘", */
/* Activations: absmax per token into [-128, 127], normalisation first;      */
/* [QP] absmax example: multiply by 127/absmax, dequantise by dividing).     */
/* ------------------------------------------------------------------------- */

/* Tokens whose absmax is below this are treated as all-zero. */
static const float TINY_ABSMAX = 0x1p-120f;

/*
 * x: bf16 bits [M][K]; gain: float32 [K] or NULL (no gain); eps: RMSNorm eps.
 * Outputs per token m:
 *   q[m][k]  int8 codes in [-128, 127]
 *   d_x[m]   float32 dequantisation multiplier absmax * rstd / 127
 *   qsum[m]  int32 sum of the token's codes
 */
int oracle_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M, int64_t K,
                     int8_t* q, float* d_x, int32_t* qsum) {
    if (M < 0 || K < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        float* u = (float*)malloc((size_t)K * sizeof(float));
        double sum_sq = 0.0;
        float a = 0.0f;
        for (int64_t k = 0; k < K; k++) {
            float xk = bf16_bits_to_float(x[m * K + k]);
            sum_sq += (double)xk * (double)xk;
            u[k] = gain ? xk * gain[k] : xk;
            if (fabsf(u[k]) > a) a = fabsf(u[k]);
        }
        const double rstd = 1.0 / sqrt(sum_sq / (double)K + (double)eps);
        int64_t s = 0;
        if (a < TINY_ABSMAX) {
            for (int64_t k = 0; k < K; k++) q[m * K + k] = 0;
            d_x[m] = 0.0f;
        } else {
            const float c = 127.0f / a;
            for (int64_t k = 0; k < K; k++) {
                float r = rintf(u[k] * c);
                if (r > 127.0f) r = 127.0f;
                if (r < -128.0f) r = -128.0f;
                q[m * K + k] = (int8_t)r;
                s += (int64_t)r;
            }
            d_x[m] = (float)(((double)a * rstd) / 127.0);
        }
        qsum[m] = (int32_t)s;
        free(u);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O3: RMSNorm + Walsh-Hadamard transform + per-token absmax int4            */
/* quantisation ([V2] "방법론": Hadamard transform before 4-bit activation    */
/* quantisation; 1/sqrt(K) normalisation folded into d_x).                    */
/* ------------------------------------------------------------------------- */

/*
 * Same arguments as oracle_quant_act; K must be a power of two.
 * Codes are in [-8, 7] (stored one per int8); d_x = absmax(t) * rstd / (7 sqrt K)
 * where t is the unnormalised transform of u.
 */
int oracle_hadamard_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M,
                              int64_t K, int8_t* q, float* d_x, int32_t* qsum) {
    if (M < 0 || K < 1 || (K & (K - 1)) != 0) return -1;
    const double sqrt_k = sqrt((double)K);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        float* t = (float*)malloc((size_t)K * sizeof(float));
        double sum_sq = 0.0;
        for (int64_t k = 0; k < K; k++) {
            float xk = bf16_bits_to_float(x[m * K + k]);
            sum_sq += (double)xk * (double)xk;
            t[k] = gain ? xk * gain[k] : xk;
        }
        const double rstd = 1.0 / sqrt(sum_sq / (double)K + (double)eps);
        oracle_fwht_f32(t, K);
        float a = 0.0f;
        for (int64_t k = 0; k < K; k++)
            if (fabsf(t[k]) > a) a = fabsf(t[k]);
        int64_t s = 0;
        if (a < TINY_ABSMAX) {
            for (int64_t k = 0; k < K; k++) q[m * K + k] = 0;
            d_x[m] = 0.0f;
        } else {
            const float c = 7.0f / a;
            for (int64_t k = 0; k < K; k++) {
                float r = rintf(t[k] * c);
                if (r > 7.0f) r = 7.0f;
                if (r < -8.0f) r = -8.0f;
                q[m * K + k] = (int8_t)r;
                s += (int64_t)r;
            }
            d_x[m] = (float)(((double)a * rstd) / (7.0 * sqrt_k));
        }
        qsum[m] = (int32_t)s;
        free(t);
    }
    return 0;
}

/*
 * Packed storage of the int4 codes ([V2] "방법론": the 4-bit activations take
 * half a byte each).  The pages fix no byte layout.  The one used here packs
 * each group of 16 consecutive codes into 8 bytes the way the 2-bit weight
 * packing places its fields: nibble slot i (0 low, 1 high) of byte j holds
 * code 16g + 8i + j, in 4-bit two's complement:
 *   out[m][8g + j] = (q[m][16g + j] & 15) | ((q[m][16g + 8 + j] & 15) << 4).
 * q [M][K] (K a multiple of 16) -> out [M][K/2].  Returns -1 on a bad shape or
 * on a code outside [-8, 7] (such a code has no 4-bit two's complement form).
 */
int oracle_pack_nibbles(const int8_t* q, int64_t M, int64_t K, uint8_t* out) {
    if (M < 0 || K < 16 || K % 16 != 0) return -1;
    int bad = 0;
    for (int64_t m = 0; m < M; m++) {
        for (int64_t g = 0; g < K / 16; g++) {
            for (int64_t j = 0; j < 8; j++) {
                const int lo = q[m * K + 16 * g + j];
                const int hi = q[m * K + 16 * g + 8 + j];
                if (lo < -8 || lo > 7 || hi < -8 || hi > 7) bad = 1;
                out[m * (K / 2) + 8 * g + j] = (uint8_t)((lo & 15) | ((hi & 15) << 4));
            }
        }
    }
    return bad ? -1 : 0;
}

/* The inverse: nibble v in 0..15 is the code v - 16 if v >= 8, else v. */
int oracle_unpack_nibbles(const uint8_t* packed, int64_t M, int64_t K, int8_t* q) {
    if (M < 0 || K < 16 || K % 16 != 0) return -1;
    for (int64_t m = 0; m < M; m++) {
        for (int64_t g = 0; g < K / 16; g++) {
            for (int64_t j = 0; j < 8; j++) {
                const int b = packed[m * (K / 2) + 8 * g + j];
                const int lo = b & 15, hi = b >> 4;
                q[m * K + 16 * g + j] = (int8_t)(lo >= 8 ? lo - 16 : lo);
                q[m * K + 16 * g + 8 + j] = (int8_t)(hi >= 8 ? hi - 16 : hi);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O4: integer contraction ([FT] "계산 패러다임": the ternary matmul needs    */
/* only integer additions; accumulated in int32).                            */
/* ------------------------------------------------------------------------- */

/* acc[m][n] = sum_k xq[m][k] * q_w[n][k], q_w unpacked from packed [N][K/4]. */
int oracle_int_gemm(const int8_t* xq, const uint8_t* packed, int64_t M, int64_t N, int64_t K,
                    int32_t* acc) {
    if (M < 0 || N < 0 || K < 16 || K % 16 != 0) return -1;
    int8_t* qw = (int8_t*)malloc((size_t)N * (size_t)K);
    if (!qw) return -1;
    oracle_unpack_weights(packed, N, K, qw);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; k++) s += (int64_t)xq[m * K + k] * (int64_t)qw[n * K + k];
            acc[m * N + n] = (int32_t)s;
        }
    }
    free(qw);
    return 0;
}

/*
 * The same contraction for a list of (m, n) output positions only, for
 * spot checks of full-size problems.  acc_out[i] = acc[rows[i]][cols[i]].
 */
int oracle_int_gemm_sampled(const int8_t* xq, const uint8_t* packed, int64_t M, int64_t N,
                            int64_t K, const int64_t* rows, const int64_t* cols, int64_t count,
                            int32_t* acc_out) {
    if (K < 16 || K % 16 != 0) return -1;
    const int64_t row_bytes = K / 4;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++) {
        const int64_t m = rows[i], n = cols[i];
        int64_t s = 0;
        if (m < 0 || m >= M || n < 0 || n >= N) {
            acc_out[i] = 0;
            continue;
        }
        for (int64_t k = 0; k < K; k++) {
            int field = (packed[n * row_bytes + packed_byte_of(k)] >> packed_shift_of(k)) & 3;
            s += (int64_t)xq[m * K + k] * (int64_t)(field - 1);
        }
        acc_out[i] = (int32_t)s;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O5: dequantisation by both scales ([FT] "양자화 메커니즘": weights are     */
/* rescaled after rounding; [QP]: dequantise by dividing by the factor).     */
/* ------------------------------------------------------------------------- */

/* y[m][n] = acc[m][n] * d_x[m] * d_w, in float64. */
void oracle_dequant(const int32_t* acc, const float* d_x, float d_w, int64_t M, int64_t N,
                    double* y) {
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            y[m * N + n] = (double)acc[m * N + n] * (double)d_x[m] * (double)d_w;
}

/* ------------------------------------------------------------------------- */
/* Backward pass under the straight-through estimator ([FT] "Straight-      */
/* Through Estimator (STE)를 이용한 학습": round() is given gradient 1, so    */
/* the quantisers pass the gradient through unchanged).                      */
/*                                                                           */
/* Seen by the estimator, the forward is y = n~ W~^T with the dequantised    */
/* operands n~[m][k] = d_x[m] q_x[m][k] (which stands for the normalised     */
/* activation n = x * gain * r, r = 1 / sqrt(mean(x^2) + eps)) and           */
/* W~[n][k] = d_w q_w[n][k] (which stands for W).  So                        */
/*   dL/dn = dL/dy W~,   dL/dW = (dL/dy)^T n~,                               */
/* and dL/dx follows from the RMSNorm that produced n.                       */
/* ------------------------------------------------------------------------- */

/*
 * The packed weights with the roles of N and K exchanged: packed [N][K/4] ->
 * packed_t [K][N/4], in the same layout along the new row (row k, word g holds
 * weights n = 16g .. 16g+15, weight 16g + 4i + b in bits 2i..2i+1 of byte b).
 * N and K must be multiples of 16.  The field values (q + 1) are copied as is.
 */
int oracle_transpose_packed(const uint8_t* packed, int64_t N, int64_t K, uint8_t* packed_t) {
    if (N < 16 || K < 16 || N % 16 != 0 || K % 16 != 0) return -1;
    const int64_t row_bytes = K / 4, row_bytes_t = N / 4;
    memset(packed_t, 0, (size_t)K * (size_t)row_bytes_t);
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            int field = (packed[n * row_bytes + packed_byte_of(k)] >> packed_shift_of(k)) & 3;
            packed_t[k * row_bytes_t + packed_byte_of(n)] |= (uint8_t)(field << packed_shift_of(n));
        }
    }
    return 0;
}

/*
 * Gradient with respect to the normalised activations:
 * grad_n[m][k] = d_w * sum_n grad_y[m][n] * q_w[n][k], in float64 (the sum
 * runs over n in order).  grad_y is bf16 [M][N]; packed is the forward's
 * [N][K/4] matrix.
 */
int oracle_linear_backward_input(const uint16_t* grad_y, const uint8_t* packed, float d_w,
                                 int64_t M, int64_t N, int64_t K, double* grad_n) {
    if (M < 0 || N < 1 || K < 16 || K % 16 != 0) return -1;
    int8_t* qw = (int8_t*)malloc((size_t)N * (size_t)K);
    if (!qw) return -1;
    oracle_unpack_weights(packed, N, K, qw);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t k = 0; k < K; k++) {
            double s = 0.0;
            for (int64_t n = 0; n < N; n++)
                s += (double)bf16_bits_to_float(grad_y[m * N + n]) * (double)qw[n * K + k];
            grad_n[m * K + k] = s * (double)d_w;
        }
    }
    free(qw);
    return 0;
}

/*
 * Gradient with respect to the latent weights:
 * grad_w[n][k] = sum_m grad_y[m][n] * d_x[m] * q_x[m][k], in float64 (the sum
 * runs over m in order).  grad_y bf16 [M][N], q_x int8 [M][K], d_x float32 [M].
 */
int oracle_linear_backward_weight(const uint16_t* grad_y, const int8_t* xq, const float* d_x,
                                  int64_t M, int64_t N, int64_t K, double* grad_w) {
    if (M < 0 || N < 1 || K < 1) return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            double s = 0.0;
            for (int64_t m = 0; m < M; m++)
                s += (double)bf16_bits_to_float(grad_y[m * N + n]) * (double)d_x[m] *
                     (double)xq[m * K + k];
            grad_w[n * K + k] = s;
        }
    }
    return 0;
}

/*
 * Backward of the RMSNorm that feeds the quantiser ([FT] "양자화 메커니즘":
 * the activations are normalised before quantisation): n[m][k] = x[m][k] * g[k] * r[m]
 * with r[m] = 1 / sqrt(sum_k x[m][k]^2 / K + eps) and g = gain (1 if NULL).
 * Given grad_n (float32 [M][K]) it returns, in float64,
 *   grad_x[m][j] = g[j] r grad_n[m][j] - x[m][j] r^3 / K * sum_k grad_n[m][k] x[m][k] g[k]
 *   grad_gain[k] = sum_m grad_n[m][k] x[m][k] r[m]          (if grad_gain != NULL)
 * which is the derivative of n written out.
 */
int oracle_rmsnorm_backward(const uint16_t* x, const float* gain, float eps, const float* grad_n,
                            int64_t M, int64_t K, double* grad_x, double* grad_gain) {
    if (M < 0 || K < 1) return -1;
    double* r = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
    if (!r) return -1;
    for (int64_t m = 0; m < M; m++) {
        double ss = 0.0, dot = 0.0;
        for (int64_t k = 0; k < K; k++) {
            const double xv = (double)bf16_bits_to_float(x[m * K + k]);
            ss += xv * xv;
        }
        r[m] = 1.0 / sqrt(ss / (double)K + (double)eps);
        for (int64_t k = 0; k < K; k++) {
            const double xv = (double)bf16_bits_to_float(x[m * K + k]);
            const double g = gain ? (double)gain[k] : 1.0;
            dot += (double)grad_n[m * K + k] * xv * g;
        }
        const double r3 = r[m] * r[m] * r[m];
        for (int64_t k = 0; k < K; k++) {
            const double xv = (double)bf16_bits_to_float(x[m * K + k]);
            const double g = gain ? (double)gain[k] : 1.0;
            grad_x[m * K + k] = g * r[m] * (double)grad_n[m * K + k] - xv * r3 / (double)K * dot;
        }
    }
    if (grad_gain) {
        for (int64_t k = 0; k < K; k++) {
            double s = 0.0;
            for (int64_t m = 0; m < M; m++)
                s += (double)grad_n[m * K + k] * (double)bf16_bits_to_float(x[m * K + k]) * r[m];
            grad_gain[k] = s;
        }
    }
    free(r);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Base-3 packing ([QP] "1.58비트는 어디서 나온거에요?": a ternary weight    */
/* carries log2 3 = 1.58 bits, so five of them fit one byte, 3^5 = 243).     */
/* ------------------------------------------------------------------------- */

/*
 * Ternary codes q [N][K] in {-1, 0, 1} -> packed3 [N][row_bytes]: byte j of a
 * row holds the weights 5j .. 5j+4 as the base-3 number
 *   c_0 + 3 c_1 + 9 c_2 + 27 c_3 + 81 c_4,   c_i = q[5j + i] + 1 in {0, 1, 2},
 * so every byte is at most 242.  Weights past K count as c = 0, and bytes past
 * ceil(K / 5) are zero.  row_bytes must hold ceil(K / 5) bytes.  Returns -1 on
 * a bad argument or a code outside {-1, 0, 1}.
 */
int oracle_pack_base3(const int8_t* q, int64_t N, int64_t K, int64_t row_bytes, uint8_t* packed3) {
    if (N < 0 || K < 1 || row_bytes < (K + 4) / 5) return -1;
    int bad = 0;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t j = 0; j < row_bytes; j++) {
            int byte = 0, place = 1;
            for (int i = 0; i < 5; i++) {
                const int64_t k = 5 * j + i;
                int c = 0;
                if (k < K) {
                    const int v = q[n * K + k];
                    if (v < -1 || v > 1) bad = 1;
                    c = v + 1;
                }
                byte += c * place;
                place *= 3;
            }
            packed3[n * row_bytes + j] = (uint8_t)byte;
        }
    }
    return bad ? -1 : 0;
}

/*
 * The inverse: the base-3 digits of each byte, c_i = (byte / 3^i) mod 3, back
 * to q = c - 1 for the K weights of each row.  Returns the number of bytes
 * above 242 (not base-3 packings of five digits); their digits are still
 * decoded.
 */
int64_t oracle_unpack_base3(const uint8_t* packed3, int64_t N, int64_t K, int64_t row_bytes, int8_t* q) {
    int64_t bad = 0;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t j = 0; j < row_bytes; j++) {
            int byte = packed3[n * row_bytes + j];
            if (byte > 242) bad++;
            for (int i = 0; i < 5; i++) {
                const int64_t k = 5 * j + i;
                if (k < K) q[n * K + k] = (int8_t)(byte % 3 - 1);
                byte /= 3;
            }
        }
    }
    return bad;
}

/* ------------------------------------------------------------------------- */
/* Warm-up blend ([FT] "동적 워밍업 양자화"): lambda = min(step / total, 1)  */
/* scales the difference between the original and the quantised values, so  */
/* a value v enters as v + lambda (Q(v) - v): lambda = 0 is the full-        */
/* precision layer, lambda = 1 the BitLinear layer.                          */
/* ------------------------------------------------------------------------- */

/* min(step / total, 1), and 0 for step <= 0; total <= 0 means no warm-up (1). */
double oracle_warmup_lambda(int64_t step, int64_t total) {
    if (total <= 0) return 1.0;
    if (step <= 0) return 0.0;
    if (step >= total) return 1.0;
    return (double)step / (double)total;
}

/*
 * The layer at blend factor lambda, in float64:
 *   n[m][k]  = u[m][k] * rstd[m]      the RMSNorm output (u = float32 x * gain as
 *                                      in O2, rstd = 1 / sqrt(mean x^2 + eps))
 *   n~[m][k] = d_x[m] * q[m][k]        its dequantised int8 codes (O2)
 *   W~[o][k] = d_w * q_w[o][k]         the dequantised ternary weights (O1)
 *   a = n + lambda (n~ - n),  b = W + lambda (W~ - W)
 *   y[m][o]  = sum_k a[m][k] b[o][k]   (k ascending)
 * x: bf16 bits [M][K]; gain [K] or NULL; W float32 [N][K]; y float64 [M][N].
 */
int oracle_linear_forward_blend(const uint16_t* x, const float* gain, float eps, int64_t M, int64_t K,
                                const float* W, int64_t N, double lambda, double* y) {
    if (M < 0 || N < 0 || K < 16 || K % 16 != 0) return -1;
    int8_t* q = (int8_t*)malloc((size_t)(M > 0 ? M : 1) * (size_t)K);
    float* d_x = (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
    int32_t* qsum = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M > 0 ? M : 1));
    double* a = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1) * (size_t)K);
    uint8_t* packed = (uint8_t*)malloc((size_t)(N > 0 ? N : 1) * (size_t)(K / 4));
    int8_t* qw = (int8_t*)malloc((size_t)(N > 0 ? N : 1) * (size_t)K);
    float w_scale[2];
    int rc = 0;
    if (!q || !d_x || !qsum || !a || !packed || !qw) rc = -1;
    if (rc == 0 && M > 0) rc = oracle_quant_act(x, gain, eps, M, K, q, d_x, qsum);
    if (rc == 0 && N > 0) rc = oracle_pack_weights(W, N, K, 0, packed, w_scale, qw);
    if (rc == 0) {
        for (int64_t m = 0; m < M; m++) {
            double sum_sq = 0.0;
            for (int64_t k = 0; k < K; k++) {
                const double xk = (double)bf16_bits_to_float(x[m * K + k]);
                sum_sq += xk * xk;
            }
            const double rstd = 1.0 / sqrt(sum_sq / (double)K + (double)eps);
            for (int64_t k = 0; k < K; k++) {
                const float xk = bf16_bits_to_float(x[m * K + k]);
                const float u = gain ? xk * gain[k] : xk;
                const double n = (double)u * rstd;
                const double nt = (double)d_x[m] * (double)q[m * K + k];
                a[m * K + k] = n + lambda * (nt - n);
            }
        }
        const double d_w = (double)w_scale[0];
#pragma omp parallel for schedule(static)
        for (int64_t o = 0; o < N; o++) {
            double* b = (double*)malloc(sizeof(double) * (size_t)K);
            for (int64_t k = 0; k < K; k++) {
                const double w = (double)W[o * K + k];
                const double wt = d_w * (double)qw[o * K + k];
                b[k] = w + lambda * (wt - w);
            }
            for (int64_t m = 0; m < M; m++) {
                double s = 0.0;
                for (int64_t k = 0; k < K; k++) s += a[m * K + k] * b[k];
                y[m * N + o] = s;
            }
            free(b);
        }
    }
    free(q);
    free(d_x);
    free(qsum);
    free(a);
    free(packed);
    free(qw);
    return rc;
}
