// blend.hip - the layer during the warm-up of quantisation (Hugging Face
// 1.58-bit write-up, section 동적 워밍업 양자화): with lambda = min(step /
// total, 1), each operand moves from its full-precision value toward its
// quantised value by lambda, v + lambda (Q(v) - v), so lambda = 0 is the dense
// layer and lambda = 1 the BitLinear layer.
//
//   a[m][k] = n + lambda (n~ - n),   n = x * gain * rstd (RMSNorm output),
//                                    n~ = d_x * q_x (its dequantised int8 codes)
//   b[o][k] = w + lambda (w~ - w),   w~ = d_w * q_w (the dequantised ternary weight)
//   y[m][o] = sum_k a[m][k] b[o][k]
//
// With lambda < 1 neither operand is ternary or integer, so the contraction is
// a dense float32 one: v_mfma_f32_32x32x2_f32 on 128 x 128 tiles, 32 K values
// per LDS stage.  The activations are blended once per token into a float32
// workspace (blend_act_kernel, after the int8 quantisation of quant_act.hip);
// the weights are blended in the stage loads from the float32 master weights
// and their packed 2-bit codes, so no blended weight matrix is stored.
//
// Float32 throughout: every blended operand is a few roundings from its
// float64 value, and the sums are float32 MFMA accumulations.
#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

constexpr int kTile = 128;              // tokens x weight rows per workgroup
constexpr int kStageK = 32;             // K values per LDS stage
constexpr int kRowFloats = kStageK + 4; // LDS row pitch (padding: conflict-free 16-byte reads)
constexpr uint32_t kBufferWord3 = 0x00020000u;
constexpr uint32_t kOutOfRange = 0x80000000u;

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 load_f4(__amdgpu_buffer_rsrc_t res, uint32_t off) {
    const v4i q = __builtin_amdgcn_raw_buffer_load_b128(res, off, 0, 0);
    return f4{__int_as_float(q[0]), __int_as_float(q[1]), __int_as_float(q[2]), __int_as_float(q[3])};
}

// One workgroup per token: a[k] = (1 - lambda) n[k] + lambda n~[k], with
// n = float32(u * rstd), u = x * gain (float32, as in the quantisation),
// rstd = 1 / sqrt(sum x^2 / K + eps) in float64, and n~ = d_x * q.
__global__ __launch_bounds__(256) void blend_act_kernel(const uint16_t* __restrict__ x, const float* __restrict__ gain,
                                                        float eps, int K, const int8_t* __restrict__ xq,
                                                        const float* __restrict__ x_scale, float lambda,
                                                        float* __restrict__ a_out) {
    __shared__ double red[4];
    const int64_t m = blockIdx.x;
    const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
    const uint16_t* xr = x + m * K;
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    for (int k = 4 * t; k < K; k += 4 * 256) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double v = (double)__uint_as_float((uint32_t)xr[k + e] << 16);
            s[e] = __fma_rn(v, v, s[e]);
        }
    }
    const double ws = wave_sum_dpp((s[0] + s[1]) + (s[2] + s[3]));
    if (lane == 0) red[wave] = ws;
    __syncthreads();
    const double ss = (red[0] + red[1]) + (red[2] + red[3]);
    const float rstd = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
    const float dx = x_scale[m];
    const float keep = 1.0f - lambda;
    for (int k = 4 * t; k < K; k += 4 * 256) {
        f4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float xv = __uint_as_float((uint32_t)xr[k + e] << 16);
            const float u = gain ? xv * gain[k + e] : xv;
            const float n = u * rstd;
            const float nq = dx * (float)xq[m * K + k + e];
            out[e] = keep * n + lambda * nq;
        }
        *reinterpret_cast<f4*>(&a_out[m * K + k]) = out;
    }
}

// y = a b^T over 128 x 128 tiles (tokens x weight rows), 4 waves of 64 x 64
// (2 x 2 blocks of 32 x 32).  MFMA 32x32x2 f32: lane l holds A[i = l % 32][k]
// and B[k][j = l % 32] for k = l / 32 of the step; over the 16 steps of a stage
// lane half h covers the stage's K values 16h .. 16h + 15, so one 64-byte read
// per block and stage gives a lane all its operands.  The result D[i][j] sits
// in lane j + 32 ((i / 4) % 2), element 4 (i / 8) + i % 4.
__global__ __launch_bounds__(256) void blend_gemm_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                                         const uint8_t* __restrict__ packed,
                                                         const float* __restrict__ w_scale, float lambda, int M,
                                                         int N, int K, float* __restrict__ y) {
    __shared__ __align__(16) float As[2][kTile * kRowFloats];
    __shared__ __align__(16) float Bs[2][kTile * kRowFloats];
    const int t = threadIdx.x, lane = t % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int wm = wave / 2, wn = wave % 2;
    const int tiles_n = (N + kTile - 1) / kTile;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * kTile;
    const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * kTile;
    const int mrows = (int)min((int64_t)kTile, (int64_t)M - m0);
    const int nrows = (int)min((int64_t)kTile, (int64_t)N - n0);
    // Resources cover the tile's valid rows: rows past M or N load zeros.
    const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + m0 * K), (short)0, mrows * K * 4, (int)kBufferWord3);
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + n0 * K), (short)0, nrows * K * 4, (int)kBufferWord3);
    const __amdgpu_buffer_rsrc_t pres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(packed + n0 * (K / 4)), (short)0, nrows * (K / 4), (int)kBufferWord3);
    const float keep = 1.0f - lambda;
    const float qscale = lambda * w_scale[0];

    // Stage loads: thread t owns row t / 2 and 16 K values at 16 (t % 2).
    const int lr = t / 2, lh = t % 2;
    f4 a_reg[4], w_reg[4];
    uint32_t p_reg;
    auto load_stage = [&](int st) {
        const int k0 = st * kStageK + 16 * lh;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            a_reg[q] = load_f4(ares, (uint32_t)((lr * K + k0 + 4 * q) * 4));
            w_reg[q] = load_f4(wres, (uint32_t)((lr * K + k0 + 4 * q) * 4));
        }
        p_reg = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(pres, (uint32_t)(lr * (K / 4) + k0 / 4), 0, 0);
    };
    // Blend the weights and store both operands.  Word k0/16 of the row holds
    // weights k0 .. k0+15; the fields of k0 + 4i + b are byte b's bits 2i.
    auto store_stage = [&](int buf) {
        float* as = &As[buf][lr * kRowFloats + 16 * lh];
        float* bs = &Bs[buf][lr * kRowFloats + 16 * lh];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *reinterpret_cast<f4*>(as + 4 * q) = a_reg[q];
            const uint32_t fields = (p_reg >> (2 * q)) & 0x03030303u;
            f4 b;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float qw = (float)((int)((fields >> (8 * e)) & 3u) - 1);
                b[e] = keep * w_reg[q][e] + qscale * qw;
            }
            *reinterpret_cast<f4*>(bs + 4 * q) = b;
        }
    };

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int nst = K / kStageK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    const int r32 = lane % 32, h = lane / 32;
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) load_stage(st + 1);
        f4 av[2][4], bv[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                av[i][q] = *reinterpret_cast<const f4*>(
                    &As[buf][(64 * wm + 32 * i + r32) * kRowFloats + 16 * h + 4 * q]);
                bv[i][q] = *reinterpret_cast<const f4*>(
                    &Bs[buf][(64 * wn + 32 * i + r32) * kRowFloats + 16 * h + 4 * q]);
            }
#pragma unroll
        for (int s = 0; s < 16; ++s)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][s / 4][s % 4], bv[j][s / 4][s % 4],
                                                                    acc[i][j], 0, 0, 0);
        if (st + 1 < nst) {
            store_stage(buf ^ 1);
            __syncthreads();
        }
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + 64 * wm + 32 * i + 8 * (e / 4) + 4 * h + (e % 4);
                const int64_t o = n0 + 64 * wn + 32 * j + r32;
                if (m < M && o < N) y[m * N + o] = acc[i][j][e];
            }
}

}  // namespace

size_t blend_workspace_bytes(int64_t M, int64_t K) {
    const size_t a = ((size_t)M * (size_t)K * 4 + 255) / 256 * 256;
    const size_t q = ((size_t)M * (size_t)K + 255) / 256 * 256;
    const size_t s = ((size_t)M * 8 + 255) / 256 * 256;
    return a + q + s;
}

hipError_t launch_linear_forward_blend(const uint16_t* x, const float* gain, float eps, const float* W,
                                       const uint8_t* packed, const float* w_scale, float lambda, int64_t M,
                                       int64_t N, int64_t K, float* y, void* workspace, hipStream_t stream) {
    char* ws = reinterpret_cast<char*>(workspace);
    float* a = reinterpret_cast<float*>(ws);
    int8_t* xq = reinterpret_cast<int8_t*>(ws + ((size_t)M * (size_t)K * 4 + 255) / 256 * 256);
    float* x_scale = reinterpret_cast<float*>(reinterpret_cast<char*>(xq) + ((size_t)M * (size_t)K + 255) / 256 * 256);
    int32_t* x_qsum = reinterpret_cast<int32_t*>(x_scale + M);
    hipError_t e = launch_quant_act(x, gain, eps, M, K, xq, x_scale, x_qsum, stream);
    if (e != hipSuccess) return e;
    e = launch_kernel(blend_act_kernel, dim3((unsigned)M), dim3(256), 0, stream, x, gain, eps, (int)K, xq, x_scale,
                      lambda, a);
    if (e != hipSuccess) return e;
    const int64_t tiles = ((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile);
    return launch_kernel(blend_gemm_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, a, W, packed, w_scale,
                         lambda, (int)M, (int)N, (int)K, y);
}

}  // namespace bitnet
