// quant_act.hip - fused RMSNorm + per-token absmax int8 activation quantisation.
//
// Follows the activation rule of the Hugging Face 1.58-bit fine-tuning write-up
// ("LLM을 1.58비트로 파인튜닝", section 양자화 메커니즘: per-token absmax into
// [-128, 127] after normalisation) with the factor 127/absmax of the
// quantization primer (endplan.ai, section 그러면 크기를 더 못줄이나요?).
//
// One 256-thread workgroup per token.  Each thread owns CH chunks of 16
// consecutive bf16 values (chunk c = thread + 256*j), kept in registers as raw
// bf16 between the two passes:
//   pass 1: u = x * gain, absmax |u| and sum x^2 (float64) -> workgroup reduce
//           (DPP within waves, one LDS exchange);
//   pass 2: codes rint(u * float32(127/absmax)), stored 16 bytes at a time.
// HBM-bound: 2K bytes read, K bytes written per token.
#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

constexpr int kQuantThreads = 256;

template <int CH>
__global__ __launch_bounds__(kQuantThreads) void quant_act_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ gain, float eps, int K,
    int8_t* __restrict__ xq, float* __restrict__ x_scale, int32_t* __restrict__ x_qsum) {
    __shared__ float red_f[kQuantThreads / kWave];
    __shared__ double red_d[kQuantThreads / kWave];
    __shared__ int red_i[kQuantThreads / kWave];

    const int64_t m = blockIdx.x;
    const int t = threadIdx.x;
    const int nchunk = K / 16;
    const uint4* xr = reinterpret_cast<const uint4*>(x + m * K);

    uint4 raw[CH][2];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = t + j * kQuantThreads;
        if (c < nchunk) {
            raw[j][0] = xr[2 * c];
            raw[j][1] = xr[2 * c + 1];
        } else {
            raw[j][0] = make_uint4(0, 0, 0, 0);
            raw[j][1] = make_uint4(0, 0, 0, 0);
        }
    }

    // Unpack 16 bf16 of chunk j into float32.
    auto unpack = [&](int j, float (&v)[16]) {
        const uint32_t w[8] = {raw[j][0].x, raw[j][0].y, raw[j][0].z, raw[j][0].w,
                               raw[j][1].x, raw[j][1].y, raw[j][1].z, raw[j][1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        }
    };
    auto apply_gain = [&](int c, float (&v)[16]) {
        if (gain != nullptr) {
            const float4* g4 = reinterpret_cast<const float4*>(gain + 16 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 g = g4[i];
                v[4 * i] *= g.x;
                v[4 * i + 1] *= g.y;
                v[4 * i + 2] *= g.z;
                v[4 * i + 3] *= g.w;
            }
        }
    };

    float amax = 0.f;
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = t + j * kQuantThreads;
        if (c < nchunk) {
            float v[16];
            unpack(j, v);
#pragma unroll
            for (int i = 0; i < 16; ++i) ss += (double)v[i] * (double)v[i];
            apply_gain(c, v);
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
        }
    }
    // Absmax and sum of squares reduced together: DPP within each wave, one
    // LDS exchange across the four waves.
    constexpr int NW = kQuantThreads / kWave;
    const int lane = t % kWave, wave = t / kWave;
    amax = wave_max_dpp(amax);
    ss = wave_sum_dpp(ss);
    if (lane == 0) {
        red_f[wave] = amax;
        red_d[wave] = ss;
    }
    __syncthreads();
    amax = red_f[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) amax = fmaxf(amax, red_f[w]);

    const bool zero = amax < kTinyAbsmax;
    const float scale = zero ? 0.f : 127.0f / amax;
    int qs = 0;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = t + j * kQuantThreads;
        if (c < nchunk) {
            float v[16];
            unpack(j, v);
            apply_gain(c, v);
            uint32_t word[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t wv = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int q = zero ? 0 : round_clamp(v[4 * i + b] * scale, -128.f, 127.f);
                    qs += q;
                    wv |= (uint32_t)(q & 0xff) << (8 * b);
                }
                word[i] = wv;
            }
            *reinterpret_cast<uint4*>(xq + m * K + 16 * c) = make_uint4(word[0], word[1], word[2], word[3]);
        }
    }
    qs = wave_sum_dpp(qs);
    if (lane == 0) red_i[wave] = qs;
    __syncthreads();

    if (t == 0) {
        double sum_sq = red_d[0];
        int qsum = red_i[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            sum_sq += red_d[w];
            qsum += red_i[w];
        }
        x_scale[m] = zero ? 0.f : token_scale(amax, sum_sq, inv_count(K), eps, 1.0 / 127.0);
        x_qsum[m] = qsum;
    }
}

template <int CH>
hipError_t launch_ch(const uint16_t* x, const float* gain, float eps, int64_t M, int64_t K,
                     int8_t* xq, float* x_scale, int32_t* x_qsum, hipStream_t stream) {
    return launch_kernel(quant_act_kernel<CH>, dim3((unsigned)M), dim3(kQuantThreads), 0, stream, x,
                       gain, eps, (int)K, xq, x_scale, x_qsum);
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M, int64_t K,
                            int8_t* xq, float* x_scale, int32_t* x_qsum, hipStream_t stream) {
    if (M == 0) return hipSuccess;
    const int64_t chunks = K / 16;
    const int64_t ch = (chunks + kQuantThreads - 1) / kQuantThreads;  // 1 .. 16 for K <= 65536
    if (ch <= 1) return launch_ch<1>(x, gain, eps, M, K, xq, x_scale, x_qsum, stream);
    if (ch <= 2) return launch_ch<2>(x, gain, eps, M, K, xq, x_scale, x_qsum, stream);
    if (ch <= 3) return launch_ch<3>(x, gain, eps, M, K, xq, x_scale, x_qsum, stream);
    if (ch <= 4) return launch_ch<4>(x, gain, eps, M, K, xq, x_scale, x_qsum, stream);
    if (ch <= 6) return launch_ch<6>(x, gain, eps, M, K, xq, x_scale, x_qsum, stream);
    if (ch <= 8) return launch_ch<8>(x, gain, eps, M, K, xq, x_scale, x_qsum, stream);
    if (ch <= 12) return launch_ch<12>(x, gain, eps, M, K, xq, x_scale, x_qsum, stream);
    return launch_ch<16>(x, gain, eps, M, K, xq, x_scale, x_qsum, stream);
}

}  // namespace bitnet
