// quant_act.hip - fused RMSNorm + per-token absmax int8 activation quantisation.
//
// Follows the activation rule of the Hugging Face 1.58-bit fine-tuning write-up
// ("LLM을 1.58비트로 파인튜닝", section 양자화 메커니즘: per-token absmax into
// [-128, 127] after normalisation) with the factor 127/absmax of the
// quantization primer (endplan.ai, section 그러면 크기를 더 못줄이나요?).
//
// One workgroup per token (256 threads, 1024 from K = 16384 up, so that a
// thread holds at most 8 vectors).  Thread t owns the 16-byte vectors
// (8 consecutive bf16 values) t, t + NT, t + 2 NT, ..., so every load and
// store instruction of a wave covers one contiguous stretch of the token; the
// raw bf16 stay in registers between the two passes:
//   pass 1: u = x * gain, absmax |u|, and sum x^2 (each square of a bf16 value
//           exact in float32, four float32 chains combined in float64)
//           -> workgroup reduce (DPP within waves, one LDS exchange);
//   pass 2: codes rint(u * float32(127/absmax)), 8 bytes per vector.
// |u| <= absmax, so |u * rn(127/absmax)| < 127.5 and the clamp to [-128, 127]
// never acts: adding 1.5 * 2^23 rounds the product to an integer (ties to
// even, the rint of the definition) and leaves it, two's complement, in the
// low byte of the float's bits.
// HBM-bound: 2K bytes read, K bytes written per token.
//
// Row-parallel shards (each GPU holds a K slice of every token and of the
// weights) split the two passes: MODE kSliceStats runs pass 1 on the slice and
// writes its absmax and sum of squares; after the cross-shard reduction (a
// maximum and a sum) MODE kGivenStats runs pass 2 on the slice with the whole
// token's values, so every shard writes exactly the codes a single GPU writes
// for those positions, and the d_x of the whole token.
#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

constexpr int kLocal = 0, kSliceStats = 1, kGivenStats = 2;

struct QuantArgs {
    const uint16_t* x;          // bf16 [M][K]
    const float* gain;          // [K] or NULL
    float eps;
    int K;                      // values per token (the slice's, for a shard)
    int8_t* xq;                 // [M][K]
    float* x_scale;             // [M]
    int32_t* x_qsum;            // [M]
    float* amax_out;            // kSliceStats: [M]
    double* ss_out;             // kSliceStats: [M]
    const float* amax_in;       // kGivenStats: [M], the whole token's absmax
    const double* ss_in;        // kGivenStats: [M], the whole token's sum of x^2
    int k_total;                // kGivenStats: the whole token's K (the mean's divisor)
};

template <int XV, int NT, int MODE>
__global__ __launch_bounds__(NT) void quant_act_kernel(const QuantArgs a) {
    __shared__ float red_f[NT / kWave];
    __shared__ double red_d[NT / kWave];
    __shared__ int red_i[NT / kWave];
    const uint16_t* __restrict__ x = a.x;
    const float* __restrict__ gain = a.gain;
    const int K = a.K;

    const int64_t m = blockIdx.x;
    const int t = threadIdx.x;
    const int nvec = K / 8;
    const uint4* xr = reinterpret_cast<const uint4*>(x + m * K);

    uint4 raw[XV];
#pragma unroll
    for (int j = 0; j < XV; ++j) {
        const int v = t + j * NT;
        raw[j] = v < nvec ? xr[v] : make_uint4(0, 0, 0, 0);
    }

    // The 8 values of vector j, times the gain when there is one.
    auto values = [&](int j, float (&u)[8], bool with_gain, bool reload) {
        const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u[2 * i] = bf16_lo(w[i]);
            u[2 * i + 1] = bf16_hi(w[i]);
        }
        const int v = t + j * NT;
        if (with_gain && gain != nullptr && v < nvec) {
            // Read again in the second pass (volatile: not kept in registers
            // across the reduction, which would double the registers per vector).
            typedef float f4v __attribute__((ext_vector_type(4)));
            const f4v* g4 = reinterpret_cast<const f4v*>(gain + 8 * v);
            const f4v g0 = reload ? *reinterpret_cast<const volatile f4v*>(g4) : g4[0];
            const f4v g1 = reload ? *reinterpret_cast<const volatile f4v*>(g4 + 1) : g4[1];
            u[0] *= g0[0]; u[1] *= g0[1]; u[2] *= g0[2]; u[3] *= g0[3];
            u[4] *= g1[0]; u[5] *= g1[1]; u[6] *= g1[2]; u[7] *= g1[3];
        }
    };

    constexpr int NW = NT / kWave;
    const int lane = t % kWave, wave = t / kWave;
    float amax = 0.f;
    if constexpr (MODE == kGivenStats) {
        amax = a.amax_in[m];
    } else {
        // Vectors past K were loaded as zeros and change neither sum.
        float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < XV; ++j) {
            float u[8];
            values(j, u, false, false);
#pragma unroll
            for (int i = 0; i < 8; ++i) sq[i % 4] = __fmaf_rn(u[i], u[i], sq[i % 4]);
            values(j, u, true, false);
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(u[i]));
        }
        double ss = ((double)sq[0] + (double)sq[1]) + ((double)sq[2] + (double)sq[3]);
        // Absmax and sum of squares reduced together: DPP within each wave, one
        // LDS exchange across the four waves.
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
        if constexpr (MODE == kSliceStats) {
            if (t == 0) {
                double sum_sq = red_d[0];
#pragma unroll
                for (int w = 1; w < NW; ++w) sum_sq += red_d[w];
                a.amax_out[m] = amax;
                a.ss_out[m] = sum_sq;
            }
            return;
        }
    }

    const bool zero = amax < kTinyAbsmax;
    const float scale = zero ? 0.f : 127.0f / amax;
    int qs = 0;
#pragma unroll
    for (int j = 0; j < XV; ++j) {
        const int v = t + j * NT;
        float u[8];
        values(j, u, true, true);
        uint32_t b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float p = __fmul_rn(u[i], scale);
            // Given statistics come from the caller: clamp so that an absmax
            // below this slice's own still yields codes in [-128, 127].
            if constexpr (MODE == kGivenStats) p = fminf(fmaxf(p, -128.0f), 127.0f);
            b[i] = __float_as_uint(__fadd_rn(p, 12582912.0f));
        }
        const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                                                  __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u), 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u),
                                                  __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u), 0x05040100u);
        if (v < nvec) {
            qs = __builtin_amdgcn_sdot4((int)lo, 0x01010101, qs, false);
            qs = __builtin_amdgcn_sdot4((int)hi, 0x01010101, qs, false);
            *reinterpret_cast<uint2*>(a.xq + m * K + 8 * v) = make_uint2(lo, hi);
        }
    }
    qs = wave_sum_dpp(qs);
    if (lane == 0) red_i[wave] = qs;
    __syncthreads();

    if (t == 0) {
        int qsum = red_i[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) qsum += red_i[w];
        double sum_sq;
        if constexpr (MODE == kGivenStats) {
            sum_sq = a.ss_in[m];
        } else {
            sum_sq = red_d[0];
#pragma unroll
            for (int w = 1; w < NW; ++w) sum_sq += red_d[w];
        }
        const int k_mean = MODE == kGivenStats ? a.k_total : K;
        a.x_scale[m] = zero ? 0.f : token_scale(amax, sum_sq, inv_count(k_mean), a.eps, 1.0 / 127.0);
        a.x_qsum[m] = qsum;
    }
}

template <int XV, int NT, int MODE>
hipError_t launch_xv(const QuantArgs& a, int64_t M, hipStream_t stream) {
    return launch_kernel((quant_act_kernel<XV, NT, MODE>), dim3((unsigned)M), dim3(NT), 0, stream, a);
}

template <int NT, int MODE>
hipError_t launch_nt(const QuantArgs& a, int64_t M, hipStream_t stream) {
    const int64_t xv = (a.K / 8 + NT - 1) / NT;
    if (xv <= 1) return launch_xv<1, NT, MODE>(a, M, stream);
    if (xv <= 2) return launch_xv<2, NT, MODE>(a, M, stream);
    if (xv <= 3) return launch_xv<3, NT, MODE>(a, M, stream);
    if (xv <= 4) return launch_xv<4, NT, MODE>(a, M, stream);
    if (xv <= 6) return launch_xv<6, NT, MODE>(a, M, stream);
    return launch_xv<8, NT, MODE>(a, M, stream);
}

// K <= 16384: 256 threads, at most 8 vectors each; K <= 65536: 1024 threads.
template <int MODE>
hipError_t launch_mode(const QuantArgs& a, int64_t M, hipStream_t stream) {
    if (M == 0) return hipSuccess;
    if (a.K <= 16384) return launch_nt<256, MODE>(a, M, stream);
    return launch_nt<1024, MODE>(a, M, stream);
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M, int64_t K,
                            int8_t* xq, float* x_scale, int32_t* x_qsum, hipStream_t stream) {
    QuantArgs a{};
    a.x = x, a.gain = gain, a.eps = eps, a.K = (int)K, a.xq = xq, a.x_scale = x_scale, a.x_qsum = x_qsum;
    return launch_mode<kLocal>(a, M, stream);
}

hipError_t launch_token_stats(const uint16_t* x, const float* gain, int64_t M, int64_t K, float* amax,
                              double* sumsq, hipStream_t stream) {
    QuantArgs a{};
    a.x = x, a.gain = gain, a.K = (int)K, a.amax_out = amax, a.ss_out = sumsq;
    return launch_mode<kSliceStats>(a, M, stream);
}

hipError_t launch_quant_act_with_stats(const uint16_t* x, const float* gain, float eps, int64_t M,
                                       int64_t K, int64_t k_total, const float* amax,
                                       const double* sumsq, int8_t* xq, float* x_scale,
                                       int32_t* x_qsum, hipStream_t stream) {
    QuantArgs a{};
    a.x = x, a.gain = gain, a.eps = eps, a.K = (int)K, a.xq = xq, a.x_scale = x_scale, a.x_qsum = x_qsum;
    a.amax_in = amax, a.ss_in = sumsq, a.k_total = (int)k_total;
    return launch_mode<kGivenStats>(a, M, stream);
}

}  // namespace bitnet
