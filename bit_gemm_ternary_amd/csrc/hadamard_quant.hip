// hadamard_quant.hip - H-BitLinear activations: RMSNorm + Walsh-Hadamard
// transform + per-token absmax int4 codes, and the row transform used to
// pre-rotate weights.
//
// Follows the BitNet v2 summary ("초저용량 LLM의 진화: BitNet v2 파헤치기",
// section 방법론): the activations are Hadamard-transformed before 4-bit
// quantisation, which spreads outliers and leaves a near-Gaussian distribution.
//
// Transform: unnormalised Sylvester order, t = H u, computed by float32
// butterflies (a, b) -> (a + b, a - b) with the butterfly distance ascending
// 1, 2, 4, ..., K/2.  Every butterfly is one IEEE add or subtract, so any
// schedule that keeps this stage order gives bit-identical results.
//
// Schedule for K = 2^P with B = K/E threads of E values each.  The index bits
// are processed in phases of log2(E) bits.  In each phase a thread holds the E
// values whose indices differ only in the phase's bits (plus, in a short last
// phase, some low bits it does not touch) and runs those stages in registers;
// between phases the values are exchanged through LDS.  Phase 0 reads its
// values straight from HBM (E contiguous elements per thread).
#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

template <int P, int E>
struct Fwht {
    static constexpr int K = 1 << P;
    static constexpr int LOG_E = ilog2(E);
    static constexpr int B = K / E;                         // threads
    static constexpr int NPH = (P + LOG_E - 1) / LOG_E;    // phases
    static constexpr int LDS_FLOATS = K + (K >> 5);
    static_assert(B >= kWave && B <= 1024 && B % kWave == 0, "block size");

    // One float of padding every 32 floats spreads strided phase accesses over
    // the LDS banks.
    __device__ static __forceinline__ int pad(int i) { return i + (i >> 5); }

    // Index held in register r of thread t during phase J: the low w bits of r
    // are the phase's index bits [b0, b0 + w); the remaining bits of r (short
    // last phase only) are index bits [0, xb); the thread id fills the rest,
    // low bits first.
    template <int J>
    __device__ static __forceinline__ int index(int t, int r) {
        constexpr int b0 = J * LOG_E;
        constexpr int w = (P - b0 < LOG_E) ? (P - b0) : LOG_E;
        constexpr int xb = LOG_E - w;
        constexpr int nlow = b0 - xb;
        const int r_lo = r & ((1 << w) - 1);
        const int r_hi = r >> w;
        const int base = ((t & ((1 << nlow) - 1)) << xb) | ((t >> nlow) << (b0 + w));
        return base | (r_lo << b0) | r_hi;
    }

    template <int J>
    __device__ static __forceinline__ void stages(float (&v)[E]) {
        constexpr int b0 = J * LOG_E;
        constexpr int w = (P - b0 < LOG_E) ? (P - b0) : LOG_E;
#pragma unroll
        for (int h = 1; h < (1 << w); h <<= 1) {
#pragma unroll
            for (int r = 0; r < E; ++r) {
                if ((r & h) == 0) {
                    const float a = v[r];
                    const float b = v[r + h];
                    v[r] = a + b;
                    v[r + h] = a - b;
                }
            }
        }
    }

    // Run phases J .. NPH-1; on return v holds the transform at index<NPH-1>.
    template <int J>
    __device__ static __forceinline__ void run(float (&v)[E], float* lds, int t) {
        stages<J>(v);
        if constexpr (J + 1 < NPH) {
#pragma unroll
            for (int r = 0; r < E; ++r) lds[pad(index<J>(t, r))] = v[r];
            __syncthreads();
#pragma unroll
            for (int r = 0; r < E; ++r) v[r] = lds[pad(index<J + 1>(t, r))];
            __syncthreads();
            run<J + 1>(v, lds, t);
        }
    }
};

// Load E consecutive bf16 values starting at p (16-byte aligned when E >= 8).
template <int E>
__device__ __forceinline__ void load_bf16(const uint16_t* p, float (&v)[E]) {
    if constexpr (E >= 8) {
        const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
        for (int q = 0; q < E / 8; ++q) {
            const uint4 w = p4[q];
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[8 * q + 2 * i] = bf16_lo(ws[i]);
                v[8 * q + 2 * i + 1] = bf16_hi(ws[i]);
            }
        }
    } else {
        static_assert(E == 4, "E");
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        v[0] = bf16_lo(w.x);
        v[1] = bf16_hi(w.x);
        v[2] = bf16_lo(w.y);
        v[3] = bf16_hi(w.y);
    }
}

// int4 code v in [-8, 7] as a 6-bit E3M2 float (sign, 3 exponent bits with
// bias 3, 2 mantissa bits), exact for every such integer.
__device__ __forceinline__ uint32_t e3m2_of_int(int v) {
    const uint32_t a = (uint32_t)(v < 0 ? -v : v);
    if (a == 0) return 0;
    const int l = 31 - __clz(a);                       // floor(log2 a): 0 .. 3
    const uint32_t m = ((a << 2) >> l) & 3u;
    return (v < 0 ? 0x20u : 0u) | ((uint32_t)(l + 3) << 2) | m;
}

// F6 = false: int8 codes, xq [M][K].  F6 = true: 6-bit E3M2 codes, xq
// [M][K/4*3] bytes, 32 values per 24-byte group; value p of a group is the
// code at K offset 16 (p % 2) + 4 (p / 8) + (p % 8) / 2 (the order in which the
// FP4 x FP6 contraction unpacks the weights).
template <int P, int E, bool F6>
__global__ __launch_bounds__((Fwht<P, E>::B)) void hadamard_quant_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ gain, float eps, double sqrt_k,
    int8_t* __restrict__ xq, float* __restrict__ x_scale, int32_t* __restrict__ x_qsum) {
    using F = Fwht<P, E>;
    constexpr int K = F::K;
    __shared__ __align__(16) float lds[F::LDS_FLOATS];
    __shared__ float red_f[F::B / kWave];
    __shared__ double red_d[F::B / kWave];
    __shared__ int red_i[F::B / kWave];

    const int64_t m = blockIdx.x;
    const int t = threadIdx.x;

    float v[E];
    load_bf16<E>(x + m * K + (int64_t)t * E, v);
    double ss = 0.0;
#pragma unroll
    for (int r = 0; r < E; ++r) ss += (double)v[r] * (double)v[r];
    if (gain != nullptr) {
        const float4* g4 = reinterpret_cast<const float4*>(gain + t * E);
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
            const float4 g = g4[q];
            v[4 * q] *= g.x;
            v[4 * q + 1] *= g.y;
            v[4 * q + 2] *= g.z;
            v[4 * q + 3] *= g.w;
        }
    }

    F::template run<0>(v, lds, t);

    // Absmax of the transform and the sum of squares, reduced together: DPP
    // within each wave, one LDS exchange across waves.  The transform's last
    // LDS read is behind a barrier, so `lds` is free from here on.
    constexpr int NW = F::B / kWave;
    const int lane = t % kWave, wave = t / kWave;
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < E; ++r) amax = fmaxf(amax, fabsf(v[r]));
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

    // Codes go through LDS (as bytes) back to natural order for wide stores;
    // each wave's code sum rides along and is added up after the same barrier.
    const bool zero = amax < kTinyAbsmax;
    const float scale = zero ? 0.f : 7.0f / amax;
    int8_t* lds8 = reinterpret_cast<int8_t*>(lds);
    int qs = 0;
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int q = zero ? 0 : round_clamp(v[r] * scale, -8.f, 7.f);
        qs += q;
        lds8[F::template index<F::NPH - 1>(t, r)] = (int8_t)q;
    }
    qs = wave_sum_dpp(qs);
    if (lane == 0) red_i[wave] = qs;
    __syncthreads();
    if constexpr (F6) {
        uint2* row = reinterpret_cast<uint2*>(xq + m * (K / 4 * 3));
        for (int g = t; g < K / 32; g += F::B) {
            const uint4 c0 = reinterpret_cast<const uint4*>(lds8 + 32 * g)[0];
            const uint4 c1 = reinterpret_cast<const uint4*>(lds8 + 32 * g)[1];
            const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            uint32_t out[6] = {0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int p = 0; p < 32; ++p) {
                const int k = 16 * (p % 2) + 4 * (p / 8) + (p % 8) / 2;
                const int v = (int)(int8_t)(cw[k / 4] >> (8 * (k % 4)));
                const uint64_t f = (uint64_t)e3m2_of_int(v) << ((6 * p) % 32);
                out[(6 * p) / 32] |= (uint32_t)f;
                if ((6 * p) % 32 > 26) out[(6 * p) / 32 + 1] |= (uint32_t)(f >> 32);
            }
            row[3 * g] = make_uint2(out[0], out[1]);
            row[3 * g + 1] = make_uint2(out[2], out[3]);
            row[3 * g + 2] = make_uint2(out[4], out[5]);
        }
    } else {
    int8_t* dst = xq + m * K + (int64_t)t * E;
    if constexpr (E >= 16) {
#pragma unroll
        for (int q = 0; q < E / 16; ++q)
            reinterpret_cast<uint4*>(dst)[q] = reinterpret_cast<const uint4*>(lds8 + t * E)[q];
    } else if constexpr (E == 8) {
        *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(lds8 + t * E);
    } else {
        *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(lds8 + t * E);
    }
    }

    if (t == 0) {
        double sum_sq = red_d[0];
        int qsum = red_i[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            sum_sq += red_d[w];
            qsum += red_i[w];
        }
        x_scale[m] = zero ? 0.f : token_scale(amax, sum_sq, 1.0 / (double)K, eps, 1.0 / (7.0 * sqrt_k));
        x_qsum[m] = qsum;
    }
}

template <int P, int E>
__global__ __launch_bounds__((Fwht<P, E>::B)) void fwht_rows_kernel(const float* __restrict__ src,
                                                                   float* __restrict__ dst) {
    using F = Fwht<P, E>;
    constexpr int K = F::K;
    __shared__ __align__(16) float lds[F::LDS_FLOATS];
    const int64_t n = blockIdx.x;
    const int t = threadIdx.x;
    float v[E];
    const float4* s4 = reinterpret_cast<const float4*>(src + n * K + (int64_t)t * E);
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
        const float4 a = s4[q];
        v[4 * q] = a.x;
        v[4 * q + 1] = a.y;
        v[4 * q + 2] = a.z;
        v[4 * q + 3] = a.w;
    }
    F::template run<0>(v, lds, t);
    // Back to natural order through LDS, then contiguous float4 stores.
#pragma unroll
    for (int r = 0; r < E; ++r) lds[F::pad(F::template index<F::NPH - 1>(t, r))] = v[r];
    __syncthreads();
    float4* d4 = reinterpret_cast<float4*>(dst + n * K + (int64_t)t * E);
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
        const int i = t * E + 4 * q;
        d4[q] = make_float4(lds[F::pad(i)], lds[F::pad(i + 1)], lds[F::pad(i + 2)], lds[F::pad(i + 3)]);
    }
}

// Elements per thread for K = 2^P: at least 64 threads, at most 1024, and 32
// values per thread from K = 8192 up (three LDS exchanges instead of four).
template <int P>
constexpr int elems_per_thread() {
    return P >= 13 ? 32 : (P >= 10 ? 16 : (1 << P) / 64);
}

int log2_exact(int64_t k) {
    int p = 0;
    while ((int64_t{1} << p) < k) ++p;
    return p;
}

template <int P, bool F6>
hipError_t launch_hq(const uint16_t* x, const float* gain, float eps, int64_t M, double sqrt_k,
                     int8_t* xq, float* x_scale, int32_t* x_qsum, hipStream_t stream) {
    constexpr int E = elems_per_thread<P>();
    return launch_kernel((hadamard_quant_kernel<P, E, F6>), dim3((unsigned)M),
                         dim3(Fwht<P, E>::B), 0, stream, x, gain, eps, sqrt_k, xq, x_scale, x_qsum);
}

template <bool F6>
hipError_t launch_hq_k(const uint16_t* x, const float* gain, float eps, int64_t M, int64_t K,
                       double sqrt_k, int8_t* xq, float* x_scale, int32_t* x_qsum,
                       hipStream_t stream) {
    if (M == 0) return hipSuccess;
    switch (log2_exact(K)) {
        case 8: return launch_hq<8, F6>(x, gain, eps, M, sqrt_k, xq, x_scale, x_qsum, stream);
        case 9: return launch_hq<9, F6>(x, gain, eps, M, sqrt_k, xq, x_scale, x_qsum, stream);
        case 10: return launch_hq<10, F6>(x, gain, eps, M, sqrt_k, xq, x_scale, x_qsum, stream);
        case 11: return launch_hq<11, F6>(x, gain, eps, M, sqrt_k, xq, x_scale, x_qsum, stream);
        case 12: return launch_hq<12, F6>(x, gain, eps, M, sqrt_k, xq, x_scale, x_qsum, stream);
        case 13: return launch_hq<13, F6>(x, gain, eps, M, sqrt_k, xq, x_scale, x_qsum, stream);
        case 14: return launch_hq<14, F6>(x, gain, eps, M, sqrt_k, xq, x_scale, x_qsum, stream);
        case 15: return launch_hq<15, F6>(x, gain, eps, M, sqrt_k, xq, x_scale, x_qsum, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int P>
hipError_t launch_rows(const float* src, float* dst, int64_t N, hipStream_t stream) {
    constexpr int E = elems_per_thread<P>();
    return launch_kernel((fwht_rows_kernel<P, E>), dim3((unsigned)N), dim3(Fwht<P, E>::B), 0, stream,
                       src, dst);
}


}  // namespace

hipError_t launch_hadamard_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M,
                                     int64_t K, double sqrt_k, int8_t* xq, float* x_scale,
                                     int32_t* x_qsum, hipStream_t stream) {
    return launch_hq_k<false>(x, gain, eps, M, K, sqrt_k, xq, x_scale, x_qsum, stream);
}

hipError_t launch_hadamard_quant_act_f6(const uint16_t* x, const float* gain, float eps,
                                        int64_t M, int64_t K, double sqrt_k, uint8_t* xq6,
                                        float* x_scale, int32_t* x_qsum, hipStream_t stream) {
    return launch_hq_k<true>(x, gain, eps, M, K, sqrt_k, reinterpret_cast<int8_t*>(xq6), x_scale,
                             x_qsum, stream);
}

hipError_t launch_fwht_rows_f32(const float* src, float* dst, int64_t N, int64_t K,
                                hipStream_t stream) {
    if (N == 0) return hipSuccess;
    switch (log2_exact(K)) {
        case 8: return launch_rows<8>(src, dst, N, stream);
        case 9: return launch_rows<9>(src, dst, N, stream);
        case 10: return launch_rows<10>(src, dst, N, stream);
        case 11: return launch_rows<11>(src, dst, N, stream);
        case 12: return launch_rows<12>(src, dst, N, stream);
        case 13: return launch_rows<13>(src, dst, N, stream);
        case 14: return launch_rows<14>(src, dst, N, stream);
        case 15: return launch_rows<15>(src, dst, N, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bitnet
