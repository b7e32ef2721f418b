// common.hpp - device helpers shared by the gfx950 kernels of the BitLinear path.
//
// gfx950 runs 64-wide wavefronts only; every helper below assumes that.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnet {

constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));

// bf16 bit patterns packed two per 32-bit word -> float32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// DPP wavefront reductions: four lane moves within each 16-lane row, then the
// four row results read out to scalars.  No LDS traffic; the combination order
// is fixed, so floating-point results are deterministic.
// ---------------------------------------------------------------------------
// Sum of v over the 64 lanes, returned wave-uniform.
__device__ __forceinline__ int wave_sum_dpp(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Lane-to-lane moves within 16-lane rows (DPP), for 32- and 64-bit values.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_move(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ float read_lane(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double read_lane(double v, int l) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Wave-uniform max / sum over the 64 lanes, reduced within each 16-lane row by
// DPP and then over the four rows; the combination order is fixed, so the
// double sum is deterministic.
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, dpp_move<0xB1>(v));
    v = fmaxf(v, dpp_move<0x4E>(v));
    v = fmaxf(v, dpp_move<0x141>(v));
    v = fmaxf(v, dpp_move<0x140>(v));
    return fmaxf(fmaxf(read_lane(v, 0), read_lane(v, 16)), fmaxf(read_lane(v, 32), read_lane(v, 48)));
}
__device__ __forceinline__ double wave_sum_dpp(double v) {
    v += dpp_move<0xB1>(v);
    v += dpp_move<0x4E>(v);
    v += dpp_move<0x141>(v);
    v += dpp_move<0x140>(v);
    return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

// Codes of one activation: clamp(rint(v), lo, hi) as an int.  rint rounds half
// to even (v_rndne_f32).
__device__ __forceinline__ int round_clamp(float v, float lo, float hi) {
    float r = __builtin_rintf(v);
    r = fminf(fmaxf(r, lo), hi);
    return (int)r;
}

// Tokens whose absmax is below this quantise to all-zero codes.
constexpr float kTinyAbsmax = 0x1p-120f;

// Per-token dequantisation factor d_x = amax * rstd * inv_denom, with
// rstd = 1 / sqrt(ss * inv_k + eps) and ss the float64 sum of x^2 over the
// token (inv_k = 1 / K; inv_denom = 1 / 127 for int8 codes, 1 / (7 sqrt K) for
// the Hadamard int4 codes).  The reciprocal square root is the hardware
// float64 estimate refined by one Newton step, and the result is rounded once
// to float32: a few float32 ulps from the correctly rounded float64 chain
// (two divisions and a square root) at a fraction of its latency.  No code
// depends on d_x; it only scales outputs.  Zero for an all-zero token.
// 1 / K for token_scale: the hardware float32 reciprocal (within an ulp or so),
// one instruction instead of a float64 division; every kernel that forms d_x
// for the int8 codes uses this same value.
__device__ __forceinline__ double inv_count(int K) {
    return (double)__builtin_amdgcn_rcpf((float)K);
}

__device__ __forceinline__ float token_scale(float amax, double ss, double inv_k, float eps,
                                             double inv_denom) {
    if (amax < kTinyAbsmax) return 0.f;
    const double v = ss * inv_k + (double)eps;
    double r = __builtin_amdgcn_rsq(v);
    r = r * (1.5 - (0.5 * v) * r * r);
    return (float)(((double)amax * r) * inv_denom);
}

}  // namespace bitnet
