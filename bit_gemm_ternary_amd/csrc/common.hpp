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
// Wavefront reductions (butterfly over the 64 lanes; every lane gets the result).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Workgroup reductions over NT threads (NT a multiple of 64, at most 1024).
// `scratch` must hold NT/64 elements; the call contains two barriers, so every
// thread of the workgroup must reach it.
template <int NT, typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, T* scratch, Op op) {
    static_assert(NT % kWave == 0 && NT <= 1024, "block size");
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = op(r, scratch[w]);
    __syncthreads();
    return r;
}

struct MaxOp {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct SumOp {
    template <typename T>
    __device__ T operator()(T a, T b) const { return a + b; }
};

// Codes of one activation: clamp(rint(v), lo, hi) as an int.  rint rounds half
// to even (v_rndne_f32).
__device__ __forceinline__ int round_clamp(float v, float lo, float hi) {
    float r = __builtin_rintf(v);
    r = fminf(fmaxf(r, lo), hi);
    return (int)r;
}

// Tokens whose absmax is below this quantise to all-zero codes.
constexpr float kTinyAbsmax = 0x1p-120f;

}  // namespace bitnet
