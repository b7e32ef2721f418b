// hadamard.hpp - the in-workgroup fast Walsh-Hadamard transform of one token
// (K = 2^P values held E per thread), shared by the H-BitLinear quantisation
// kernel and the fused one-token H-BitLinear decode.
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
#pragma once

#include "common.hpp"

namespace bitnet {
namespace hadamard {

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
    // low bits first.  The thread's bits and the register's bits are disjoint,
    // so the index is base<J>(t) + offset<J>(r), and (the padding adds the
    // index shifted down by 5, which keeps disjoint bits disjoint) the padded
    // LDS slot is pad(base) + pad(offset): one address per thread and phase,
    // with the register's part a compile-time offset.
    template <int J>
    __device__ static __forceinline__ int base(int t) {
        constexpr int b0 = J * LOG_E;
        constexpr int w = (P - b0 < LOG_E) ? (P - b0) : LOG_E;
        constexpr int xb = LOG_E - w;
        constexpr int nlow = b0 - xb;
        return ((t & ((1 << nlow) - 1)) << xb) | ((t >> nlow) << (b0 + w));
    }
    template <int J>
    __device__ static constexpr int offset(int r) {
        constexpr int b0 = J * LOG_E;
        constexpr int w = (P - b0 < LOG_E) ? (P - b0) : LOG_E;
        return ((r & ((1 << w) - 1)) << b0) | (r >> w);
    }
    template <int J>
    __device__ static __forceinline__ int index(int t, int r) {
        return base<J>(t) | offset<J>(r);
    }
    static constexpr int pad_c(int i) { return i + (i >> 5); }
    // Index bits [0, xbits) of the last phase come from the register number
    // (r >> w): the 2^xbits registers that differ only there hold adjacent
    // indices.
    template <int J>
    static constexpr int xbits() {
        constexpr int w = (P - J * LOG_E < LOG_E) ? (P - J * LOG_E) : LOG_E;
        return LOG_E - w;
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
            float* wr = lds + pad(base<J>(t));
            float* rd = lds + pad(base<J + 1>(t));
#pragma unroll
            for (int r = 0; r < E; ++r) wr[pad_c(offset<J>(r))] = v[r];
            __syncthreads();
#pragma unroll
            for (int r = 0; r < E; ++r) v[r] = rd[pad_c(offset<J + 1>(r))];
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

// Byte address in LDS of code k for store_codes: natural order.  A layout's
// addr must be additive over disjoint bits of k (a thread's base index and its
// register offsets are mapped separately and added).
struct NaturalCodes {
    static constexpr int addr(int k) { return k; }
};

// Integer codes of a thread's transform values after Fwht::run: rint(v * scale)
// for |v| * scale < 127.5, stored as bytes at L::addr(index) in lds8 (free
// LDS; K bytes in natural order).  Adding 1.5 * 2^23 to the product rounds it to an
// integer (ties to even, the rint of the definition) and leaves it, two's
// complement, in the low byte of the float's bits; with scale = rn(c / amax)
// and |v| <= amax the product's magnitude stays below c + 0.5, so no clamp is
// needed for integer c <= 127.  Registers that hold adjacent indices are stored together (a byte,
// a 16-bit or a 32-bit word per store).  Returns the sum of the thread's codes.
template <int P, int E, class L = NaturalCodes>
__device__ __forceinline__ int store_codes(const float (&v)[E], float scale, int8_t* lds8, int t) {
    using F = Fwht<P, E>;
    uint32_t b[E];
#pragma unroll
    for (int r = 0; r < E; ++r) b[r] = __float_as_uint(__fadd_rn(__fmul_rn(v[r], scale), 12582912.0f));
    auto pack4 = [](uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
        return __builtin_amdgcn_perm(__builtin_amdgcn_perm(b3, b2, 0x0c0c0400u),
                                     __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u), 0x05040100u);
    };
    constexpr int J = F::NPH - 1;
    constexpr int G = 1 << F::template xbits<J>();   // adjacent codes per register group
    constexpr int W = E / G;
    constexpr int B0 = J * F::LOG_E;
    int8_t* cdst = lds8 + L::addr(F::template base<J>(t));
    int qs = 0;
    if constexpr (G >= 4) {
#pragma unroll
        for (int rl = 0; rl < W; ++rl)
#pragma unroll
            for (int q = 0; q < G / 4; ++q) {
                const uint32_t word = pack4(b[rl + (4 * q) * W], b[rl + (4 * q + 1) * W],
                                            b[rl + (4 * q + 2) * W], b[rl + (4 * q + 3) * W]);
                qs = __builtin_amdgcn_sdot4((int)word, 0x01010101, qs, false);
                *reinterpret_cast<uint32_t*>(cdst + L::addr((rl << B0) + 4 * q)) = word;
            }
    } else {
#pragma unroll
        for (int i = 0; i < E / 4; ++i)
            qs = __builtin_amdgcn_sdot4((int)pack4(b[4 * i], b[4 * i + 1], b[4 * i + 2], b[4 * i + 3]),
                                        0x01010101, qs, false);
#pragma unroll
        for (int rl = 0; rl < W; ++rl) {
            if constexpr (G == 2)
                *reinterpret_cast<uint16_t*>(cdst + L::addr(rl << B0)) =
                    (uint16_t)__builtin_amdgcn_perm(b[rl + W], b[rl], 0x0c0c0400u);
            else
                cdst[L::addr(rl << B0)] = (int8_t)b[rl];
        }
    }
    return qs;
}

}  // namespace hadamard
}  // namespace bitnet
