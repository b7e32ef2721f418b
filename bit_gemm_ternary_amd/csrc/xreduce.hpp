// xreduce.hpp - transposing wave reductions for kernels that end a batch of
// rows with one partial sum per row (and token) in every lane.
//
// NV partial sums per lane (NV a power of 2, <= 64) are summed over the 64
// lanes by a butterfly over the lane-index bits (v_permlane32_swap,
// v_permlane16_swap, then DPP moves inside 16-lane rows).  Each transposing
// step halves the number of values per lane while adding pairs, so the NV
// totals cost about 2 NV + 12 lane operations rather than NV separate wave
// reductions; lane L then holds the total of value L >> (6 - log2 NV).
#pragma once

#include "common.hpp"

namespace bitnet {

// tstep<M>(a, b): lanes with lane bit M clear keep a, lanes with it set keep
// b, and each adds the copy of the kept value held by a partner lane whose bit
// M differs (and whose higher bits agree).
template <int M>
__device__ __forceinline__ int tstep(int a, int b, int lane) {
    if constexpr (M == 32) {  // lanes 0-31 get (a, a of lane + 32), lanes 32-63 (b of lane - 32, b)
        const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
        return (int)r[0] + (int)r[1];
    } else if constexpr (M == 16) {  // the same between 16-lane rows 0|1 and 2|3
        const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
        return (int)r[0] + (int)r[1];
    } else if constexpr (M == 8) {  // row_ror:8 pairs lane ^ 8; banks 2, 3 are the lanes with bit 3
        const int x = __builtin_amdgcn_update_dpp(a, b, 0x128, 0xF, 0xC, false);
        const int y = __builtin_amdgcn_update_dpp(b, a, 0x128, 0xF, 0x3, false);
        return x + y;
    } else if constexpr (M == 4) {  // row_half_mirror pairs lane ^ 7; banks 1, 3 have bit 2
        const int x = __builtin_amdgcn_update_dpp(a, b, 0x141, 0xF, 0xA, false);
        const int y = __builtin_amdgcn_update_dpp(b, a, 0x141, 0xF, 0x5, false);
        return x + y;
    } else {  // quad_perm lane ^ 2 or lane ^ 1
        constexpr int ctrl = M == 2 ? 0x4E : 0xB1;
        const bool hi = (lane & M) != 0;
        return (hi ? b : a) + __builtin_amdgcn_update_dpp(0, hi ? a : b, ctrl, 0xF, 0xF, false);
    }
}
// Plain butterfly step: v plus the partner's v.
template <int M>
__device__ __forceinline__ int pstep(int v) {
    if constexpr (M == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (int)r[0] + (int)r[1];
    } else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (int)r[0] + (int)r[1];
    } else {
        constexpr int ctrl = M == 8 ? 0x128 : (M == 4 ? 0x141 : (M == 2 ? 0x4E : 0xB1));
        return v + __builtin_amdgcn_update_dpp(0, v, ctrl, 0xF, 0xF, false);
    }
}
template <int M, int NV>
__device__ __forceinline__ void xstage(int (&p)[NV], int& n, int lane) {
    if (n > 1) {
        const int h = n / 2;
#pragma unroll
        for (int i = 0; i < NV / 2; ++i)
            if (i < h) p[i] = tstep<M>(p[i], p[i + h], lane);
        n = h;
    } else {
        p[0] = pstep<M>(p[0]);
    }
}
// Sums each of the NV values (a power of 2, <= 64) over the 64 lanes; afterwards
// p[0] of lane L is the total of value L >> (6 - log2 NV).  The masks are taken
// from the top lane bit down, so the transposing steps consume the high bits and
// the plain steps pair lanes that hold the same value.
template <int NV>
__device__ __forceinline__ void xreduce(int (&p)[NV], int lane) {
    int n = NV;
    xstage<32>(p, n, lane);
    xstage<16>(p, n, lane);
    xstage<8>(p, n, lane);
    xstage<4>(p, n, lane);
    xstage<2>(p, n, lane);
    xstage<1>(p, n, lane);
}

constexpr int log2_of(int v) { return v <= 1 ? 0 : 1 + log2_of(v / 2); }

}  // namespace bitnet
