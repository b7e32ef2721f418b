// gemm_mfma.hip - compute-bound prefill contraction on int8 matrix cores.
//
// acc[m][n] = sum_k q_x[m][k] * q_w[n][k] in int32, y = acc * d_x[m] * d_w.
// The pages describe the contraction as integer additions (Hugging Face
// 1.58-bit write-up, section 계산 패러다임) done by kernels that unpack the
// packed weights on the fly (section 추론 최적화 및 커스텀 커널) over tiles held in
// fast on-chip memory (section 타일링 매트릭스 곱셈).  At prefill sizes the
// contraction is dense and MFMA-bound, so here it runs on
// v_mfma_i32_32x32x32_i8 with the weights' offset codes (q + 1, values 0..2)
// as the A operand and the int8 activations as the B operand; the offset is
// removed in the epilogue with the per-token code sums.  (On gfx950 the
// 32x32x32 form sustains about 1.7x the int8 rate of 16x16x64 in a pure
// register loop, 4.8 vs 2.8 POP/s, so the tiles are built from 32x32 blocks.)
//
// Tiling.  A workgroup of WN x WM wavefronts computes a BN (weight rows) x BM
// (tokens) tile, each wave (BN/WN) x (BM/WM) as 32x32 MFMA blocks.  K advances
// in stages of 256: the int8 activation tile (BM rows x 256 B) and the packed
// weight tile (BN rows x 64 B) are copied straight from HBM/L2 into LDS by
// buffer_load ... lds (no register staging), double buffered, one barrier per
// stage.  64 bytes per weight row per stage is the narrowest access that still
// streams full memory sectors: at 32 bytes per row the weight loads ran at a
// third of the activation loads' rate.
//
// K assignment.  MFMA 32x32x32 takes, per lane, 16 K-values of one A row and
// the same 16 K-values of one B column (lane l: row/column l % 32, half
// h = l / 32); any assignment of K-values to (half, byte) shared by A and B
// gives the same sum.  Here, in K step s (0..7) of a stage, half h covers the
// 16 weights of packed word 8h + s of the stage's 16 words per row (weights
// 128h + 16s .. +15).  So two 16-byte LDS reads give a lane its weight words for
// all eight K steps, each unpacked to natural order by (word >> 2i) & 0x03030303;
// the activation fragment is the matching 16 bytes.  The result D[i][j] sits
// in lane j + 32 * ((i / 4) % 2), element 4 * (i / 8) + i % 4.
//
// LDS layouts (bank-conflict free for the 16-byte fragment reads):
//   activations: row r of 256 B as 16 segments, segment s stored at s ^ (r & 15);
//   weights: row r of 64 B as 4 pieces, piece f stored at f ^ ((r >> 1) ^ (r >> 3)) & 3.
// Rows past M or N and the K tail are zero-filled by the buffer loads' range
// check (the resource covers only the block's valid rows).
//
// Block order.  Workgroups are dispatched round-robin over the 8 XCDs (each
// with its own L2); the launch index is remapped so that each XCD works on a
// contiguous range of tiles, ordered in groups of 8 token tiles per weight
// tile column, so concurrently running blocks on one XCD share operands in L2.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kBK = 256;                         // K values per LDS stage
constexpr int kXcds = 8;                         // XCDs on MI355X
constexpr int kGroupM = 8;                       // token tiles per group in the tile order
constexpr uint32_t kBufferWord3 = 0x00020000u;   // gfx9-family raw buffer descriptor word 3
constexpr uint32_t kOutOfRange = 0x80000000u;    // offset past any block's buffer: loads 0

typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Activation formats of the tiled kernel.
constexpr int kXInt8 = 0, kXE3M2 = 1, kXNibble = 2;

template <int BN_, int BM_, int WN_, int WM_, int OCC_, int S_ = 2, int XF_ = kXInt8, int KS_ = 1>
struct GemmCfg {
    static constexpr int BN = BN_, BM = BM_, WN = WN_, WM = WM_;
    static constexpr int S = S_;                    // LDS stage buffers (S - 1 stages in flight)
    // K groups: KS sets of WN x WM waves share the tile; group g takes the
    // stages g, g + KS, ... with its own stage buffers, and the groups' sums
    // are added through LDS at the end.  With small tiles a single group runs
    // one wave per SIMD, whose stage work (LDS reads, unpacking, dependent
    // MFMAs) has nothing to overlap with; a second group fills that gap.
    // Activation format: int8 codes, 6-bit E3M2 codes (F6: 192 bytes per
    // row per stage, padded to 208 in LDS so 16-byte reads of 16 consecutive
    // rows fall in distinct bank groups), or packed 4-bit codes (I4: 128 bytes
    // per row per stage, eight 16-byte slots stored at s ^ x4_swizzle(r)).
    static constexpr bool F6 = XF_ == kXE3M2;
    static constexpr bool I4 = XF_ == kXNibble;
    static constexpr int X_ROW = F6 ? 208 : (I4 ? kBK / 2 : kBK);   // LDS bytes per activation row
    static constexpr int X_ROW_SLOTS = X_ROW / 16;
    static constexpr int STEPS = F6 ? 4 : 8;         // MFMA K steps per stage (64 or 32 K each)
    static constexpr int OCC = OCC_;                // workgroups per CU the tile is sized for
    static constexpr int KS = KS_;
    static constexpr int NTG = WN * WM * kWave;      // threads per K group
    static constexpr int NT = NTG * KS;
    static constexpr int TN = BN / WN, TM = BM / WM;
    static constexpr int FN = TN / 32, FM = TM / 32;
    static constexpr int X_STAGE = BM * X_ROW;       // bytes
    static constexpr int W_STAGE = BN * (kBK / 4);   // bytes
    static constexpr int X_SLOTS = BM * X_ROW_SLOTS; // 16-byte slots per stage
    static constexpr int W_SLOTS = BN * 4;
    static constexpr int XL = (X_SLOTS + NTG - 1) / NTG;
    static constexpr int WL = (W_SLOTS + NTG - 1) / NTG;
    static constexpr int ROW_F = TN + 4;             // epilogue staging row stride (floats)
    static_assert((ROW_F / 4) % 2 == 1, "odd number of 16-byte units per staging row");
    static_assert(WN * WM * 16 * ROW_F * 4 <= S * (X_STAGE + W_STAGE), "epilogue staging fits");
    static_assert(TN % 32 == 0 && TM % 32 == 0, "wave tile must be whole MFMA blocks");
    static_assert(X_SLOTS % kWave == 0 && W_SLOTS % kWave == 0, "whole waves per load");
    static_assert(KS * S * (X_STAGE + W_STAGE) <= 160 * 1024, "LDS");
    static_assert(KS == 1 || WN * WM * kWave * FN * FM * 16 * 4 <= S * (X_STAGE + W_STAGE),
                  "a K group's partial sums fit its stage buffers");
    // With more than one stage in flight the stage barrier counts outstanding
    // loads, so every wave must issue the same number per stage.
    static_assert(S == 2 || (X_SLOTS % NTG == 0 && W_SLOTS % NTG == 0), "uniform loads per wave");
    static_assert(S >= 2 && (S - 2) * (XL + WL) <= 63, "vmcnt range");
    static_assert(NT <= 1024, "workgroup size");
};

// Two packed words (32 offset codes c = q + 1, weights 0..15 in w and 16..31
// in w2) -> 32 FP4 (E2M1) values: code c of weight 4 d + b of w goes to
// nibble 2 b of dword d, that of w2 to nibble 2 b + 1.  The nibble is the code
// itself, the E2M1 value c / 2 (0, 0.5 and 1 are exact: 0.5 is the subnormal),
// and the operand's block scale 2^1 makes it c again.  Per dword: the code
// fields of w masked in place and those of w2 shifted into the high nibble,
// merged by one and-or.
__device__ __forceinline__ v8i unpack_fp4(uint32_t w, uint32_t w2) {
    v8i r = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    r[0] = (int)((w & 0x03030303u) | ((w2 << 4) & 0x30303030u));
    r[1] = (int)(((w >> 2) & 0x03030303u) | ((w2 << 2) & 0x30303030u));
    r[2] = (int)(((w >> 4) & 0x03030303u) | (w2 & 0x30303030u));
    r[3] = (int)(((w >> 6) & 0x03030303u) | ((w2 >> 2) & 0x30303030u));
    return r;
}

constexpr int kFmtFp4 = 4;      // MFMA operand format selector: FP4 E2M1
constexpr int kFmtE3M2 = 3;     // MFMA operand format selector: 6-bit E3M2
constexpr int kScaleOne = 127;  // E8M0 block scale 2^0
constexpr int kScaleTwo = 128;  // E8M0 block scale 2^1 (the FP4 weight operand: nibble c means c / 2)

__device__ __forceinline__ v4i unpack_codes(uint32_t w) {
    v4i r;
    r[0] = (int)(w & 0x03030303u);
    r[1] = (int)((w >> 2) & 0x03030303u);
    r[2] = (int)((w >> 4) & 0x03030303u);
    r[3] = (int)((w >> 6) & 0x03030303u);
    return r;
}

// Weight-tile swizzle: piece f of row r is stored at piece f ^ w_swizzle(r).
// Any 8 consecutive rows (and any 16 rows of a 16-row block) then hit distinct
// 16-byte bank groups when a lane group reads the same piece of each row.
__device__ __forceinline__ int w_swizzle(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// Nibble activation rows (128 bytes, eight 16-byte slots): slot s of row r is
// stored at s ^ x4_swizzle(r).  LDS serves 256 bytes per cycle, so two rows
// cover its banks; pairing the row's parity with three more row bits gives 16
// consecutive rows distinct banks for a 16-byte read of the same slot.
__device__ __forceinline__ int x4_swizzle(int r) { return (r >> 1) & 7; }

// All of this wave's loads into LDS have landed and its LDS reads are done,
// then the workgroup barrier.  Written as one asm statement with a memory
// clobber so the compiler neither moves LDS accesses across it nor adds a
// wait of its own for loads still in flight elsewhere.
template <int N>
__device__ __forceinline__ void stage_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Activation codes as 6-bit E3M2 floats (the f6 format), for the FP4 x FP6
// matrix core: a 32-value group is 24 bytes; value p of the group (bits 6p ..
// 6p+5 of its little-endian 192-bit word) is the code at K offset
// 16 (p % 2) + 4 (p / 8) + (p % 8) / 2, the order in which the packed weights
// unpack into FP4 nibbles below.
template <class C>
__global__ __launch_bounds__(C::NT, C::OCC) void gemm_kernel(
    const int8_t* __restrict__ X, const uint8_t* __restrict__ P, const float* __restrict__ x_scale,
    const int32_t* __restrict__ x_qsum, const RowScales scales, int M, int N, int K,
    int vec_store, float* __restrict__ y, int32_t* __restrict__ acc_out) {
    __shared__ __align__(16) int8_t lds_all[C::KS][C::S][C::X_STAGE + C::W_STAGE];

    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wave_all = __builtin_amdgcn_readfirstlane(t / kWave);   // wave-uniform, in an SGPR
    const int kg = wave_all / (C::WN * C::WM);                       // K group
    const int wave = wave_all % (C::WN * C::WM);                     // wave within the group
    const int wn = wave % C::WN, wm = wave / C::WN;
    auto& lds = lds_all[kg];

    // Launch index -> tile: contiguous ranges per XCD, grouped order.
    const int tiles_n = (N + C::BN - 1) / C::BN;
    const int tiles_m = (M + C::BM - 1) / C::BM;
    const int total = tiles_n * tiles_m;
    const int per = total / kXcds, rem = total % kXcds;
    const int xcd = (int)blockIdx.x % kXcds, idx = (int)blockIdx.x / kXcds;
    const int tile = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
    const int group = tile / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int in_group = tile % (kGroupM * tiles_n);
    const int tm = first_m + in_group % gsize;
    const int tn = in_group / gsize;
    const int64_t n0 = (int64_t)tn * C::BN;
    const int64_t m0 = (int64_t)tm * C::BM;
    const int row_bytes = K / 4;

    // Buffer resources cover only this block's valid rows.
    const int x_rows = (int)min((int64_t)C::BM, (int64_t)M - m0);
    const int w_rows = (int)min((int64_t)C::BN, (int64_t)N - n0);
    const int x_row_bytes = C::F6 ? K / 4 * 3 : (C::I4 ? K / 2 : K);   // activation bytes per token in HBM
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(X + m0 * x_row_bytes), (short)0, x_rows * x_row_bytes, (int)kBufferWord3);
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(P + n0 * row_bytes), (short)0, w_rows * row_bytes, (int)kBufferWord3);

    // Copy one stage into LDS buffer `buf`: load instruction idx (0 .. XL + WL - 1)
    // of this wave moves 1 KiB; lane l of the wave fills the 16-byte slot
    // base + l, so the global address each lane reads is chosen to realise the
    // swizzled layout.
    // When `live` is false the load reads out of range (zeros, no memory
    // traffic) but is still issued, so a stage's loads are straight-line code
    // and every wave counts the same number of them.
    constexpr int kLoads = C::XL + C::WL;
    auto issue_one = [&](int buf, int k0, int idx, bool live) {
        if (idx < C::XL) {
            const int base = idx * C::NTG + wave * kWave;   // wave-uniform
            if (C::X_SLOTS % C::NTG == 0 || base < C::X_SLOTS) {
                const int p = base + lane;
                uint32_t off;
                if constexpr (C::F6) {
                    // 12 data slots and one padding slot per row, in order.
                    const int r = p / C::X_ROW_SLOTS, s = p % C::X_ROW_SLOTS;
                    const int b = k0 / 4 * 3 + 16 * s;             // byte in the token's row
                    off = (live && s < 12 && b < x_row_bytes) ? (uint32_t)(r * x_row_bytes + b) : kOutOfRange;
                } else if constexpr (C::I4) {
                    const int r = p >> 3, s = (p & 7) ^ x4_swizzle(r);
                    const int b = k0 / 2 + 16 * s;
                    off = (live && b < x_row_bytes) ? (uint32_t)(r * x_row_bytes + b) : kOutOfRange;
                } else {
                    const int r = p >> 4, s = (p & 15) ^ (r & 15);
                    const int k = k0 + 16 * s;
                    off = (live && k < K) ? (uint32_t)(r * K + k) : kOutOfRange;
                }
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_void*)&lds[buf][base * 16], 16,
                                                         (int)off, 0, 0, 0);
            }
        } else {
            const int base = (idx - C::XL) * C::NTG + wave * kWave;
            if (C::W_SLOTS % C::NTG == 0 || base < C::W_SLOTS) {
                const int p = base + lane;
                const int r = p >> 2, f = (p & 3) ^ w_swizzle(r);
                const int k = k0 + 64 * f;
                const uint32_t off = (live && k < K) ? (uint32_t)(r * row_bytes + k / 4) : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    wres, (lds_void*)&lds[buf][C::X_STAGE + base * 16], 16, (int)off, 0, 0, 0);
            }
        }
    };

    using Acc = typename std::conditional<C::F6, v16f, v16i>::type;
    Acc acc[C::FN][C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    const int fr = lane % 32, fh = lane / 32;
    // One stage of MFMAs on LDS buffer `buf`; the loads of a later stage (into
    // buffer `nbuf`) are issued during the first four of the eight K steps, so
    // the address unit works while the matrix cores do (instead of every wave
    // issuing all its loads at once after the barrier) and the loads still have
    // the rest of the stage to land.
    auto compute = [&](int buf, bool has_next, int nbuf, int next_k0) {
        const int8_t* xs = &lds[buf][0];
        const int8_t* ws = &lds[buf][C::X_STAGE];
        v4u wv[C::FN][2];
        v4u xr[C::FM];   // I4: the 16-byte slot holding two K steps' codes
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
            const int r = wn * C::TN + i * 32 + fr;
#pragma unroll
            for (int p = 0; p < 2; ++p)
                wv[i][p] = *reinterpret_cast<const v4u*>(
                    &ws[r * 64 + 16 * ((2 * fh + p) ^ w_swizzle(r))]);
        }
#pragma unroll
        for (int st = 0; st < C::STEPS; ++st) {
            // Waves on one SIMD are otherwise served oldest first, so within a
            // stage the youngest wave finishes last while the others wait at
            // the barrier with the matrix core half idle.  Lowering a wave's
            // priority as it advances through the stage lets the waves that
            // are behind catch up (measured: about 4% on the prefill shape).
            if (st == 0) __builtin_amdgcn_s_setprio(3);
            if (st == C::STEPS / 4) __builtin_amdgcn_s_setprio(2);
            if (st == C::STEPS / 2) __builtin_amdgcn_s_setprio(1);
            if (st == 3 * C::STEPS / 4) __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int idx = 0; idx < kLoads; ++idx)
                if (idx * (C::STEPS / 2) / kLoads == st) issue_one(nbuf, next_k0, idx, has_next);
            if constexpr (C::F6) {
                // K step st of lane half fh: packed words 8 fh + 2 st and 8 fh + 2 st + 1
                // (64 consecutive K values per step over the two halves) against the
                // activation group 4 fh + st (24 bytes).
                v8i b[C::FM];
#pragma unroll
                for (int j = 0; j < C::FM; ++j) {
                    const int r = wm * C::TM + j * 32 + fr;
                    const uint2* src = reinterpret_cast<const uint2*>(&xs[r * C::X_ROW + 96 * fh + 24 * st]);
                    const uint2 q0 = src[0], q1 = src[1], q2 = src[2];
                    b[j] = v8i{(int)q0.x, (int)q0.y, (int)q1.x, (int)q1.y, (int)q2.x, (int)q2.y, 0, 0};
                }
#pragma unroll
                for (int i = 0; i < C::FN; ++i) {
                    const uint32_t w = wv[i][st / 2][2 * (st % 2)];
                    const uint32_t w2 = wv[i][st / 2][2 * (st % 2) + 1];
                    const v8i a = unpack_fp4(w, w2);
#pragma unroll
                    for (int j = 0; j < C::FM; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            a, b[j], acc[i][j], kFmtFp4, kFmtE3M2, 0, kScaleTwo, 0, kScaleOne);
                }
            } else {
                v4i b[C::FM];
#pragma unroll
                for (int j = 0; j < C::FM; ++j) {
                    const int r = wm * C::TM + j * 32 + fr;
                    if constexpr (C::I4) {
                        // Group 8 fh + st of the stage (16 codes in 8 bytes): byte i
                        // holds codes i and 8 + i, so masking the high nibbles of
                        // the two dwords (and of the dwords shifted up by 4) gives
                        // 16 q in natural order, as int8.  The sums are 16 times
                        // the codes' and are scaled back in the epilogue.
                        if (st % 2 == 0)
                            xr[j] = *reinterpret_cast<const v4u*>(
                                &xs[r * C::X_ROW + 16 * ((4 * fh + st / 2) ^ x4_swizzle(r))]);
                        const uint32_t lo = xr[j][2 * (st % 2)], hi = xr[j][2 * (st % 2) + 1];
                        b[j] = v4i{(int)((lo << 4) & 0xF0F0F0F0u), (int)((hi << 4) & 0xF0F0F0F0u),
                                   (int)(lo & 0xF0F0F0F0u), (int)(hi & 0xF0F0F0F0u)};
                    } else {
                        b[j] = *reinterpret_cast<const v4i*>(&xs[r * kBK + 16 * ((8 * fh + st) ^ (r & 15))]);
                    }
                }
#pragma unroll
                for (int i = 0; i < C::FN; ++i) {
                    const v4i a = unpack_codes(wv[i][st / 4][st % 4]);
#pragma unroll
                    for (int j = 0; j < C::FM; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b[j], acc[i][j], 0, 0, 0);
                }
            }
        }
    };

    // Group kg takes the stages kg, kg + KS, ...; every group runs the same
    // number of iterations (a group past the end computes nothing and loads
    // zeros) so the workgroup barriers line up.
    const int nk = (K + kBK - 1) / kBK;
    const int nkl = (nk + C::KS - 1) / C::KS;
    auto stage_k0 = [&](int local) { return (local * C::KS + kg) * kBK; };
    auto stage_live = [&](int local) { return local * C::KS + kg < nk; };
#pragma unroll
    for (int sp = 0; sp < C::S - 1; ++sp) {
        if (sp < nkl) {
#pragma unroll
            for (int idx = 0; idx < kLoads; ++idx) issue_one(sp, stage_k0(sp), idx, stage_live(sp));
        }
    }
    for (int kt = 0; kt < nkl; ++kt) {
        // Stage kt has landed once at most the loads of the stages issued after
        // it are outstanding; every wave has finished reading buffer
        // (kt - 1) % S, which the loads of stage kt + S - 1 overwrite.
        if (kt + C::S - 2 < nkl)
            stage_barrier<(C::S - 2) * kLoads>();
        else
            stage_barrier<0>();
        // (A stage past K holds zeros and adds nothing; its loads are still
        // issued, so the outstanding-load counts stay uniform.)
        const int ahead = kt + C::S - 1;
        compute(kt % C::S, stage_live(ahead), ahead % C::S, stage_k0(ahead));
    }

    // The last stages' out-of-range loads may still be writing (zeros) into
    // LDS; every wave waits for its own before the stage buffers are reused.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (C::KS > 1) {
        // Groups 1.. add their sums into group 0 through LDS (each group's
        // stage buffers hold its partials), group by group.
        __syncthreads();
        using Elem = typename std::conditional<C::F6, float, int>::type;
        Elem* part = reinterpret_cast<Elem*>(&lds_all[kg][0][0]) + wave * (kWave * C::FN * C::FM * 16);
        if (kg > 0) {
#pragma unroll
            for (int i = 0; i < C::FN; ++i)
#pragma unroll
                for (int j = 0; j < C::FM; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) part[((i * C::FM + j) * 16 + e) * kWave + lane] = acc[i][j][e];
        }
        __syncthreads();
        if (kg > 0) return;   // wave-uniform; no workgroup barrier follows
#pragma unroll
        for (int g = 1; g < C::KS; ++g) {
            const Elem* src = reinterpret_cast<const Elem*>(&lds_all[g][0][0]) + wave * (kWave * C::FN * C::FM * 16);
#pragma unroll
            for (int i = 0; i < C::FN; ++i)
#pragma unroll
                for (int j = 0; j < C::FM; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][j][e] += src[((i * C::FM + j) * 16 + e) * kWave + lane];
        }
    }

    // Epilogue.  D[n][m] of a 32x32 block sits in lane m + 32 * ((n / 4) % 2),
    // element 4 * (n / 8) + n % 4: a lane holds four runs of 4 consecutive
    // outputs of one token, so direct stores would each cover 32 rows of y with
    // 16 bytes.  Instead each wave dequantises 16 tokens at a time into its own
    // LDS region (row stride TN + 4 floats keeps the 16-byte writes conflict
    // free) and writes them back as whole row segments of TN floats.
    const float dw0 = scales.w_scale[0];
    if constexpr (C::KS == 1) __syncthreads();   // every wave is done with the stage buffers
    float* stage = reinterpret_cast<float*>(&lds_all[0][0][0]) + wave * 16 * C::ROW_F;
    constexpr int PPR = C::TN / 4;              // 16-byte pieces per row segment
    constexpr int RPI = kWave / PPR;            // row segments per store instruction
    static_assert(RPI >= 1 && 16 % RPI == 0, "row segments per store");
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t mr = m0 + wm * C::TM + j * 32 + half * 16;   // first token staged
            if (fr / 16 == half) {
                const int64_t m = mr + fr % 16;
                const int32_t qs = m < M ? x_qsum[m] : 0;
                const float sx = m < M ? x_scale[m] : 0.f;
#pragma unroll
                for (int i = 0; i < C::FN; ++i) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int nl = i * 32 + 8 * q + 4 * fh;   // wave-local output column
                        const int64_t ng = n0 + wn * C::TN + nl;   // its global column
                        // (the FP4 x FP6 sums are exact integers in float32)
                        v4i a = v4i{(int)acc[i][j][4 * q], (int)acc[i][j][4 * q + 1],
                                    (int)acc[i][j][4 * q + 2], (int)acc[i][j][4 * q + 3]};
                        if constexpr (C::I4) a = a >> 4;   // exact: the sums are multiples of 16
                        a -= v4i{qs, qs, qs, qs};
                        // Columns past N read row N-1's scale; they are never stored.
                        float4 v;
                        v.x = ((float)a[0] * sx) * scales.of(min(ng, (int64_t)N - 1), dw0);
                        v.y = ((float)a[1] * sx) * scales.of(min(ng + 1, (int64_t)N - 1), dw0);
                        v.z = ((float)a[2] * sx) * scales.of(min(ng + 2, (int64_t)N - 1), dw0);
                        v.w = ((float)a[3] * sx) * scales.of(min(ng + 3, (int64_t)N - 1), dw0);
                        *reinterpret_cast<float4*>(&stage[(fr % 16) * C::ROW_F + nl]) = v;
                        if (acc_out != nullptr && m < M) {
                            const int64_t nb = n0 + wn * C::TN + nl;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (nb + e < N) acc_out[m * N + nb + e] = a[e];
                        }
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int rr = 0; rr < 16; rr += RPI) {
                const int row = rr + lane / PPR, piece = lane % PPR;
                const int64_t m = mr + row;
                const int64_t nb = n0 + wn * C::TN + 4 * piece;
                if (lane < RPI * PPR && m < M && nb < N) {
                    const float4 v =
                        *reinterpret_cast<const float4*>(&stage[row * C::ROW_F + 4 * piece]);
                    if (vec_store && nb + 3 < N) {
                        // Streaming store: y is written once and not re-read by this
                        // kernel, so it should not displace operand lines in L2.
                        __builtin_nontemporal_store(f4{v.x, v.y, v.z, v.w},
                                                    reinterpret_cast<f4*>(&y[m * N + nb]));
                    } else {
                        const float ve[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (nb + e < N) y[m * N + nb + e] = ve[e];
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
    }
}

// Skinny contraction (M <= 16 tokens).  One workgroup owns R blocks of 16
// weight rows; its K range is split over the workgroup's KW waves (stage kt
// goes to wave kt % KW, so at any time the waves read adjacent bytes of each
// row).  A lane's MFMA fragments are contiguous in memory (16 bytes of packed
// weights per row block, 64 bytes of activations per stage, in the K assignment
// described above), so they are loaded straight into registers with no LDS
// staging; the next stage's loads are issued before the current stage's MFMAs.
// A wave loads each activation fragment once and uses it for all R row blocks,
// so the activations read from L2 shrink to 64 / R bytes per 16 bytes of packed
// weights.  The KW partial accumulators are summed through LDS, row block r by
// wave r % KW, which runs its epilogue.
template <int KW, int R>
__global__ __launch_bounds__(KW * kWave) void skinny_kernel(
    const int8_t* __restrict__ X, const uint8_t* __restrict__ P, const float* __restrict__ x_scale,
    const int32_t* __restrict__ x_qsum, const RowScales scales, int M, int N, int K,
    int vec_store, float* __restrict__ y, int32_t* __restrict__ acc_out) {
    __shared__ v4i part[KW][R][kWave];
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int fr = lane % 16, fg = lane / 16;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * R;
    const int row_bytes = K / 4;
    bool w_ok[R];
    const uint8_t* wp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = n0 + 16 * r + fr;
        w_ok[r] = n < N;
        // Rows past N or M read row 0 (always valid) and are masked to zero.
        wp[r] = P + (w_ok[r] ? n * row_bytes : 0) + 16 * fg;
    }
    const bool x_ok = fr < M;
    const int8_t* xp = X + (x_ok ? (int64_t)fr * K : 0) + 64 * fg;
    const int nk = (K + kBK - 1) / kBK;

    struct Frag {
        v4u w[R];
        v4i x[4];
    };
    auto load = [&](int kt, Frag& f) {
        const int k0 = kt * kBK;
        // K is a multiple of 64, so a lane group's 64 K-values are all in range or all out.
        const bool in_k = kt < nk && k0 + 64 * fg < K;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (in_k && w_ok[r]) {
                f.w[r] = *reinterpret_cast<const v4u*>(wp[r] + k0 / 4);
            } else {
                f.w[r] = v4u{0, 0, 0, 0};
            }
        }
        if (in_k && x_ok) {
            const v4i* src = reinterpret_cast<const v4i*>(xp + k0);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) f.x[ks] = src[ks];
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) f.x[ks] = v4i{0, 0, 0, 0};
        }
    };

    v4i acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = v4i{0, 0, 0, 0};
    Frag cur, nxt;
    load(wave, cur);
    for (int kt = wave; kt < nk; kt += KW) {
        load(kt + KW, nxt);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack_codes(cur.w[r][ks]), cur.x[ks], acc[r],
                                                               0, 0, 0);
        cur = nxt;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) part[wave][r][lane] = acc[r];
    __syncthreads();

    const int m = fr;
    const int32_t qs = m < M ? x_qsum[m] : 0;
    const float sx = m < M ? x_scale[m] : 0.f;
    const float dw0 = scales.w_scale[0];
    for (int r = wave; r < R; r += KW) {   // wave-uniform
        v4i a = part[0][r][lane];
#pragma unroll
        for (int w = 1; w < KW; ++w) a += part[w][r][lane];
        // D[n][m] sits in lane m + 16 * (n / 4), element n % 4.
        const int64_t nb = n0 + 16 * r + 4 * fg;
        if (m >= M || nb >= N) continue;
        a -= v4i{qs, qs, qs, qs};
        if (vec_store && nb + 3 < N) {
            if (acc_out != nullptr) *reinterpret_cast<v4i*>(&acc_out[m * N + nb]) = a;
            float4 v;
            v.x = ((float)a[0] * sx) * scales.of(nb, dw0);
            v.y = ((float)a[1] * sx) * scales.of(nb + 1, dw0);
            v.z = ((float)a[2] * sx) * scales.of(nb + 2, dw0);
            v.w = ((float)a[3] * sx) * scales.of(nb + 3, dw0);
            *reinterpret_cast<float4*>(&y[m * N + nb]) = v;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (nb + e < N) {
                    if (acc_out != nullptr) acc_out[m * N + nb + e] = a[e];
                    y[m * N + nb + e] = ((float)a[e] * sx) * scales.of(nb + e, dw0);
                }
            }
        }
    }
}

template <int KW, int R>
hipError_t launch_skinny(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                         const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                         int64_t K, float* y, int32_t* acc, hipStream_t stream) {
    const int vec_store = (N % 4 == 0) && ((uintptr_t)y % 16 == 0) &&
                          (acc == nullptr || (uintptr_t)acc % 16 == 0);
    return launch_kernel(skinny_kernel<KW, R>, dim3((unsigned)((N + 16 * R - 1) / (16 * R))),
                         dim3(KW * kWave), 0, stream, xq, packed, x_scale, x_qsum, scales, (int)M,
                         (int)N, (int)K, vec_store, y, acc);
}

template <class C>
int64_t tiles_of(int64_t M, int64_t N) {
    return ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
}

template <class C>
hipError_t launch_cfg(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                      const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N, int64_t K,
                      float* y, int32_t* acc, hipStream_t stream) {
    const int vec_store = (N % 4 == 0) && ((uintptr_t)y % 16 == 0) &&
                          (acc == nullptr || (uintptr_t)acc % 16 == 0);
    return launch_kernel(gemm_kernel<C>, dim3((unsigned)tiles_of<C>(M, N)), dim3(C::NT), 0, stream,
                         xq, packed, x_scale, x_qsum, scales, (int)M, (int)N, (int)K, vec_store, y,
                         acc);
}

// Tile configurations (weight rows x tokens, waves along N x along M,
// workgroups per CU, stage buffers, 6-bit activations, K groups).
template <int XF>
struct Tiles {
    using Large = GemmCfg<448, 128, 7, 2, 1, 2, XF>;        // 14 waves, wave tile 64 x 64
    using Square = GemmCfg<128, 128, 4, 2, 1, 2, XF>;       // 8 waves, wave tile 32 x 64
    using TallK3 = GemmCfg<128, 64, 2, 2, 1, 2, XF, 3>;     // 3 K groups of 4 waves (64 x 32)
    using TallK2 = GemmCfg<128, 64, 2, 2, 1, 2, XF, 2>;     // 2 K groups of 4 waves (64 x 32)
    using Tiny = GemmCfg<64, 64, 2, 2, 2, 2, XF>;           // 4 waves, wave tile 32 x 32 (tile count only)
    using TinyK2 = GemmCfg<64, 64, 2, 2, 2, 2, XF, 2>;      // 2 K groups of 4 waves
    using TinyK4 = GemmCfg<64, 64, 2, 2, 1, 2, XF, 4>;      // 4 K groups of 4 waves
};

constexpr int64_t kCus = 256;

// Tile choice.  The 448 x 128 tile when it gives two or more full rounds of
// the 256 CUs, or between three quarters of one round and one round; else the
// 128 x 128 tile when it gives at least 7/8 of a round; below that 128 x 64
// and 64 x 64 tiles, whose waves (one 64 x 32 or 32 x 32 block each) have
// little to overlap a stage's LDS reads and dependent MFMAs with: K groups add
// waves that work on other stages of the same tile, the more the longer K or
// the fewer the tiles (128 x 64 tiles in two K groups when there are >= 384
// 64 x 64 tiles' worth of output and <= 32 stages: 5% ahead of one group of
// 64 x 64 tiles at M 256 x N 6144 and M 512 x N 4096; four K groups of 64 x 64
// tiles up to one round: 7-9% ahead of two at M 256, N 4096 and 1024).  Measured (graph replays
// over >= 1 GiB of weight copies) on the prefill, H-BitLinear (M 512) and
// Llama-block (M 256) shapes and on M 256 ... 2048 at N 8192 ... 28672: the
// 128 x 128 tile beat the 256 x 128 and 256 x 64 tiles it replaced by 3-15%
// wherever they were chosen (and the K-group 64 x 64 tiles at K 14336 and
// 16384 by 11-12% once it has 7/8 of a round), lost to the 448 x 128 tile
// between 3/4 and one round of that tile (51.1 against 55.4 us at M 768,
// N 14336) and at two rounds (the prefill FFN shape), and won at 1.5 rounds.
template <int XF>
hipError_t launch_tiled(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                        const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                        int64_t K, float* y, int32_t* acc, hipStream_t stream) {
    using T = Tiles<XF>;
    const int64_t large = tiles_of<typename T::Large>(M, N);
    if (large >= 2 * kCus || (large >= 3 * kCus / 4 && large <= kCus))
        return launch_cfg<typename T::Large>(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, stream);
    if (tiles_of<typename T::Square>(M, N) >= 7 * kCus / 8)
        return launch_cfg<typename T::Square>(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, stream);
    const int64_t tiles = tiles_of<typename T::Tiny>(M, N);
    const int64_t stages = (K + kBK - 1) / kBK;
    if (stages >= 48 && tiles >= 2 * kCus)
        return launch_cfg<typename T::TallK3>(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, stream);
    if (stages >= 48)
        return launch_cfg<typename T::TinyK4>(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, stream);
    if (tiles >= 384 && stages <= 32)
        return launch_cfg<typename T::TallK2>(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, stream);
    if (tiles <= kCus)
        return launch_cfg<typename T::TinyK4>(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, stream);
    return launch_cfg<typename T::TinyK2>(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, stream);
}

}  // namespace

hipError_t launch_gemm(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                       const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                       int64_t K, float* y, int32_t* acc, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    if (M <= 16) {
        // Row blocks per workgroup grow with N (fewer activation re-reads from
        // L2) while the grid keeps >= ~1300 waves; K is split eight ways, or
        // four for the largest N.  Measured at M = 16 on 7B / 8B projection
        // shapes (N 1024 ... 28672, K 4096 ... 14336).
        if (N >= 24576)
            return launch_skinny<4, 4>(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, stream);
        if (N >= 10240)
            return launch_skinny<8, 4>(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, stream);
        if (N >= 5120)
            return launch_skinny<8, 2>(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, stream);
        return launch_skinny<8, 1>(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, stream);
    }
    return launch_tiled<kXInt8>(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, stream);
}

hipError_t launch_gemm_f6(const uint8_t* xq6, const float* x_scale, const int32_t* x_qsum,
                          const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                          int64_t K, float* y, int32_t* acc, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    return launch_tiled<kXE3M2>(reinterpret_cast<const int8_t*>(xq6), x_scale, x_qsum, packed, scales, M,
                                N, K, y, acc, stream);
}

hipError_t launch_gemm_i4(const uint8_t* xq4, const float* x_scale, const int32_t* x_qsum,
                          const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                          int64_t K, float* y, int32_t* acc, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    return launch_tiled<kXNibble>(reinterpret_cast<const int8_t*>(xq4), x_scale, x_qsum, packed, scales,
                                  M, N, K, y, acc, stream);
}

}  // namespace bitnet
