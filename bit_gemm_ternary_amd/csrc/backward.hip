// backward.hip - BitLinear backward under the straight-through estimator.
//
// The estimator gives round() the gradient 1 (Hugging Face 1.58-bit write-up,
// section "Straight-Through Estimator (STE)를 이용한 학습"), so both quantisers
// pass gradients through unchanged.  Seen by it, the forward is y = n~ W~^T
// with the dequantised operands n~ = d_x q_x (standing for the normalised
// activation n = x * gain * r) and W~ = d_w q_w (standing for W), hence
//   dL/dn = dL/dy W~        (bf16 x ternary contraction over the N outputs)
//   dL/dW = (dL/dy)^T n~    (contraction over the M tokens)
// and dL/dx follows from the RMSNorm in front of the quantiser (section
// "양자화 메커니즘": the activations are normalised before quantisation).
//
// Both contractions run on v_mfma_f32_32x32x16_bf16 in one "NT" GEMM kernel,
// C[r][c] = sum_j A[r][j] B[c][j], with both operands contiguous along j and
// staged into LDS by the buffer-load-to-LDS path.  For dL/dn, B is the packed
// ternary matrix transposed once to [K][N/4] (pack once, like the forward):
// its tile stays 2-bit in LDS and each lane turns 8 codes into 8 bf16 values
// in {-1, 0, 1} with byte permutes (the codes index a table of bf16 bytes),
// so the products grad_y * q are exact and only the float32 accumulation
// rounds.  That conversion is vector-ALU work per 32 x 32 block of B, shared
// by the WR blocks of A a wave multiplies it with, so dL/dn uses tall wave
// tiles (128 x 64) and two K groups to keep two waves per SIMD.  For dL/dW,
// p = grad_y * d_x is carried as a bf16 pair hi + lo (hi = bf16(p),
// lo = bf16(p - hi), |p - hi - lo| <= 2^-16 |p|) and the activation codes
// (exact in bf16) are shared: the operands are A = [hi | lo] ([N][2 Mp]) and
// B = codes ([K][Mp]), transposed so that the token index m runs along the
// rows; a stage holds both planes of A, and each B fragment read from LDS
// feeds the hi and the lo product.  With both tiles bf16 the kernel is bound
// by LDS bandwidth and capacity.
#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer descriptor word 3 (gfx9 family)
constexpr uint32_t kOutOfRange = 0x80000000u;   // offset past every buffer here: loads 0
constexpr int kBJ = 64;                          // reduction values per LDS stage
constexpr int kThreads = 256;
constexpr int kXcds = 8;                         // XCDs on MI355X, each with its own L2

__device__ __forceinline__ uint16_t bf16_rne(float f) {  // finite inputs
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------------------
// packed [N][K/4] -> packed_t [K][N/4], both in the forward's layout along
// their rows (word g holds values 16g..16g+15; value 16g + 4i + b at bits
// 2i..2i+1 of byte b).  A workgroup moves 64 rows of N by kTK values of K:
// each thread loads 16 bytes of one row and writes the 16 bytes (64 codes)
// of one output row.
// ---------------------------------------------------------------------------
constexpr int kTK = 256;

__global__ __launch_bounds__(kThreads) void transpose_packed_kernel(const uint8_t* __restrict__ packed,
                                                                   int N, int K,
                                                                   uint8_t* __restrict__ packed_t) {
    static_assert(kTK == kThreads && kTK % 64 == 0, "one output row per thread");
    __shared__ uint32_t tile[64][kTK / 16 + 1];  // [n][word of k], padded
    const int n0 = (int)blockIdx.y * 64, k0 = (int)blockIdx.x * kTK;
    const int t = threadIdx.x;
    {
        const int r = t / 4, p = t % 4;  // row n0 + r, values k0 + 64p .. k0 + 64p + 63
        uint4 v = make_uint4(0, 0, 0, 0);
        if (k0 + 64 * p < K)
            v = *reinterpret_cast<const uint4*>(packed + (int64_t)(n0 + r) * (K / 4) + k0 / 4 + 16 * p);
        tile[r][4 * p] = v.x;
        tile[r][4 * p + 1] = v.y;
        tile[r][4 * p + 2] = v.z;
        tile[r][4 * p + 3] = v.w;
    }
    __syncthreads();
    const int k = k0 + t;  // my output row
    if (k >= K) return;
    const int kw = t / 16, kshift = 8 * (t % 4) + 2 * ((t % 16) / 4);
    uint32_t out[4] = {0, 0, 0, 0};  // word wn: n = n0 + 16 wn .. n0 + 16 wn + 15
#pragma unroll
    for (int wn = 0; wn < 4; ++wn)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t field = (tile[16 * wn + 4 * i + b][kw] >> kshift) & 3u;
                out[wn] |= field << (8 * b + 2 * i);
            }
    *reinterpret_cast<uint4*>(packed_t + (int64_t)k * (N / 4) + n0 / 4) = make_uint4(out[0], out[1], out[2], out[3]);
}

// ---------------------------------------------------------------------------
// NT GEMM on the bf16 matrix cores.  Workgroup tile BR x BC = 64 WR x 64 WC,
// 2 x 2 waves, a wave WR x WC blocks of 32 x 32; K steps of 16 inside LDS
// stages of 64.  TERN: B is 2-bit codes q+1 ([C][J/4] bytes), else bf16.
// ---------------------------------------------------------------------------
template <int WR_, int WC_, int GR_, int GC_, int KS_, bool TERN_, int NS_, int GROUP_, int PL_ = 1>
struct BwdCfg {
    static constexpr bool TERN = TERN_;                      // B is 2-bit codes, else bf16
    // A planes: with PL = 2 a row of A holds two J-long planes (the hi and lo
    // halves of dL/dW's left operand), both multiplied with the same B value,
    // so each B fragment read from LDS serves both.
    static constexpr int PL = PL_;
    static constexpr int WR = WR_, WC = WC_;                 // 32 x 32 blocks per wave
    static constexpr int GR = GR_, GC = GC_;                 // waves of a K group along rows / columns
    static constexpr int KS = KS_;                           // K groups (stage js goes to group js % KS)
    static constexpr int NS = NS_;                           // LDS stages in each group's ring
    static constexpr int GROUP = GROUP_;                     // row tiles per group of the tile order
    static constexpr int GW = GR * GC;                       // waves per K group
    static constexpr int GT = GW * kWave;                    // threads per K group
    static constexpr int NT = GT * KS;                       // threads per workgroup
    static constexpr int BR = 32 * WR * GR;                  // rows per workgroup
    static constexpr int BC = 32 * WC * GC;                  // columns per workgroup
    static constexpr int A_PLANE = BR * kBJ * 2;             // one A plane of a stage
    static constexpr int A_BYTES = PL * A_PLANE;
    static constexpr int B_BYTES = TERN ? BC * kBJ / 4 : BC * kBJ * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int RING = NS * STAGE;                  // one group's stages
    static constexpr int A_SLOTS = A_BYTES / 16;              // 16-byte load slots
    static constexpr int B_SLOTS = B_BYTES / 16;
    // 2-bit B: waves 0 .. B_WAVES - 1 of a group load the codes, the others
    // issue an out-of-range load into a spare 1 KiB, so every wave counts the
    // same loads.
    static constexpr int B_WAVES = TERN ? B_SLOTS / kWave : 0;
    static constexpr int SPARE = TERN && B_WAVES < GW ? kWave * 16 : 0;
    static constexpr int LOADS = A_SLOTS / GT + (TERN ? 1 : B_SLOTS / GT);  // per wave per stage
    static constexpr int PARTIAL = KS > 1 ? GW * WR * WC * 16 * kWave * 4 : 0;  // one group's sums
    static constexpr int LDS = KS * RING + SPARE > PARTIAL ? KS * RING + SPARE : PARTIAL;
    static_assert(A_SLOTS % GT == 0 && (A_PLANE / 16) % GT == 0, "whole A loads per thread and plane");
    static_assert(PL == 1 || (PL == 2 && !TERN), "two A planes only with bf16 B");
    static_assert(TERN ? (B_SLOTS % kWave == 0 && B_WAVES <= GW) : B_SLOTS % GT == 0, "whole B loads per wave");
    static_assert(NS >= 2 && (NS - 2) * LOADS <= 63, "vmcnt range");
    static_assert(LDS <= 160 * 1024, "LDS");
};

// This wave's loads older than the newest N have landed and its LDS reads are
// done, then the workgroup barrier: one asm statement with a memory clobber,
// so the compiler neither moves LDS accesses across it nor adds a wait of its
// own for the loads still in flight.
template <int N>
__device__ __forceinline__ void stage_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Four bf16 values (-1, 0 or +1), two per dword, from the codes (0, 1, 2) in
// the four bytes of d: the codes select from a table of low bytes (80 00 80)
// and from one of high bytes (BF 00 3F) of the bf16 patterns of c - 1, and two
// permutes interleave the low and high bytes into bf16 pairs.
__device__ __forceinline__ void codes_to_bf16x4(uint32_t d, uint32_t& v01, uint32_t& v23) {
    const uint32_t lo = __builtin_amdgcn_perm(0u, 0x00800080u, d);
    const uint32_t hi = __builtin_amdgcn_perm(0u, 0x003F00BFu, d);
    v01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    v23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

template <class C>
__global__ __launch_bounds__(C::NT) void bwd_gemm_kernel(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ B, int R, int Cn, int J,
    const float* __restrict__ scale_ptr, float* __restrict__ out) {
    constexpr bool TERN = C::TERN;
    constexpr int WR = C::WR, WC = C::WC, NS = C::NS, KS = C::KS;
    __shared__ __align__(16) uint8_t lds[C::LDS];
    const int t = threadIdx.x, lane = t % kWave;
    const int wave_all = __builtin_amdgcn_readfirstlane(t / kWave);
    const int kg = wave_all / C::GW, wave = wave_all % C::GW;
    const int wr = wave / C::GC, wc = wave % C::GC;
    uint8_t* ring = lds + kg * C::RING;

    // Launch index -> tile: a contiguous range of tiles per XCD (workgroups go
    // round-robin over the XCDs), ordered in groups of GROUP row tiles with the
    // column index outermost, so the blocks running together on one XCD share
    // their A rows and B columns in its L2.
    const int tiles_r = (R + C::BR - 1) / C::BR, tiles_c = (Cn + C::BC - 1) / C::BC;
    const int total = tiles_r * tiles_c;
    const int per = total / kXcds, rem = total % kXcds;
    const int xcd = (int)blockIdx.x % kXcds, idx = (int)blockIdx.x / kXcds;
    const int tile = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
    const int first_r = tile / (C::GROUP * tiles_c) * C::GROUP;
    const int gsize = min(tiles_r - first_r, C::GROUP);
    const int in_group = tile % (C::GROUP * tiles_c);
    // (the divisions run on the vector unit: readfirstlane keeps the tile origin,
    // and so the buffer resources, in scalar registers)
    const int64_t r0 = (int64_t)__builtin_amdgcn_readfirstlane(first_r + in_group % gsize) * C::BR;
    const int64_t c0 = (int64_t)__builtin_amdgcn_readfirstlane(in_group / gsize) * C::BC;

    const float scale = scale_ptr != nullptr ? scale_ptr[0] : 1.0f;
    const int a_rows = (int)min((int64_t)C::BR, (int64_t)R - r0);
    const int b_rows = (int)min((int64_t)C::BC, (int64_t)Cn - c0);
    const int b_row_bytes = TERN ? J / 4 : J * 2;
    const int a_stride = C::PL * J;  // values per row of A
    const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + r0 * a_stride), (short)0, a_rows * a_stride * 2, (int)kBufferWord3);
    const __amdgpu_buffer_rsrc_t bres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(B + c0 * b_row_bytes), (short)0, b_rows * b_row_bytes, (int)kBufferWord3);
    const int nj = J / kBJ;                 // J is a multiple of kBJ
    const int steps = (nj + KS - 1) / KS;  // stages per group, the same for every group

    // Group kg's i-th stage is stage js = kg + KS i.  A (and B when bf16)
    // tiles: row r of 64 values = 8 granules of 16 bytes, granule g stored at
    // position g ^ (r & 7) so that the 32 rows a fragment read touches spread
    // over all banks.  Slot p of the tile is filled by a load of row p / 8,
    // granule (p % 8) ^ (row & 7).  Each lane's load offsets are fixed up front
    // (kFar for rows past the block's valid rows); a stage adds its column
    // offset, or kFar for a stage past the last, which then reads out of range
    // (zeros, no memory traffic) but is still issued, so every wave counts
    // LOADS loads per stage.  A buffer here spans at most 2^30 bytes, so
    // kFar, and kFar plus any offset, lies past its end.
    constexpr uint32_t kFar = 0x40000000u;
    constexpr int AL = C::A_SLOTS / C::GT, BL = TERN ? 1 : C::B_SLOTS / C::GT;
    uint32_t a_off[AL], b_off[BL];
#pragma unroll
    for (int u = 0; u < AL; ++u) {
        const int pa = u * C::GT + wave * kWave + lane;
        const int plane = pa / (C::A_PLANE / 16), p = pa % (C::A_PLANE / 16);
        const int r = p / 8, g = (p % 8) ^ (r & 7);
        a_off[u] = r < a_rows ? (uint32_t)((r * a_stride + plane * J + 8 * g) * 2) : kFar;
    }
    if constexpr (TERN) {
        const int c = wave * kWave + lane;  // row c: 16 bytes (64 codes) per stage, slot c
        b_off[0] = (wave < C::B_WAVES && c < b_rows) ? (uint32_t)(c * b_row_bytes) : kFar;
    } else {
#pragma unroll
        for (int u = 0; u < BL; ++u) {
            const int p = u * C::GT + wave * kWave + lane, r = p / 8, g = (p % 8) ^ (r & 7);
            b_off[u] = r < b_rows ? (uint32_t)((r * J + 8 * g) * 2) : kFar;
        }
    }
    auto load_stage = [&](int i, int slot) {
        const int js = kg + KS * i;
        const bool live = js < nj;
        const uint32_t a_add = live ? (uint32_t)(js * kBJ * 2) : kFar;
        const uint32_t b_add = live ? (uint32_t)(TERN ? js * kBJ / 4 : js * kBJ * 2) : kFar;
        uint8_t* st = ring + slot * C::STAGE;
#pragma unroll
        for (int u = 0; u < AL; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ares, (lds_void*)(st + (u * C::GT + wave * kWave) * 16), 16,
                                                     (int)(a_off[u] + a_add), 0, 0, 0);
        if constexpr (TERN) {
            uint8_t* dst = wave < C::B_WAVES ? st + C::A_BYTES + wave * kWave * 16 : lds + KS * C::RING;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(bres, (lds_void*)dst, 16, (int)(b_off[0] + b_add), 0, 0, 0);
        } else {
#pragma unroll
            for (int u = 0; u < BL; ++u)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    bres, (lds_void*)(st + C::A_BYTES + (u * C::GT + wave * kWave) * 16), 16,
                    (int)(b_off[u] + b_add), 0, 0, 0);
        }
    };

    v16f acc[WR][WC];
#pragma unroll
    for (int i = 0; i < WR; ++i)
#pragma unroll
        for (int j = 0; j < WC; ++j) acc[i][j] = v16f{};

    const int h = lane / 32, l32 = lane % 32;
    auto frag = [&](const uint8_t* tile, int row, int g) {
        return *reinterpret_cast<const v4u*>(tile + (row * 8 + (g ^ (row & 7))) * 16);
    };
    auto compute = [&](int slot) {
        const uint8_t* at = ring + slot * C::STAGE;
        const uint8_t* bt = at + C::A_BYTES;
        v4u bq[WC];
        if constexpr (TERN) {
#pragma unroll
            for (int cb = 0; cb < WC; ++cb)
                bq[cb] = *reinterpret_cast<const v4u*>(bt + (wc * (32 * WC) + cb * 32 + l32) * 16);
        }
#pragma unroll
        for (int s = 0; s < kBJ / 16; ++s) {
            v4u bf[WC];
#pragma unroll
            for (int cb = 0; cb < WC; ++cb) {
                if constexpr (TERN) {
                    const uint32_t w = bq[cb][s] >> (4 * h);
                    // values 8h .. 8h+3 of the step, then 8h+4 .. 8h+7
                    uint32_t v0, v1, v2, v3;
                    codes_to_bf16x4(w & 0x03030303u, v0, v1);
                    codes_to_bf16x4((w >> 2) & 0x03030303u, v2, v3);
                    bf[cb] = v4u{v0, v1, v2, v3};
                } else {
                    bf[cb] = frag(bt, wc * (32 * WC) + cb * 32 + l32, 2 * s + h);
                }
            }
#pragma unroll
            for (int pl = 0; pl < C::PL; ++pl)  // planes in turn: WR x WC MFMAs between dependent ones
#pragma unroll
                for (int rb = 0; rb < WR; ++rb) {
                    const int row = wr * (32 * WR) + rb * 32 + l32;
                    const v4u af = frag(at + pl * C::A_PLANE, row, 2 * s + h);
#pragma unroll
                    for (int cb = 0; cb < WC; ++cb)
                        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(v8bf, af), __builtin_bit_cast(v8bf, bf[cb]), acc[rb][cb], 0, 0, 0);
                }
        }
    };

    // Each group's ring of NS stages: NS - 1 in flight ahead of the one being
    // computed.  At step i the slot refilled is the one computed at step i - 1,
    // which the barrier has just released; step i uses slot i % NS.
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) load_stage(i, i);
    for (int i0 = 0; i0 < steps; i0 += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {  // slot u: fixed LDS addresses in the unrolled body
            if (i0 + u < steps) {
                stage_barrier<(NS - 2) * C::LOADS>();  // stage i0 + u landed for every wave
                load_stage(i0 + u + NS - 1, (u + NS - 1) % NS);
                if (kg + KS * (i0 + u) < nj) compute(u);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no transfer into LDS outlives the workgroup

    // K groups: group 0 adds the other groups' sums, group KS - 1 first.
    if constexpr (KS > 1) {
        float* part = reinterpret_cast<float*>(lds);
#pragma unroll 1
        for (int g = KS - 1; g >= 1; --g) {
            __syncthreads();  // every wave is done with the stage buffers (or the previous sums)
            if (kg == g) {
#pragma unroll
                for (int rb = 0; rb < WR; ++rb)
#pragma unroll
                    for (int cb = 0; cb < WC; ++cb)
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            part[((wave * WR * WC + rb * WC + cb) * 16 + e) * kWave + lane] = acc[rb][cb][e];
            }
            __syncthreads();
            if (kg == 0) {
#pragma unroll
                for (int rb = 0; rb < WR; ++rb)
#pragma unroll
                    for (int cb = 0; cb < WC; ++cb)
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            acc[rb][cb][e] += part[((wave * WR * WC + rb * WC + cb) * 16 + e) * kWave + lane];
            }
        }
        if (kg != 0) return;
    }

    // D[i][j] of a 32 x 32 block: lane j + 32 ((i / 4) % 2), element 4 (i / 8) + i % 4.
#pragma unroll
    for (int rb = 0; rb < WR; ++rb)
#pragma unroll
        for (int cb = 0; cb < WC; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = r0 + wr * (32 * WR) + rb * 32 + 8 * (e / 4) + 4 * h + e % 4;
                const int64_t col = c0 + wc * (32 * WC) + cb * 32 + l32;
                if (row < R && col < Cn) out[row * Cn + col] = acc[rb][cb][e] * scale;
            }
}

// ---------------------------------------------------------------------------
// Operands of dL/dW (Mp = M rounded up to 64; columns m >= M are zero):
// a[n] = [hi of p[.][n] | lo of p[.][n]], 2 Mp values, with
// p = grad_y[m][n] * d_x[m], and b[k] = codes[.][k] in bf16, Mp values.
// One 64 x 64 tile per workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void prep_grad_kernel(const uint16_t* __restrict__ g,
                                                             const float* __restrict__ d_x, int M,
                                                             int N, int Mp, uint16_t* __restrict__ a) {
    __shared__ float tile[64][65];  // [m][n]
    const int m0 = (int)blockIdx.x * 64, n0 = (int)blockIdx.y * 64;
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // 64 rows x 8 granules of 8 bf16
        const int p = t + kThreads * i, r = p / 8, gr = p % 8;
        const int m = m0 + r;
        uint4 v = make_uint4(0, 0, 0, 0);
        float s = 0.f;
        if (m < M) {
            v = *reinterpret_cast<const uint4*>(g + (int64_t)m * N + n0 + 8 * gr);
            s = d_x[m];
        }
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tile[r][8 * gr + 2 * e] = bf16_lo(w[e]) * s;
            tile[r][8 * gr + 2 * e + 1] = bf16_hi(w[e]) * s;
        }
    }
    __syncthreads();
    const int nr = t / 4, mc = (t % 4) * 16;  // output row n0 + nr, m = m0 + mc .. +15
    uint32_t hw[8], lw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float p0 = tile[mc + 2 * e][nr], p1 = tile[mc + 2 * e + 1][nr];
        const uint16_t h0 = bf16_rne(p0), h1 = bf16_rne(p1);
        const uint16_t l0 = bf16_rne(p0 - __uint_as_float((uint32_t)h0 << 16));
        const uint16_t l1 = bf16_rne(p1 - __uint_as_float((uint32_t)h1 << 16));
        hw[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lw[e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    uint4* ho = reinterpret_cast<uint4*>(a + (int64_t)(n0 + nr) * 2 * Mp + m0 + mc);
    uint4* lo4 = reinterpret_cast<uint4*>(a + (int64_t)(n0 + nr) * 2 * Mp + Mp + m0 + mc);
    ho[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    ho[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
    lo4[0] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    lo4[1] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
}

__global__ __launch_bounds__(kThreads) void prep_codes_kernel(const int8_t* __restrict__ xq, int M,
                                                              int K, int Mp, uint16_t* __restrict__ b) {
    __shared__ int tile[64][65];  // [m][k]
    const int m0 = (int)blockIdx.x * 64, k0 = (int)blockIdx.y * 64;
    const int t = threadIdx.x;
    {
        const int r = t / 4, gr = t % 4;  // 64 rows x 4 granules of 16 codes
        const int m = m0 + r;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (m < M) v = *reinterpret_cast<const uint4*>(xq + (int64_t)m * K + k0 + 16 * gr);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 16; ++e) tile[r][16 * gr + e] = (int)(int8_t)(w[e / 4] >> (8 * (e % 4)));
    }
    __syncthreads();
    const int kr = t / 4, mc = (t % 4) * 16;
    uint32_t o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {  // a code is exact in bf16: the top half of its float
        const uint32_t b0 = __float_as_uint((float)tile[mc + 2 * e][kr]) >> 16;
        const uint32_t b1 = __float_as_uint((float)tile[mc + 2 * e + 1][kr]) >> 16;
        o[e] = b0 | (b1 << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(b + (int64_t)(k0 + kr) * Mp + m0 + mc);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// ---------------------------------------------------------------------------
// RMSNorm backward, one workgroup per token: float64 sums of x^2 and of
// grad_n * x * gain, then grad_x = gain r grad_n - x r^3 dot / K in float32.
// r goes to the workspace for the gain gradient.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void rmsnorm_bwd_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ gain, float eps,
    const float* __restrict__ grad_n, int K, float* __restrict__ grad_x, double* __restrict__ r_out) {
    __shared__ double red[2][kThreads / kWave];
    const int64_t m = blockIdx.x;
    const int t = threadIdx.x, lane = t % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const uint16_t* xr = x + m * K;
    const float* gr = grad_n + m * K;
    double ss = 0.0, dot = 0.0;
    for (int k = t; k < K; k += kThreads) {
        const double xv = (double)__uint_as_float((uint32_t)xr[k] << 16);
        const double g = gain != nullptr ? (double)gain[k] : 1.0;
        ss = __fma_rn(xv, xv, ss);
        dot = __fma_rn((double)gr[k] * xv, g, dot);
    }
    ss = wave_sum_dpp(ss);
    dot = wave_sum_dpp(dot);
    if (lane == 0) {
        red[0][wave] = ss;
        red[1][wave] = dot;
    }
    __syncthreads();
    ss = 0.0;
    dot = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
        ss += red[0][w];
        dot += red[1][w];
    }
    const double r = 1.0 / sqrt(ss / (double)K + (double)eps);
    const double coef = r * r * r * dot / (double)K;
    for (int k = t; k < K; k += kThreads) {
        const double xv = (double)__uint_as_float((uint32_t)xr[k] << 16);
        const double g = gain != nullptr ? (double)gain[k] : 1.0;
        grad_x[m * K + k] = (float)(g * r * (double)gr[k] - xv * coef);
    }
    if (t == 0 && r_out != nullptr) r_out[m] = r;
}

// grad_gain[k] = sum_m grad_n[m][k] x[m][k] r[m]: partial sums over token
// chunks (float64), then the chunks in order.
constexpr int kGainChunk = 64;
__global__ __launch_bounds__(kThreads) void gain_partial_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ grad_n, const double* __restrict__ r,
    int M, int K, double* __restrict__ part) {
    const int k = (int)blockIdx.x * kThreads + threadIdx.x;
    const int mc = (int)blockIdx.y;
    if (k >= K) return;
    double s = 0.0;
    const int m1 = min(M, (mc + 1) * kGainChunk);
    for (int m = mc * kGainChunk; m < m1; ++m) {
        const double xv = (double)__uint_as_float((uint32_t)x[(int64_t)m * K + k] << 16);
        s = __fma_rn((double)grad_n[(int64_t)m * K + k] * xv, r[m], s);
    }
    part[(int64_t)mc * K + k] = s;
}

__global__ __launch_bounds__(kThreads) void gain_final_kernel(const double* __restrict__ part, int chunks,
                                                              int K, float* __restrict__ grad_gain) {
    const int k = (int)blockIdx.x * kThreads + threadIdx.x;
    if (k >= K) return;
    double s = 0.0;
    for (int c = 0; c < chunks; ++c) s += part[(int64_t)c * K + k];
    grad_gain[k] = (float)s;
}

__global__ __launch_bounds__(kThreads) void zero_kernel(float* __restrict__ p, int64_t count) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count; i += (int64_t)gridDim.x * kThreads)
        p[i] = 0.f;
}

// dL/dn: 256 x 128 tiles of 2 x 2 waves with 128 x 64 each, two K groups (8
// waves, one workgroup per CU); the grid is small (M/256 x K/128 tiles), so
// consecutive tiles on an XCD share their grad_y rows.
using CfgIn = BwdCfg<4, 2, 2, 2, 2, true, 2, 1>;
// dL/dW: 128 x 256 tiles of 2 x 4 waves with 64 x 64 each and the hi and lo
// planes of A in one stage (one workgroup per CU: bf16 B tiles leave no LDS
// for a second), groups of 8 row tiles.
using CfgW = BwdCfg<2, 2, 2, 4, 1, false, 2, 8, 2>;

template <class C>
dim3 bwd_grid(int64_t R, int64_t Cn) {
    return dim3((unsigned)(((R + C::BR - 1) / C::BR) * ((Cn + C::BC - 1) / C::BC)));
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

}  // namespace

hipError_t launch_zero_f32(float* p, int64_t count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((count + kThreads - 1) / kThreads, 4096);
    return launch_kernel(zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, count);
}

hipError_t launch_transpose_packed(const uint8_t* packed, int64_t N, int64_t K, uint8_t* packed_t,
                                   hipStream_t stream) {
    return launch_kernel(transpose_packed_kernel, dim3((unsigned)((K + kTK - 1) / kTK), (unsigned)(N / 64)),
                         dim3(kThreads),
                         0, stream, packed, (int)N, (int)K, packed_t);
}

hipError_t launch_backward_input(const uint16_t* grad_y, const uint8_t* packed_t, const float* w_scale,
                                 int64_t M, int64_t N, int64_t K, float* grad_n, hipStream_t stream) {
    // Row ranges of at most 2^20 tokens per launch keep the tile count and the
    // one-dimensional grid well inside 32 bits.
    constexpr int64_t kRowsPerLaunch = int64_t(1) << 20;
    static_assert(kRowsPerLaunch % CfgIn::BR == 0, "whole tiles per launch");
    for (int64_t m0 = 0; m0 < M; m0 += kRowsPerLaunch) {
        const int64_t rows = std::min(M - m0, kRowsPerLaunch);
        const hipError_t e = launch_kernel(bwd_gemm_kernel<CfgIn>, bwd_grid<CfgIn>(rows, K), dim3(CfgIn::NT), 0,
                                           stream, grad_y + m0 * N, packed_t, (int)rows, (int)K, (int)N, w_scale,
                                           grad_n + m0 * K);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

size_t backward_weight_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const int64_t Mp = round_up(M, 64);
    return (size_t)((2 * N + K) * Mp * 2);
}

hipError_t launch_backward_weight(const uint16_t* grad_y, const int8_t* xq, const float* x_scale,
                                  int64_t M, int64_t N, int64_t K, float* grad_w, void* workspace,
                                  hipStream_t stream) {
    const int64_t Mp = round_up(M, 64);
    uint16_t* a = static_cast<uint16_t*>(workspace);  // [N][2 Mp]: hi and lo planes
    uint16_t* b = a + N * 2 * Mp;                       // [K][Mp]
    hipError_t e = launch_kernel(prep_grad_kernel, dim3((unsigned)(Mp / 64), (unsigned)(N / 64)), dim3(kThreads),
                                 0, stream, grad_y, x_scale, (int)M, (int)N, (int)Mp, a);
    if (e != hipSuccess) return e;
    e = launch_kernel(prep_codes_kernel, dim3((unsigned)(Mp / 64), (unsigned)(K / 64)), dim3(kThreads), 0, stream,
                      xq, (int)M, (int)K, (int)Mp, b);
    if (e != hipSuccess) return e;
    return launch_kernel(bwd_gemm_kernel<CfgW>, bwd_grid<CfgW>(N, K), dim3(CfgW::NT), 0, stream, (const uint16_t*)a,
                         reinterpret_cast<const uint8_t*>(b), (int)N, (int)K, (int)Mp, (const float*)nullptr,
                         grad_w);
}

size_t rmsnorm_backward_workspace_bytes(int64_t M, int64_t K) {
    const int64_t chunks = (M + kGainChunk - 1) / kGainChunk;
    return (size_t)(round_up(M, 32) * 8 + chunks * K * 8);
}

hipError_t launch_rmsnorm_backward(const uint16_t* x, const float* gain, float eps, const float* grad_n,
                                   int64_t M, int64_t K, float* grad_x, float* grad_gain, void* workspace,
                                   hipStream_t stream) {
    double* r = static_cast<double*>(workspace);
    hipError_t e = launch_kernel(rmsnorm_bwd_kernel, dim3((unsigned)M), dim3(kThreads), 0, stream, x, gain, eps,
                                 grad_n, (int)K, grad_x, grad_gain != nullptr ? r : (double*)nullptr);
    if (e != hipSuccess || grad_gain == nullptr) return e;
    const int chunks = (int)((M + kGainChunk - 1) / kGainChunk);
    double* part = r + round_up(M, 32);
    const unsigned kb = (unsigned)((K + kThreads - 1) / kThreads);
    e = launch_kernel(gain_partial_kernel, dim3(kb, (unsigned)chunks), dim3(kThreads), 0, stream, x, grad_n,
                      (const double*)r, (int)M, (int)K, part);
    if (e != hipSuccess) return e;
    return launch_kernel(gain_final_kernel, dim3(kb), dim3(kThreads), 0, stream, (const double*)part, chunks,
                         (int)K, grad_gain);
}

}  // namespace bitnet
