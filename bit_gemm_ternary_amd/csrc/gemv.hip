// gemv.hip - bandwidth-bound decode contraction for M <= 4 tokens, standalone
// (int8 codes in) and fused with the activation quantisation (bf16 in).
//
// The ternary matmul needs only integer additions (Hugging Face 1.58-bit
// write-up, section 계산 패러다임), and at decode the packed weights are the only
// large stream, so the kernel is bound by HBM bandwidth on those bytes: each
// weight is read once, 2 bits per weight, with 128-bit loads, and unpacked in
// registers (section 추론 최적화 및 커스텀 커널: weights unpacked on the fly
// inside the matmul).
//
// Mapping: wave g of the W waves in the grid owns the weight rows g, g + W,
// g + 2W, ...  (interleaved, so the waves of the whole chip stream one
// contiguous stretch of the matrix at a time).  A wave's rows are processed in
// batches of RB rows whose loads are all in flight together: one batch when the
// wave owns at most RB rows, else two register sets that alternate (the loads of
// the next batch are issued before the current one is used).  Lane l owns the
// 16-byte chunks l, l + 64, ... of every row (64 weights per chunk), so one load
// instruction reads 1 KiB of a row, fully coalesced; the matching activation
// codes stay in registers for all rows.
//
// Unpack: a packed word holds weights 16g..16g+15; with the field of weight
// 16g+4i+b at bits 8b+2i, (word & (3 << 2i) per byte) gives the four codes
// (q+1) of weights 16g+4i..16g+4i+3 times 4^i, in byte order, which
// v_dot4_i32_i8 multiplies with the activation dword 4g+i.  Slots i = 0, 1, 2
// need only the mask (codes times 1, 4, 16 fit a signed byte); slot 3 is shifted
// down first.  Slots 0 and 3 share an accumulator; the three sums are combined
// exactly as s03 + s1/4 + s2/16.  The offset code q + 1 is corrected at the end:
// sum q x = sum (q+1) x - sum x.
//
// Row totals: after a batch every lane holds one partial sum per (row, token),
// NV = RB * MT values.  A transposing butterfly over the lane-index bits
// (v_permlane32_swap, v_permlane16_swap, then DPP moves inside 16-lane rows)
// halves the number of values per lane at each step while adding pairs, so all
// NV totals cost about 2 NV + 12 lane operations rather than NV separate wave
// reductions; lane L then holds the total of value L >> (6 - log2 NV).
//
// Loads use buffer resources: an out-of-range offset returns zeros, so the tail
// rows and chunks need no branches and the compiler counts the loads of a batch
// exactly when it waits for the first of them.  The wave index is made
// wave-uniform explicitly, so the row bookkeeping lives in scalar registers.
//
// Fused variant: each workgroup first quantises the (<= 4) tokens itself
// (RMSNorm + absmax int8, the arithmetic of quant_act.hip) from the bf16 input,
// which every workgroup reads from L2, and shares the codes through LDS.  The
// activation (and gain) loads are issued first, then the first rows of each
// wave's batch, and the rest of the batch once the token is reduced, so the
// weight stream is in flight through that prologue without the token queueing
// behind the whole batch.  The prologue is straight-line code between its two
// barriers (vectors past K are zeros): the float64 scale d_x and the code sums
// are formed alongside the codes, so after the second barrier a wave only
// reads its codes and starts on rows.
//
// One token, fused, N < 16384 with ceil(N / 1024) rows per wave in one register
// set (the 7B / 8B decode projections): decode1_kernel below, the same
// arithmetic laid out for one 256-thread workgroup per CU with exact rows per
// wave, every weight load issued before the token's arithmetic.
#include "common.hpp"
#include "launch.hpp"
#include "xreduce.hpp"

namespace bitnet {
namespace {

constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer descriptor word 3 (gfx9 family)
constexpr uint32_t kOutOfRange = 0x80000000u;   // offset past every buffer used here: loads 0
constexpr int kMaxRecords = 0x7fffffff;         // buffer size used for the weight batches
constexpr int kMaxXRegsChunks = 8;
// Where decode_kernel's codes come from: int8 codes in memory, the fused
// quantisation of bf16 tokens, or packed 4-bit codes in memory.
constexpr int kInt8Codes = 0, kFused = 1, kNibbleCodes = 2;              // MT * CH limit: 16 * MT * CH code VGPRs

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}
// Signed 4-bit dot product of eight nibble lanes, accumulated (v_dot8_i32_i4).
__device__ __forceinline__ int dot8(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}
__device__ __forceinline__ int dot4_first(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, 0, true);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t res, uint32_t off) {
    const v4i q = __builtin_amdgcn_raw_buffer_load_b128(res, off, 0, 0);
    return make_uint4((uint32_t)q[0], (uint32_t)q[1], (uint32_t)q[2], (uint32_t)q[3]);
}


// The fused kernels' codes in LDS, piece-major: the 16-byte piece q (codes
// 16q .. 16q + 15) of chunk c sits at q * kPlane + 16 c.  A lane reading piece
// q of its own chunk then meets its 15 neighbours on 15 other 16-byte bank
// groups (chunk-major rows, 64 bytes apart, put four lanes on each group: the
// reads were 4-way bank conflicts), and with the plane stride a multiple of
// 256 bytes plus 64 the 8-byte code writes of consecutive vectors (one
// thread's 8 codes) land on distinct banks as well.
template <int CH>
struct CodeLds {
    static constexpr int kPlane = CH * 1024 + 64;
    static constexpr int kBytes = 4 * kPlane;
    // Byte address of the codes 8v .. 8v + 7.
    __device__ static __forceinline__ int of_vector(int v) {
        return ((v >> 1) & 3) * kPlane + 16 * (v >> 3) + 8 * (v & 1);
    }
    // Byte address of piece q of chunk c.
    __device__ static __forceinline__ int of_piece(int c, int q) { return q * kPlane + 16 * c; }
};

// Largest batch (rows in flight per register set) for CH chunks per lane.
template <int CH>
constexpr int max_batch() {
    return CH == 1 ? 16 : (CH == 2 ? 8 : (CH <= 4 ? 4 : 2));
}

struct Args {
    const uint16_t* x;       // fused: bf16 tokens [MT][K]
    const float* gain;       // fused: [K] or NULL
    float eps;
    const int8_t* xq;        // standalone: codes [MT][K]
    const uint8_t* xq4;      // standalone, nibbles: codes [MT][K/2]
    const float* x_scale;    // standalone: d_x [MT]
    const int32_t* x_qsum;   // standalone: sum of codes [MT]
    const uint8_t* packed;   // [N][K/4]
    RowScales scales;
    int N, K;
    float* y;                // [MT][N]
    int8_t* xq_out;          // fused: codes, scales and sums written by workgroup 0
    float* x_scale_out;
    int32_t* x_qsum_out;
    int32_t* acc;            // [MT][N] or NULL
};

// MT tokens, CH 16-byte chunks per lane per row (K <= CH * 4096), NT threads,
// RB rows per batch, MULTI: more than RB rows per wave.
template <int MT, int CH, int NT, int RB, bool MULTI, int MODE>
__global__ __launch_bounds__(NT) void decode_kernel(const Args a) {
    constexpr bool FUSED = MODE == kFused;
    constexpr bool I4 = MODE == kNibbleCodes;
    constexpr int XD = I4 ? 8 : 16;                // code dwords per chunk per token
    constexpr int NW = NT / kWave;
    constexpr int MTP = MT == 3 ? 4 : MT;  // tokens per row in the reduction (a power of 2)
    constexpr int NV = MTP * RB;
    constexpr int LV = log2_of(NV);
    constexpr int XV = (CH * 512 + NT - 1) / NT;  // 8-value bf16 vectors per thread per token
    static_assert(NV <= kWave && (NV & (NV - 1)) == 0, "values per batch: a power of 2, <= 64");
    static_assert(XV * NT == CH * 512, "the fused prologue's vectors tile the code array exactly");
    __shared__ __align__(16) int8_t codes[MT][FUSED ? CodeLds<CH>::kBytes : 16];
    __shared__ float red_f[MT][NW];
    __shared__ double red_d[MT][NW];
    __shared__ int red_i[MT][NW];

    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int g = (int)blockIdx.x * NW + wave;
    const int W = (int)gridDim.x * NW;
    const int N = a.N, K = a.K;
    const int nchunk = K / 64;
    const int row_bytes = K / 4;
    // Row i of this wave is g + i W; it exists while that is below N.
    auto has_row = [&](int i) { return (int64_t)g + (int64_t)i * W < N; };
    const float dw0 = a.scales.w_scale[0];              // before any store (see RowScales::of)

    // Weight loads of rows i0 + rb0 .. i0 + rb1 - 1 of this wave's batch
    // starting at row i0 (zeros past the last row).
    auto load_rows = [&](uint4 (&w)[RB][CH], int i0, int rb0, int rb1) {
        const int64_t r0 = has_row(i0) ? (int64_t)g + (int64_t)i0 * W : 0;
        const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.packed + r0 * row_bytes), (short)0, kMaxRecords, (int)kBufferWord3);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (rb < rb0 || rb >= rb1) continue;   // compile-time after unrolling
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int c = lane + kWave * j;
                const uint32_t off = (has_row(i0 + rb) && c < nchunk)
                                         ? (uint32_t)(rb * W * row_bytes + 16 * c)
                                         : kOutOfRange;
                w[rb][j] = load16(res, off);
            }
        }
    };
    auto load = [&](uint4 (&w)[RB][CH], int i0) { load_rows(w, i0, 0, RB); };
    // Fused single batch: rows issued before the token is reduced.  The rest
    // follow once it is, so a wave's own token does not queue behind its
    // whole batch (measured: up to 13% per launch on the 7B / 8B shapes).
    constexpr int kEarlyRows = RB >= 4 ? 2 : 1;
    // Two register sets with 6 or more chunks per lane: the second set is
    // issued once the token's bf16 values are dead, so the prologue does not
    // hold both sets, the token and the codes at once.
    constexpr bool kLateSecondSet = MT * CH >= 6;

    uint32_t xv[MT][CH][XD];  // codes of my chunks: chunk c covers x[64c .. 64c+63]
    int tok_sum[MT];
    float tok_scale[MT];
    uint4 w0[RB][CH], w1[RB][CH];

    if constexpr (FUSED) {
        const double inv_k = inv_count(K);
        // 1. Activation (and gain) loads, then the first weight batch, which
        // stays in flight through the prologue.
        const int nvec = K / 8;
        const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
            (void*)a.x, (short)0, MT * K * 2, (int)kBufferWord3);
        uint4 raw[MT][XV];
#pragma unroll
        for (int tok = 0; tok < MT; ++tok)
#pragma unroll
            for (int i = 0; i < XV; ++i) {
                const int v = t + NT * i;
                raw[tok][i] = load16(xres, v < nvec ? (uint32_t)(tok * K * 2 + 16 * v) : kOutOfRange);
            }
        float gv[XV][8];
        const bool has_gain = a.gain != nullptr;
        if (has_gain) {
            const __amdgpu_buffer_rsrc_t gres = __builtin_amdgcn_make_buffer_rsrc(
                (void*)a.gain, (short)0, K * 4, (int)kBufferWord3);
#pragma unroll
            for (int i = 0; i < XV; ++i) {
                const int v = t + NT * i;
                const uint4 g0 = load16(gres, v < nvec ? (uint32_t)(32 * v) : kOutOfRange);
                const uint4 g1 = load16(gres, v < nvec ? (uint32_t)(32 * v + 16) : kOutOfRange);
                gv[i][0] = __uint_as_float(g0.x); gv[i][1] = __uint_as_float(g0.y);
                gv[i][2] = __uint_as_float(g0.z); gv[i][3] = __uint_as_float(g0.w);
                gv[i][4] = __uint_as_float(g1.x); gv[i][5] = __uint_as_float(g1.y);
                gv[i][6] = __uint_as_float(g1.z); gv[i][7] = __uint_as_float(g1.w);
            }
        }
        if constexpr (MULTI) {
            load(w0, 0);
            if constexpr (!kLateSecondSet) load(w1, RB);
        } else {
            load_rows(w0, 0, 0, kEarlyRows);
        }

        auto values = [&](int tok, int i, float (&u)[8], bool with_gain) {
            const uint32_t ws[4] = {raw[tok][i].x, raw[tok][i].y, raw[tok][i].z, raw[tok][i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u[2 * e] = bf16_lo(ws[e]);
                u[2 * e + 1] = bf16_hi(ws[e]);
            }
            if (with_gain && has_gain) {
#pragma unroll
                for (int e = 0; e < 8; ++e) u[e] *= gv[i][e];
            }
        };

        // 2. Per-token absmax of x*gain and sum of x^2 (four independent f64
        // chains per thread): one workgroup reduction.  Vectors past K were
        // loaded as zeros and leave both unchanged, so no guard is needed.
#pragma unroll
        for (int tok = 0; tok < MT; ++tok) {
            float amax = 0.f;
            double ss[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int i = 0; i < XV; ++i) {
                float u[8];
                values(tok, i, u, false);
#pragma unroll
                for (int e = 0; e < 8; ++e) ss[e % 4] = __fma_rn((double)u[e], (double)u[e], ss[e % 4]);
                values(tok, i, u, true);
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(u[e]));
            }
            amax = wave_max_dpp(amax);
            const double s = wave_sum_dpp((ss[0] + ss[1]) + (ss[2] + ss[3]));
            if (lane == 0) {
                red_f[tok][wave] = amax;
                red_d[tok][wave] = s;
            }
        }
        if constexpr (!MULTI) load_rows(w0, 0, kEarlyRows, RB);
        __syncthreads();

        // 3. Codes into LDS.  For |v| <= 127.00002, v + 1.5 * 2^23 rounds v to
        // an integer (ties to even, the rint of the definition) and leaves it,
        // two's complement, in the low byte of the float's bit pattern.  The
        // clamp to [-128, 127] never acts: |x * gain| <= amax, so
        // |x * gain * rn(127 / amax)| < 127.5.
        // The per-token factor d_x = amax * rstd / 127 is computed here too, by
        // every wave, in the same straight-line code as the codes, so its
        // latency overlaps the code work instead of following the second
        // barrier.  Vectors past K give zero codes, written to the LDS slots
        // of chunks past K (the array has room for the XV * NT * 8 = CH * 4096
        // codes of every vector) and never read.  Each thread also sums its
        // codes; the wave totals go to LDS with the codes.
#pragma unroll
        for (int tok = 0; tok < MT; ++tok) {
            float amax = red_f[tok][0];
#pragma unroll
            for (int wv = 1; wv < NW; ++wv) amax = fmaxf(amax, red_f[tok][wv]);
            double ss = red_d[tok][0];
#pragma unroll
            for (int wv = 1; wv < NW; ++wv) ss += red_d[tok][wv];
            tok_scale[tok] = token_scale(amax, ss, inv_k, a.eps, 1.0 / 127.0);
            const float scale = amax < kTinyAbsmax ? 0.f : 127.0f / amax;
            int part = 0;
#pragma unroll
            for (int i = 0; i < XV; ++i) {
                const int v = t + NT * i;
                float u[8];
                values(tok, i, u, true);
                uint32_t b[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    b[e] = __float_as_uint(__fadd_rn(__fmul_rn(u[e], scale), 12582912.0f));
                const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                                                          __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u),
                                                          0x05040100u);
                const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u),
                                                          __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u),
                                                          0x05040100u);
                *reinterpret_cast<uint2*>(&codes[tok][CodeLds<CH>::of_vector(v)]) = make_uint2(lo, hi);
                part = dot4(lo, 0x01010101u, part);
                part = dot4(hi, 0x01010101u, part);
            }
            part = wave_sum_dpp(part);
            if (lane == 0) red_i[tok][wave] = part;
        }
        if constexpr (MULTI && kLateSecondSet) load(w1, RB);  // the bf16 token registers are free now
        __syncthreads();

        // 4. Codes of my chunks into registers (chunks past K read as zeros);
        // the token's code sum from the wave totals.
#pragma unroll
        for (int tok = 0; tok < MT; ++tok) {
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int c = lane + kWave * j;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (c < nchunk) v = *reinterpret_cast<const uint4*>(&codes[tok][CodeLds<CH>::of_piece(c, q)]);
                    xv[tok][j][4 * q] = v.x;
                    xv[tok][j][4 * q + 1] = v.y;
                    xv[tok][j][4 * q + 2] = v.z;
                    xv[tok][j][4 * q + 3] = v.w;
                }
            }
            int sum = red_i[tok][0];
#pragma unroll
            for (int wv = 1; wv < NW; ++wv) sum += red_i[tok][wv];
            tok_sum[tok] = sum;
        }
        if (blockIdx.x == 0) {
            for (int tok = 0; tok < MT; ++tok)
                for (int v = t; v < K / 16; v += NT)
                    reinterpret_cast<uint4*>(a.xq_out + (int64_t)tok * K)[v] =
                        *reinterpret_cast<const uint4*>(&codes[tok][CodeLds<CH>::of_piece(v >> 2, v & 3)]);
            if (t == 0) {
#pragma unroll
                for (int tok = 0; tok < MT; ++tok) {
                    a.x_scale_out[tok] = tok_scale[tok];
                    a.x_qsum_out[tok] = tok_sum[tok];
                }
            }
        }
    } else if constexpr (I4) {
        // Nibble codes of my chunks (32 bytes per chunk) from memory, ahead of
        // the weights: dwords 2d and 2d + 1 of a chunk hold the 16-code group d.
        const __amdgpu_buffer_rsrc_t qres = __builtin_amdgcn_make_buffer_rsrc(
            (void*)a.xq4, (short)0, MT * (K / 2), (int)kBufferWord3);
#pragma unroll
        for (int tok = 0; tok < MT; ++tok)
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int c = lane + kWave * j;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint4 v = load16(qres, c < nchunk ? (uint32_t)(tok * (K / 2) + 32 * c + 16 * q)
                                                            : kOutOfRange);
                    xv[tok][j][4 * q] = v.x;
                    xv[tok][j][4 * q + 1] = v.y;
                    xv[tok][j][4 * q + 2] = v.z;
                    xv[tok][j][4 * q + 3] = v.w;
                }
            }
#pragma unroll
        for (int tok = 0; tok < MT; ++tok) {
            tok_sum[tok] = a.x_qsum[tok];
            tok_scale[tok] = a.x_scale[tok];
        }
        load(w0, 0);
        if constexpr (MULTI) load(w1, RB);
    } else {
        // Codes of my chunks straight from memory, ahead of the weights.
        const __amdgpu_buffer_rsrc_t qres = __builtin_amdgcn_make_buffer_rsrc(
            (void*)a.xq, (short)0, MT * K, (int)kBufferWord3);
#pragma unroll
        for (int tok = 0; tok < MT; ++tok)
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int c = lane + kWave * j;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 v = load16(qres, c < nchunk ? (uint32_t)(tok * K + 64 * c + 16 * q) : kOutOfRange);
                    xv[tok][j][4 * q] = v.x;
                    xv[tok][j][4 * q + 1] = v.y;
                    xv[tok][j][4 * q + 2] = v.z;
                    xv[tok][j][4 * q + 3] = v.w;
                }
            }
#pragma unroll
        for (int tok = 0; tok < MT; ++tok) {
            tok_sum[tok] = a.x_qsum[tok];
            tok_scale[tok] = a.x_scale[tok];
        }
        load(w0, 0);
        if constexpr (MULTI) load(w1, RB);
    }
    if (g >= N) return;  // after the last barrier: wave-uniform exit

    // 5. Contraction and epilogue, one batch at a time.
    auto batch = [&](const uint4 (&w)[RB][CH], int i0) {
        int p[NV];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int tok = 0; tok < MTP; ++tok) p[rb * MTP + tok] = 0;
            if (has_row(i0 + rb)) {  // wave-uniform
#pragma unroll
                for (int tok = 0; tok < MT; ++tok) {
                    if constexpr (I4) {
                        // Fields of slots 0 and 2 (w & 0x33333333) and of slots 1
                        // and 3 ((w >> 2) & 0x33333333) are 4-bit lanes holding
                        // q + 1 for the weights 16g + j, 16g + 8 + j and
                        // 16g + 4 + j, 16g + 12 + j: the nibble order of the
                        // group's two code dwords.
                        int s = 0;
#pragma unroll
                        for (int j = 0; j < CH; ++j) {
                            const uint32_t ws[4] = {w[rb][j].x, w[rb][j].y, w[rb][j].z, w[rb][j].w};
#pragma unroll
                            for (int d = 0; d < 4; ++d) {
                                s = dot8(ws[d] & 0x33333333u, xv[tok][j][2 * d], s);
                                s = dot8((ws[d] >> 2) & 0x33333333u, xv[tok][j][2 * d + 1], s);
                            }
                        }
                        p[rb * MTP + tok] = s;
                    } else {
                        int s03 = 0, s1 = 0, s2 = 0;
#pragma unroll
                        for (int j = 0; j < CH; ++j) {
                            const uint32_t ws[4] = {w[rb][j].x, w[rb][j].y, w[rb][j].z, w[rb][j].w};
#pragma unroll
                            for (int d = 0; d < 4; ++d) {
                                const uint32_t word = ws[d];
                                s03 = dot4(word & 0x03030303u, xv[tok][j][4 * d + 0], s03);
                                s1 = dot4(word & 0x0C0C0C0Cu, xv[tok][j][4 * d + 1], s1);
                                s2 = dot4(word & 0x30303030u, xv[tok][j][4 * d + 2], s2);
                                s03 = dot4((word >> 6) & 0x03030303u, xv[tok][j][4 * d + 3], s03);
                            }
                        }
                        p[rb * MTP + tok] = s03 + (s1 >> 2) + (s2 >> 4);
                    }
                }
            }
        }
        xreduce<NV>(p, lane);
        const int idx = lane >> (6 - LV);
        const int rb = idx / MTP, tok = idx % MTP;
        if ((lane & ((kWave >> LV) - 1)) == 0 && has_row(i0 + rb) && tok < MT) {
            const int64_t r = (int64_t)g + (int64_t)(i0 + rb) * W;
            int qs = tok_sum[0];
            float ts = tok_scale[0];
#pragma unroll
            for (int k = 1; k < MT; ++k) {  // selects: register arrays take no runtime index
                qs = tok == k ? tok_sum[k] : qs;
                ts = tok == k ? tok_scale[k] : ts;
            }
            const int acc = p[0] - qs;
            if (a.acc != nullptr) a.acc[(int64_t)tok * N + r] = acc;
            a.y[(int64_t)tok * N + r] = ((float)acc * ts) * a.scales.of(r, dw0);
        }
    };
    if constexpr (!MULTI) {
        batch(w0, 0);
    } else {
        for (int i0 = 0; has_row(i0); i0 += 2 * RB) {
            batch(w0, i0);
            if (has_row(i0 + 2 * RB)) load(w0, i0 + 2 * RB);
            if (has_row(i0 + RB)) {
                batch(w1, i0 + RB);
                if (has_row(i0 + 3 * RB)) load(w1, i0 + 3 * RB);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// One token, fused: the decode fast path for matrices whose rows spread over
// 1024 waves fit one register set per wave.  One 256-thread workgroup per CU
// (one wave per SIMD); wave g owns exactly the RB rows g, g + W, ..., so there
// is no per-row branch (rows past N load zeros and store nothing).  Order of
// work in a wave:
//   1. the token's loads (and the gain's), then every weight load of the
//      wave's rows at once;
//   2. absmax over the workgroup (an integer maximum of the bf16 magnitude
//      bits when there is no gain), one barrier;
//   3. this thread's share of the codes into LDS, with its code sum and its
//      part of sum x^2 (exact float32 squares in four float32 chains,
//      combined in float64), one barrier;
//   4. the wave's code registers from LDS and the token's d_x, the dot
//      products of each row as its loads land, one transposing reduction over
//      the rows, the stores.
// The arithmetic of every step is that of decode_kernel above.
// ---------------------------------------------------------------------------
template <int CH, int RB, bool GAIN>
__global__ __launch_bounds__(256) void decode1_kernel(const Args a) {
    constexpr int NT = 256;
    constexpr int NW = NT / kWave;
    constexpr int NV = RB <= 1 ? 1 : (RB <= 2 ? 2 : (RB <= 4 ? 4 : (RB <= 8 ? 8 : 16)));
    constexpr int LV = log2_of(NV);
    constexpr int XV = CH * 512 / NT;   // 8-value vectors of the token per thread
    static_assert(RB <= 16 && RB * CH <= 16, "one register set of rows");
    __shared__ __align__(16) int8_t codes[CodeLds<CH>::kBytes];
    __shared__ float red_f[NW];
    __shared__ double red_d[NW];
    __shared__ int red_i[NW];

    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int g = (int)blockIdx.x * NW + wave;
    const int W = (int)gridDim.x * NW;
    const int N = a.N, K = a.K;
    const int nchunk = K / 64;
    const int row_bytes = K / 4;
    const int nvec = K / 8;

    // Arguments used only at the end are read with the first ones: a scalar
    // load issued later would be waited for with the LDS traffic.
    float* const y_out = a.y;
    int32_t* const acc_out = a.acc;
    const int groups = a.scales.groups;
    const float eps = a.eps;
    asm volatile("" ::"s"(y_out), "s"(acc_out), "s"(groups), "s"(eps));

    // 1. Token (and gain), then all weight loads.
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, K * 2,
                                                                         (int)kBufferWord3);
    uint4 raw[XV];
#pragma unroll
    for (int i = 0; i < XV; ++i) {
        const int v = t + NT * i;
        raw[i] = load16(xres, v < nvec ? (uint32_t)(16 * v) : kOutOfRange);
    }
    // d_w by a vector load issued with the token's: a scalar load here would
    // be waited for at the first barrier (the LDS and scalar-memory counters
    // are one), a full memory latency on the critical path.
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc((void*)a.scales.w_scale, (short)0, 4,
                                                                         (int)kBufferWord3);
    const float dw0 = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(sres, 0, 0, 0));
    float gv[GAIN ? XV : 1][8];
    if constexpr (GAIN) {
        const __amdgpu_buffer_rsrc_t gres = __builtin_amdgcn_make_buffer_rsrc((void*)a.gain, (short)0, K * 4,
                                                                             (int)kBufferWord3);
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int v = t + NT * i;
            const uint4 g0 = load16(gres, v < nvec ? (uint32_t)(32 * v) : kOutOfRange);
            const uint4 g1 = load16(gres, v < nvec ? (uint32_t)(32 * v + 16) : kOutOfRange);
            gv[i][0] = __uint_as_float(g0.x); gv[i][1] = __uint_as_float(g0.y);
            gv[i][2] = __uint_as_float(g0.z); gv[i][3] = __uint_as_float(g0.w);
            gv[i][4] = __uint_as_float(g1.x); gv[i][5] = __uint_as_float(g1.y);
            gv[i][6] = __uint_as_float(g1.z); gv[i][7] = __uint_as_float(g1.w);
        }
    }
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.packed + (int64_t)(g < N ? g : 0) * row_bytes), (short)0, kMaxRecords, (int)kBufferWord3);
    uint4 w[RB][CH];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = lane + kWave * j;
            const bool ok = (int64_t)g + (int64_t)rb * W < N && c < nchunk;
            w[rb][j] = load16(wres, ok ? (uint32_t)(rb * W * row_bytes + 16 * c) : kOutOfRange);
        }
    // The weight loads stay ahead of the token's arithmetic (the scheduler
    // would otherwise sink them below the wait for the token).
    __builtin_amdgcn_sched_barrier(0);

    auto values = [&](int i, float (&u)[8], bool with_gain) {
        const uint32_t ws[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[2 * e] = bf16_lo(ws[e]);
            u[2 * e + 1] = bf16_hi(ws[e]);
        }
        if constexpr (GAIN) {
            if (with_gain) {
#pragma unroll
                for (int e = 0; e < 8; ++e) u[e] *= gv[i][e];
            }
        }
    };

    // 2. absmax of x * gain over the workgroup.
    float amax = 0.f;
    if constexpr (!GAIN) {
        typedef unsigned short us2 __attribute__((ext_vector_type(2)));
        us2 m2 = {0, 0};
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const uint32_t ws[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t mag = ws[e] & 0x7fff7fffu;
                us2 v;
                __builtin_memcpy(&v, &mag, 4);
                m2 = __builtin_elementwise_max(m2, v);
            }
        }
        amax = __uint_as_float((uint32_t)(m2.x > m2.y ? m2.x : m2.y) << 16);
    } else {
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            float u[8];
            values(i, u, true);
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(u[e]));
        }
    }
    amax = wave_max_dpp(amax);
    if (lane == 0) red_f[wave] = amax;
    __syncthreads();
    amax = red_f[0];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) amax = fmaxf(amax, red_f[wv]);

    // 3. Codes (the rounding of decode_kernel step 3), code sum, sum of x^2.
    const float scale = amax < kTinyAbsmax ? 0.f : 127.0f / amax;
    int part = 0;
#pragma unroll
    for (int i = 0; i < XV; ++i) {
        const int v = t + NT * i;
        float u[8];
        values(i, u, true);
        uint32_t b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = __float_as_uint(__fadd_rn(__fmul_rn(u[e], scale), 12582912.0f));
        const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                                                  __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u), 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u),
                                                  __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u), 0x05040100u);
        *reinterpret_cast<uint2*>(&codes[CodeLds<CH>::of_vector(v)]) = make_uint2(lo, hi);
        part = dot4(lo, 0x01010101u, part);
        part = dot4(hi, 0x01010101u, part);
    }
    float sf[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < XV; ++i) {
        float u[8];
        values(i, u, false);
#pragma unroll
        for (int e = 0; e < 8; ++e) sf[e % 4] = __fmaf_rn(u[e], u[e], sf[e % 4]);
    }
    part = wave_sum_dpp(part);
    const double ssw = wave_sum_dpp(((double)sf[0] + (double)sf[1]) + ((double)sf[2] + (double)sf[3]));
    if (lane == 0) {
        red_i[wave] = part;
        red_d[wave] = ssw;
    }
    __syncthreads();

    // 4. Code registers, token scale and sum; the rows.  Every chunk slot of
    // the LDS array holds codes (step 3 writes all XV * NT vectors, zeros past
    // K) and the weights of chunks past K load as zeros, so the code reads
    // need no bounds test (a masked read costs a branch and register clears
    // right where the rows start).
    uint32_t xv[CH][16];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = lane + kWave * j;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = *reinterpret_cast<const uint4*>(&codes[CodeLds<CH>::of_piece(c, q)]);
            xv[j][4 * q] = v.x;
            xv[j][4 * q + 1] = v.y;
            xv[j][4 * q + 2] = v.z;
            xv[j][4 * q + 3] = v.w;
        }
    }
    int tok_sum = red_i[0];
    double ss = red_d[0];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) {
        tok_sum += red_i[wv];
        ss += red_d[wv];
    }
    // d_x (a float64 chain with a quarter-rate reciprocal square root) is
    // formed before the rows, while their loads are still landing: after them
    // it would lengthen the work left once the last weights arrive.
    const float tok_scale = token_scale(amax, ss, inv_count(K), eps, 1.0 / 127.0);
    if (blockIdx.x == 0) {
        for (int v = t; v < K / 16; v += NT)
            reinterpret_cast<uint4*>(a.xq_out)[v] =
                *reinterpret_cast<const uint4*>(&codes[CodeLds<CH>::of_piece(v >> 2, v & 3)]);
        if (t == 0) {
            a.x_scale_out[0] = tok_scale;
            a.x_qsum_out[0] = tok_sum;
        }
    }
    if (g >= N) return;  // after the last barrier: wave-uniform exit

    int p[NV];
#pragma unroll
    for (int r = 0; r < NV; ++r) p[r] = 0;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int s03 = 0, s1 = 0, s2 = 0;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const uint32_t ws[4] = {w[rb][j].x, w[rb][j].y, w[rb][j].z, w[rb][j].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t word = ws[d];
                if (j == 0 && d == 0) {
                    s03 = dot4_first(word & 0x03030303u, xv[0][0]);
                    s1 = dot4_first(word & 0x0C0C0C0Cu, xv[0][1]);
                    s2 = dot4_first(word & 0x30303030u, xv[0][2]);
                } else {
                    s03 = dot4(word & 0x03030303u, xv[j][4 * d + 0], s03);
                    s1 = dot4(word & 0x0C0C0C0Cu, xv[j][4 * d + 1], s1);
                    s2 = dot4(word & 0x30303030u, xv[j][4 * d + 2], s2);
                }
                s03 = dot4((word >> 6) & 0x03030303u, xv[j][4 * d + 3], s03);
            }
        }
        p[rb] = s03 + (s1 >> 2) + (s2 >> 4);
    }
    xreduce<NV>(p, lane);
    const int idx = lane >> (6 - LV);
    if ((lane & ((kWave >> LV) - 1)) == 0 && idx < RB) {
        const int64_t r = (int64_t)g + (int64_t)idx * W;
        if (r < N) {
            const int acc = p[0] - tok_sum;
            if (acc_out != nullptr) acc_out[r] = acc;
            y_out[r] = ((float)acc * tok_scale) * (groups == 1 ? dw0 : a.scales.of(r, dw0));
        }
    }
}

// ---------------------------------------------------------------------------
// Launch shape.  A wave's rows stay in registers, so the grid decides how much
// of the matrix is in flight: about 1024 waves of 256-thread workgroups, or
// 2048 waves of 512-thread workgroups for one token and matrices larger than
// 4096 x 4096 (one workgroup per CU either way, since every workgroup repeats
// the quantisation; the larger workgroup splits that work over more threads).
// Measured on the decode projections of a 7B model.  Oversized batches (loads
// and butterfly steps for absent rows) cost more than they save, so RB is the
// smallest power of two that holds a wave's rows.
// ---------------------------------------------------------------------------
int chunks_per_lane(int64_t K) { return (int)((K / 64 + kWave - 1) / kWave); }

// The chunk counts instantiated: 1, 2, 3, 4, 6, 8 (larger counts are not supported).
int rounded_ch(int ch) { return ch <= 4 ? ch : (ch <= 6 ? 6 : (ch <= 8 ? 8 : ch)); }

template <int MT, int CH, int NT, int RB, bool MULTI, int MODE>
hipError_t launch_shape(const Args& a, int64_t waves, hipStream_t stream) {
    constexpr int NW = NT / kWave;
    const int64_t blocks = (waves + NW - 1) / NW;
    return launch_kernel((decode_kernel<MT, CH, NT, RB, MULTI, MODE>), dim3((unsigned)blocks),
                         dim3(NT), 0, stream, a);
}

// Pick RB (and MULTI) for a wave owning up to rpw rows.
template <int MT, int CH, int NT, int MODE>
hipError_t launch_rb(const Args& a, int64_t rpw, int64_t waves, hipStream_t stream) {
    constexpr int CAP = max_batch<CH>();
    constexpr int MTP = MT == 3 ? 4 : MT;
    constexpr int CAP_MT = MTP * CAP <= kWave ? CAP : kWave / MTP;
    if (rpw <= 2 && CAP_MT >= 2) return launch_shape<MT, CH, NT, 2, false, MODE>(a, waves, stream);
    if constexpr (CAP_MT >= 4)
        if (rpw <= 4) return launch_shape<MT, CH, NT, 4, false, MODE>(a, waves, stream);
    if constexpr (CAP_MT >= 8)
        if (rpw <= 8) return launch_shape<MT, CH, NT, 8, false, MODE>(a, waves, stream);
    if constexpr (CAP_MT >= 16)
        if (rpw <= 16) return launch_shape<MT, CH, NT, 16, false, MODE>(a, waves, stream);
    // Two alternating register sets: with 6 or more chunks per lane, two sets
    // of two rows next to the codes exceed the register file (the compiler
    // spilled 129 registers at 8 chunks), so each set holds one row.
    constexpr int MRB = MT * CH >= 6 ? 1 : CAP_MT;
    return launch_shape<MT, CH, NT, MRB, true, MODE>(a, waves, stream);
}

template <int MT, int CH, int MODE>
hipError_t launch_ch(const Args& a, hipStream_t stream) {
    const int64_t N = a.N;
    // 512-thread workgroups (2048 waves) for single tokens and matrices larger
    // than 4096 x 4096: they halve each thread's share of the quantisation.
    if constexpr (MT == 1) {
        // Two such workgroups per CU (4096 waves) for N >= 16384 when K <= 8192
        // and a wave's rows fit one register set: those variants need at most
        // ~128 registers, so both workgroups fit, and the second hides the
        // first's prologue and reduction latency (measured: 8192 -> 28672
        // 16.8 -> 13.8 us, 4096 -> 28672 8.9 -> 8.3 us; no gain below
        // N = 16384).
        if (CH <= 2 && N >= 16384 && N <= 4096 * max_batch<CH>()) {
            const int64_t rpw = (N + 4095) / 4096;
            return launch_rb<MT, CH, 512, MODE>(a, rpw, (N + rpw - 1) / rpw, stream);
        }
        if (N >= 4096 && (N > 4096 || a.K > 4096)) {
            const int64_t rpw = (N + 2047) / 2048;
            return launch_rb<MT, CH, 512, MODE>(a, rpw, (N + rpw - 1) / rpw, stream);
        }
    }
    const int64_t rpw = (N + 1023) / 1024;
    return launch_rb<MT, CH, 256, MODE>(a, rpw, (N + rpw - 1) / rpw, stream);
}

template <int MT, int MODE>
hipError_t dispatch_ch(int ch, const Args& a, hipStream_t stream) {
#define BITNET_GEMV_CH(C)                                                          \
    if (ch <= C) {                                                                 \
        if constexpr (MT * C <= kMaxXRegsChunks) return launch_ch<MT, C, MODE>(a, stream); \
        return hipErrorInvalidValue;                                               \
    }
    BITNET_GEMV_CH(1)
    BITNET_GEMV_CH(2)
    BITNET_GEMV_CH(3)
    BITNET_GEMV_CH(4)
    BITNET_GEMV_CH(6)
    BITNET_GEMV_CH(8)
#undef BITNET_GEMV_CH
    return hipErrorInvalidValue;
}

template <int MODE>
hipError_t dispatch(int64_t M, const Args& a, hipStream_t stream) {
    const int ch = chunks_per_lane(a.K);
    switch (M) {
        case 1: return dispatch_ch<1, MODE>(ch, a, stream);
        case 2: return dispatch_ch<2, MODE>(ch, a, stream);
        case 3: return dispatch_ch<3, MODE>(ch, a, stream);
        case 4: return dispatch_ch<4, MODE>(ch, a, stream);
        default: return hipErrorInvalidValue;
    }
}

// The one-token fused kernel for N < 16384 rows when ceil(N / 1024) rows per
// wave fit one register set; hipErrorNotSupported otherwise (the caller falls
// back to decode_kernel).  RB = ceil(N / 1024) rows per wave over ceil(N / RB)
// waves: one workgroup per CU, or a few CUs idle.
template <int CH, int RB>
hipError_t launch_decode1_rb(const Args& a, hipStream_t stream) {
    const int64_t waves = (a.N + RB - 1) / RB;
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (a.gain != nullptr) return launch_kernel((decode1_kernel<CH, RB, true>), grid, dim3(256), 0, stream, a);
    return launch_kernel((decode1_kernel<CH, RB, false>), grid, dim3(256), 0, stream, a);
}

template <int CH>
hipError_t launch_decode1_ch(const Args& a, hipStream_t stream) {
    const int64_t rpw = (a.N + 1023) / 1024;
    if (a.N >= 16384 || rpw > 16 / CH) return hipErrorNotSupported;
#define BITNET_DECODE1_RB(R) \
    if constexpr (R * CH <= 16) \
        if (rpw == R) return launch_decode1_rb<CH, R>(a, stream);
    BITNET_DECODE1_RB(1) BITNET_DECODE1_RB(2) BITNET_DECODE1_RB(3) BITNET_DECODE1_RB(4)
    BITNET_DECODE1_RB(5) BITNET_DECODE1_RB(6) BITNET_DECODE1_RB(7) BITNET_DECODE1_RB(8)
    BITNET_DECODE1_RB(9) BITNET_DECODE1_RB(10) BITNET_DECODE1_RB(11) BITNET_DECODE1_RB(12)
    BITNET_DECODE1_RB(13) BITNET_DECODE1_RB(14) BITNET_DECODE1_RB(15) BITNET_DECODE1_RB(16)
#undef BITNET_DECODE1_RB
    return hipErrorNotSupported;
}

hipError_t dispatch_decode1(const Args& a, hipStream_t stream) {
    switch (chunks_per_lane(a.K)) {
        case 1: return launch_decode1_ch<1>(a, stream);
        case 2: return launch_decode1_ch<2>(a, stream);
        case 3: return launch_decode1_ch<3>(a, stream);
        case 4: return launch_decode1_ch<4>(a, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

bool gemv_supported(int64_t M, int64_t K) {
    if (M < 1 || M > 4) return false;
    return M * rounded_ch(chunks_per_lane(K)) <= kMaxXRegsChunks;
}

hipError_t launch_gemv(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                       const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                       int64_t K, float* y, int32_t* acc, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    Args a{};
    a.xq = xq, a.x_scale = x_scale, a.x_qsum = x_qsum, a.packed = packed, a.scales = scales;
    a.N = (int)N, a.K = (int)K, a.y = y, a.acc = acc;
    return dispatch<kInt8Codes>(M, a, stream);
}

hipError_t launch_gemv_i4(const uint8_t* xq4, const float* x_scale, const int32_t* x_qsum,
                          const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                          int64_t K, float* y, int32_t* acc, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    Args a{};
    a.xq4 = xq4, a.x_scale = x_scale, a.x_qsum = x_qsum, a.packed = packed, a.scales = scales;
    a.N = (int)N, a.K = (int)K, a.y = y, a.acc = acc;
    return dispatch<kNibbleCodes>(M, a, stream);
}

hipError_t launch_fused_decode(const uint16_t* x, const float* gain, float eps,
                               const uint8_t* packed, const RowScales& scales, int64_t M,
                               int64_t N, int64_t K, float* y, int8_t* xq, float* x_scale,
                               int32_t* x_qsum, int32_t* acc, hipStream_t stream) {
    Args a{};
    a.x = x, a.gain = gain, a.eps = eps, a.packed = packed, a.scales = scales;
    a.N = (int)N, a.K = (int)K, a.y = y, a.xq_out = xq, a.x_scale_out = x_scale;
    a.x_qsum_out = x_qsum, a.acc = acc;
    if (M == 1 && N >= 1) {
        const hipError_t e = dispatch_decode1(a, stream);
        if (e != hipErrorNotSupported) return e;
    }
    return dispatch<kFused>(M, a, stream);
}

}  // namespace bitnet
