// base3.hip - ternary weights packed five per byte (base 3), and the decode
// GEMV that reads them.
//
// A ternary weight carries log2 3 = 1.58 bits (primer on 1.58-bit
// quantisation, section "1.58비트는 어디서 나온거에요?"), and 3^5 = 243 <= 256,
// so five weights fit one byte: byte j of a row is the base-3 number
//   c_0 + 3 c_1 + 9 c_2 + 27 c_3 + 81 c_4,   c_i = q_{5j+i} + 1 in {0, 1, 2},
// 1.6 bits per weight against the 2 bits of the 2-bit layout.  Rows are padded
// with zero bytes to a multiple of 16 bytes; weights past K count as digit 0
// and meet activation codes that are zero, so they add nothing.
//
// GEMV for one token: a table in LDS turns a byte into its five digits
// (digits 0..3 as the bytes of one dword, digit 4 in the low byte of a second),
// one 8-byte read per byte.  The table index is the weight byte itself, so the
// 64 lanes of a read hit data-dependent entries; with one shared copy of the
// table those reads collided on the LDS banks (about 3.5 conflict cycles per
// read).  Here the table is held in 32 copies side by side, entry v of copy c
// at byte 256 v + 8 c, and lane l reads copy l % 32: a lane's reads stay on its
// own two banks whatever the byte, so a read is conflict free (lanes l and
// l + 32 share banks and are served in the instruction's two halves).  The
// read address is built from the weight byte and the lane's copy offset with
// one byte permute.  v_dot4 takes digits 0..3 of byte b against activation
// codes 5b .. 5b+3, and the fifth digits of four bytes, gathered into one dword
// by byte permutes, against codes 5b+4 of those bytes; each wave arranges the
// token's codes in that order once.  As in the 2-bit GEMV the digits are the offset codes q + 1,
// the token's code sum is subtracted at the end, a wave keeps a batch of rows
// in flight (two alternating register sets when it owns more rows than one
// batch), and the batch's row totals come from one transposing reduction.
#include "common.hpp"
#include "launch.hpp"
#include "xreduce.hpp"

namespace bitnet {
namespace {

constexpr int kB3Rows = 256;                     // table entries (bytes above 242 never occur in a packing)
constexpr int kB3Copies = 32;                    // table copies, one per lane pair
constexpr uint32_t kB3Word3 = 0x00020000u;       // raw buffer descriptor word 3 (gfx9 family)
constexpr uint32_t kB3OutOfRange = 0x80000000u;  // offset past every buffer here: loads 0
constexpr int kB3MaxRecords = 0x7fffffff;        // buffer size used for the weight batches

__device__ __forceinline__ uint4 b3_load16(__amdgpu_buffer_rsrc_t res, uint32_t off) {
    const v4i q = __builtin_amdgcn_raw_buffer_load_b128(res, off, 0, 0);
    return make_uint4((uint32_t)q[0], (uint32_t)q[1], (uint32_t)q[2], (uint32_t)q[3]);
}

// 2-bit packed [N][K/4] -> base-3 packed [N][row_bytes], one output byte per
// thread.  Weight k of a 2-bit row is field (k % 16) / 4 of byte 4 (k / 16) +
// k % 4, holding q + 1.
__global__ __launch_bounds__(256) void pack_base3_kernel(const uint8_t* __restrict__ packed, int64_t N, int K,
                                                         int row_bytes, uint8_t* __restrict__ packed3) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= N * row_bytes) return;
    const int64_t n = idx / row_bytes;
    const int j = (int)(idx % row_bytes);
    const uint8_t* row = packed + n * (K / 4);
    int v = 0, place = 1;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int k = 5 * j + i;
        if (k < K) v += ((row[4 * (k / 16) + k % 4] >> (2 * ((k % 16) / 4))) & 3) * place;
        place *= 3;
    }
    packed3[idx] = (uint8_t)v;
}

// Largest batch (rows in flight) for CH chunks per lane: in one register set,
// and in each of two alternating sets.  A chunk holds 20 code registers (16 in
// the 2-bit layout); these are the largest batches that do not spill at 512
// threads.
template <int CH>
constexpr int b3_max_batch() {
    return CH == 1 ? 16 : (CH == 2 ? 8 : (CH == 3 ? 4 : 1));
}
template <int CH>
constexpr int b3_multi_batch() {
    return CH == 1 ? 16 : (CH == 2 ? 4 : (CH == 3 ? 2 : 1));
}

// One token.  CH 16-byte chunks per lane cover a row (chunk c: weights
// 80c .. 80c + 79); wave g owns rows g, g + W, g + 2W, ..., RB at a time, with
// two alternating register sets (the next batch loaded while the current one
// is used) when MULTI.
template <int CH, int NT, int RB, bool MULTI>
__global__ __launch_bounds__(NT) void base3_gemv_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, const int32_t* __restrict__ x_qsum,
    const uint8_t* __restrict__ packed3, const float* __restrict__ w_scale, int N, int K, int row_bytes,
    float* __restrict__ y, int32_t* __restrict__ acc_out) {
    constexpr int NW = NT / kWave;
    constexpr int LV = log2_of(RB);
    static_assert(RB <= kWave && (RB & (RB - 1)) == 0, "rows per batch: a power of 2, <= 64");
    static_assert(NT % 16 == 0, "the table fill gives each thread a fixed 16-byte slot");
    __shared__ __align__(16) uint2 lut[kB3Rows * kB3Copies];   // 64 KiB

    const int t = threadIdx.x, lane = t % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int g = (int)blockIdx.x * NW + wave;
    const int W = (int)gridDim.x * NW;
    const int nchunk = row_bytes / 16;
    auto has_row = [&](int i) { return (int64_t)g + (int64_t)i * W < N; };

    // Weight loads of the batch of this wave's rows i0 .. i0 + RB - 1 (zeros
    // past the last row and past the row's chunks).
    auto load = [&](uint4 (&w)[RB][CH], int i0) {
        const int64_t r0 = has_row(i0) ? (int64_t)g + (int64_t)i0 * W : 0;
        const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(packed3 + r0 * row_bytes), (short)0, kB3MaxRecords, (int)kB3Word3);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int c = lane + kWave * j;
                const uint32_t off = (has_row(i0 + rb) && c < nchunk) ? (uint32_t)(rb * W * row_bytes + 16 * c)
                                                                       : kB3OutOfRange;
                w[rb][j] = b3_load16(res, off);
            }
    };

    // 1. The token's codes of my chunks, then the first weight batch(es), all
    // in flight while the table is built.
    uint32_t raw[CH][20];
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)xq, (short)0, K, (int)kB3Word3);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = lane + kWave * j;
#pragma unroll
        for (int v = 0; v < 5; ++v) {
            const uint4 q = b3_load16(xres, c < nchunk ? (uint32_t)(80 * c + 16 * v) : kB3OutOfRange);
            raw[j][4 * v] = q.x, raw[j][4 * v + 1] = q.y, raw[j][4 * v + 2] = q.z, raw[j][4 * v + 3] = q.w;
        }
    }
    uint4 w0[RB][CH], w1[RB][CH];
    load(w0, 0);
    if constexpr (MULTI) load(w1, RB);

    // 2. The table: entry v = (digits 0..3 of v as bytes, digit 4).  Thread t
    // works out the digits of v = t % 256 and writes 16 / H of the row's 16
    // slots (two copies per 16-byte store; H = NT / 256 threads per row),
    // starting at a slot rotated by v so that a wave's stores spread over the
    // banks.  Plain arithmetic: a load from a constant table would queue behind
    // the weight loads above and hold the table back until they land.
    {
        constexpr int H = NT / kB3Rows;
        static_assert(NT % kB3Rows == 0, "whole threads per table row");
        const int v = t % kB3Rows, h = t / kB3Rows;
        uint32_t d = (uint32_t)v, lo = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo |= (d % 3u) << (8 * i);
            d /= 3u;
        }
        const uint4 entry = make_uint4(lo, d % 3u, lo, d % 3u);
#pragma unroll
        for (int i = 0; i < 16 / H; ++i) {
            const int slot = (h * (16 / H) + i + v) % 16;
            *reinterpret_cast<uint4*>(&lut[v * kB3Copies + 2 * slot]) = entry;
        }
    }

    // 3. Codes in digit order: xa[j][b] = codes 5b .. 5b+3 of chunk j, x4[j][k]
    // = codes 20k+4, 20k+9, 20k+14, 20k+19 (the fifth digits' codes of bytes
    // 4k .. 4k+3), which sit in byte 0, 1, 2, 3 of the raw dwords 5k+1 .. 5k+4.
    uint32_t xa[CH][16], x4[CH][4];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const int p = 5 * b;
            xa[j][b] = p % 4 == 0 ? raw[j][p / 4]
                                  : __builtin_amdgcn_alignbyte(raw[j][p / 4 + 1], raw[j][p / 4], p % 4);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            x4[j][k] = (raw[j][5 * k + 1] & 0x000000ffu) | (raw[j][5 * k + 2] & 0x0000ff00u) |
                       (raw[j][5 * k + 3] & 0x00ff0000u) | (raw[j][5 * k + 4] & 0xff000000u);
    }
    __syncthreads();  // the table is complete
    if (g >= N) return;  // after the only barrier: wave-uniform exit
    const int32_t qs = x_qsum[0];
    const float sx = x_scale[0], dw = w_scale[0];
    const uint32_t copy_off = 8u * (uint32_t)(lane % kB3Copies);
    const char* lut_bytes = reinterpret_cast<const char*>(lut);

    // Table entries of the 16 bytes of a weight chunk.  Address 256 * byte +
    // 8 * copy: byte i of word k goes to bits 8..15 next to the copy offset.
    auto reads = [&](const uint4& wc, uint2 (&e)[16]) {
        const uint32_t ws[4] = {wc.x, wc.y, wc.z, wc.w};
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const uint32_t addr = __builtin_amdgcn_perm(ws[b / 4], copy_off, 0x0c0c0000u | ((4u + b % 4) << 8));
            e[b] = *reinterpret_cast<const uint2*>(lut_bytes + addr);
        }
    };

    // 4. Contraction and epilogue, one batch at a time.  Up to three chunks per
    // lane, each group of four table reads is followed by its dot products
    // and the compiler overlaps the groups.  With four chunks (K above 15360)
    // the chunks (row rb, chunk j) are taken in order u = rb * CH + j and the 16
    // reads of chunk u + 1 are issued before the dot products of chunk u,
    // held there by scheduling barriers: measured faster at K 16384 (43.1
    // against 46.3 us for a 174.7 MB matrix) and slower at the smaller shapes.
    auto dots = [&](const uint2 (&e)[16], int j, int s) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int i = 0; i < 4; ++i) s = __builtin_amdgcn_sdot4((int)e[4 * k + i].x, (int)xa[j][4 * k + i], s, false);
            const uint32_t d = __builtin_amdgcn_perm(__builtin_amdgcn_perm(e[4 * k + 3].y, e[4 * k + 2].y, 0x0c0c0400u),
                                                     __builtin_amdgcn_perm(e[4 * k + 1].y, e[4 * k].y, 0x0c0c0400u),
                                                     0x05040100u);
            s = __builtin_amdgcn_sdot4((int)d, (int)x4[j][k], s, false);
        }
        return s;
    };
    auto batch = [&](const uint4 (&w)[RB][CH], int i0) {
        int p[RB];
        if constexpr (CH < 4) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                int s = 0;
                if (has_row(i0 + rb)) {  // wave-uniform
#pragma unroll
                    for (int j = 0; j < CH; ++j) {
                        const uint32_t ws[4] = {w[rb][j].x, w[rb][j].y, w[rb][j].z, w[rb][j].w};
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            uint32_t d4[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const uint32_t addr =
                                    __builtin_amdgcn_perm(ws[k], copy_off, 0x0c0c0000u | ((4u + i) << 8));
                                const uint2 e = *reinterpret_cast<const uint2*>(lut_bytes + addr);
                                s = __builtin_amdgcn_sdot4((int)e.x, (int)xa[j][4 * k + i], s, false);
                                d4[i] = e.y;
                            }
                            const uint32_t d = __builtin_amdgcn_perm(__builtin_amdgcn_perm(d4[3], d4[2], 0x0c0c0400u),
                                                                     __builtin_amdgcn_perm(d4[1], d4[0], 0x0c0c0400u),
                                                                     0x05040100u);
                            s = __builtin_amdgcn_sdot4((int)d, (int)x4[j][k], s, false);
                        }
                    }
                }
                p[rb] = s;
            }
        } else {
            uint2 e[2][16];
            if (has_row(i0)) reads(w[0][0], e[0]);
#pragma unroll
            for (int u = 0; u < RB * CH; ++u) {
                const int rb = u / CH, j = u % CH;
                if (j == 0) p[rb] = 0;
                if (u + 1 < RB * CH && has_row(i0 + (u + 1) / CH))
                    reads(w[(u + 1) / CH][(u + 1) % CH], e[(u + 1) % 2]);
                __builtin_amdgcn_sched_barrier(0);
                if (has_row(i0 + rb)) p[rb] = dots(e[u % 2], j, p[rb]);  // wave-uniform
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        xreduce<RB>(p, lane);
        const int rb = lane >> (6 - LV);
        if ((lane & ((kWave >> LV) - 1)) == 0 && has_row(i0 + rb)) {
            const int64_t r = (int64_t)g + (int64_t)(i0 + rb) * W;
            const int a = p[0] - qs;
            y[r] = ((float)a * sx) * dw;
            if (acc_out != nullptr) acc_out[r] = a;
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

template <int CH, int NT, int RB, bool MULTI>
hipError_t launch_b3_shape(const int8_t* xq, const float* x_scale, const int32_t* x_qsum, const uint8_t* packed3,
                           const float* w_scale, int64_t N, int64_t K, int row_bytes, int64_t waves, float* y,
                           int32_t* acc, hipStream_t stream) {
    constexpr int NW = NT / kWave;
    const int64_t blocks = (waves + NW - 1) / NW;
    return launch_kernel(base3_gemv_kernel<CH, NT, RB, MULTI>, dim3((unsigned)blocks), dim3(NT), 0, stream, xq,
                         x_scale, x_qsum, packed3, w_scale, (int)N, (int)K, row_bytes, y, acc);
}

// Launch shape as the 2-bit GEMV's: about 1024 waves of 256-thread workgroups
// for matrices up to 4096 x 4096, else 2048 waves of 512-thread workgroups
// (one workgroup per CU either way; the 64 KiB table allows two); RB the
// smallest power of two that holds a wave's rows, else two register sets of
// the largest batch.
template <int CH, int NT>
hipError_t launch_b3_rb(const int8_t* xq, const float* x_scale, const int32_t* x_qsum, const uint8_t* packed3,
                        const float* w_scale, int64_t N, int64_t K, int row_bytes, int64_t rpw, float* y,
                        int32_t* acc, hipStream_t stream) {
    constexpr int CAP = b3_max_batch<CH>();
    const int64_t waves = (N + rpw - 1) / rpw;
#define BITNET_B3_RB(R)                                                                                      \
    if constexpr (CAP >= R)                                                                                  \
        if (rpw <= R)                                                                                        \
            return launch_b3_shape<CH, NT, R, false>(xq, x_scale, x_qsum, packed3, w_scale, N, K, row_bytes, \
                                                     waves, y, acc, stream);
    BITNET_B3_RB(1)
    BITNET_B3_RB(2)
    BITNET_B3_RB(4)
    BITNET_B3_RB(8)
    BITNET_B3_RB(16)
#undef BITNET_B3_RB
    return launch_b3_shape<CH, NT, b3_multi_batch<CH>(), true>(xq, x_scale, x_qsum, packed3, w_scale, N, K,
                                                               row_bytes, waves, y, acc, stream);
}

template <int CH>
hipError_t launch_b3(const int8_t* xq, const float* x_scale, const int32_t* x_qsum, const uint8_t* packed3,
                     const float* w_scale, int64_t N, int64_t K, int row_bytes, float* y, int32_t* acc,
                     hipStream_t stream) {
    if (N > 4096 || K > 4096)
        return launch_b3_rb<CH, 512>(xq, x_scale, x_qsum, packed3, w_scale, N, K, row_bytes, (N + 2047) / 2048,
                                     y, acc, stream);
    return launch_b3_rb<CH, 256>(xq, x_scale, x_qsum, packed3, w_scale, N, K, row_bytes, (N + 1023) / 1024, y,
                                 acc, stream);
}

}  // namespace

int64_t base3_row_bytes(int64_t K) { return ((K + 4) / 5 + 15) / 16 * 16; }

bool base3_gemv_supported(int64_t K) { return (base3_row_bytes(K) / 16 + kWave - 1) / kWave <= kBase3MaxChunks; }

hipError_t launch_pack_base3(const uint8_t* packed, int64_t N, int64_t K, uint8_t* packed3, hipStream_t stream) {
    const int64_t rb = base3_row_bytes(K);
    const int64_t total = N * rb;
    if (total == 0) return hipSuccess;
    return launch_kernel(pack_base3_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, packed, N,
                         (int)K, (int)rb, packed3);
}

hipError_t launch_base3_gemv(const int8_t* xq, const float* x_scale, const int32_t* x_qsum, const uint8_t* packed3,
                             const float* w_scale, int64_t N, int64_t K, float* y, int32_t* acc,
                             hipStream_t stream) {
    if (N == 0) return hipSuccess;
    const int rb = (int)base3_row_bytes(K);
    const int ch = (rb / 16 + kWave - 1) / kWave;
    switch (ch) {
        case 1: return launch_b3<1>(xq, x_scale, x_qsum, packed3, w_scale, N, K, rb, y, acc, stream);
        case 2: return launch_b3<2>(xq, x_scale, x_qsum, packed3, w_scale, N, K, rb, y, acc, stream);
        case 3: return launch_b3<3>(xq, x_scale, x_qsum, packed3, w_scale, N, K, rb, y, acc, stream);
        case 4: return launch_b3<4>(xq, x_scale, x_qsum, packed3, w_scale, N, K, rb, y, acc, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bitnet
