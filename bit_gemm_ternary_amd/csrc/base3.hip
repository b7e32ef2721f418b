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
// GEMV for one token: a 256-entry table in LDS turns a byte into its five
// digits (digits 0..3 as the bytes of one dword, digit 4 in a second), so a
// lane decodes its 16 bytes (80 weights) with 16 table reads.  v_dot4 takes
// digits 0..3 of byte b against activation codes 5b .. 5b+3, and the fifth
// digits of four bytes, gathered into one dword, against codes 5b+4 of those
// bytes; each wave arranges the token's codes in that order once, so the rows
// need no reshuffling.  As in the 2-bit GEMV the digits are the offset codes
// q + 1, and the token's code sum is subtracted at the end.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

constexpr int kB3Threads = 256;
// One row in flight per wave over up to 8192 waves: measured 3-5% faster than
// two rows over 4096 waves and 12-16% faster than four over 2048 on the 4096-
// and 11008-wide decode shapes and on a 218 MB matrix; eight rows per wave
// were slower still.
constexpr int kB3Batch = 1;                      // rows in flight per wave
constexpr int kB3MaxWaves = 8192;
constexpr uint32_t kB3Word3 = 0x00020000u;       // raw buffer descriptor word 3 (gfx9 family)
constexpr uint32_t kB3OutOfRange = 0x80000000u;  // offset past every buffer here: loads 0

__device__ __forceinline__ uint4 b3_load16(__amdgpu_buffer_rsrc_t res, uint32_t off) {
    const v4i q = __builtin_amdgcn_raw_buffer_load_b128(res, off, 0, 0);
    return make_uint4((uint32_t)q[0], (uint32_t)q[1], (uint32_t)q[2], (uint32_t)q[3]);
}

__device__ __forceinline__ uint32_t byte_of(const uint32_t (&w)[20], int p) {
    return (w[p / 4] >> (8 * (p % 4))) & 0xffu;
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

// One token.  CH 16-byte chunks per lane cover a row (chunk c: weights
// 80c .. 80c + 79); wave g owns rows g, g + W, g + 2W, ..., kB3Batch at a time.
template <int CH>
__global__ __launch_bounds__(kB3Threads) void base3_gemv_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, const int32_t* __restrict__ x_qsum,
    const uint8_t* __restrict__ packed3, const float* __restrict__ w_scale, int N, int K, int row_bytes,
    float* __restrict__ y, int32_t* __restrict__ acc_out) {
    __shared__ uint2 lut[256];
    const int t = threadIdx.x, lane = t % kWave;
    {
        // digits of byte t (bytes above 242 never occur in a packing)
        uint32_t v = (uint32_t)t, lo = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo |= (v % 3u) << (8 * i);
            v /= 3u;
        }
        lut[t] = make_uint2(lo, v % 3u);
    }
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int g = (int)blockIdx.x * (kB3Threads / kWave) + wave;
    const int W = (int)gridDim.x * (kB3Threads / kWave);
    const int nchunk = row_bytes / 16;

    // The token's codes of my chunks, in the order the digits come out: xa[j][b]
    // = codes 5b .. 5b+3 of chunk j, xb[j][k] = codes 20k+4, 20k+9, 20k+14, 20k+19.
    uint32_t xa[CH][16], xb[CH][4];
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)xq, (short)0, K, (int)kB3Word3);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = lane + kWave * j;
        uint32_t raw[20];
#pragma unroll
        for (int v = 0; v < 5; ++v) {
            const uint4 q = b3_load16(xres, c < nchunk ? (uint32_t)(80 * c + 16 * v) : kB3OutOfRange);
            raw[4 * v] = q.x, raw[4 * v + 1] = q.y, raw[4 * v + 2] = q.z, raw[4 * v + 3] = q.w;
        }
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const int p = 5 * b;
            xa[j][b] = p % 4 == 0 ? raw[p / 4] : __builtin_amdgcn_alignbyte(raw[p / 4 + 1], raw[p / 4], p % 4);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            xb[j][k] = byte_of(raw, 20 * k + 4) | (byte_of(raw, 20 * k + 9) << 8) |
                       (byte_of(raw, 20 * k + 14) << 16) | (byte_of(raw, 20 * k + 19) << 24);
    }
    __syncthreads();  // the table is complete
    if (g >= N) return;
    const int32_t qs = x_qsum[0];
    const float sx = x_scale[0], dw = w_scale[0];

    for (int64_t r0 = g; r0 < N; r0 += (int64_t)kB3Batch * W) {  // r0 + stride may pass 2^31 - 1
        uint4 w[kB3Batch][CH];
#pragma unroll
        for (int rb = 0; rb < kB3Batch; ++rb) {
            const int64_t r = (int64_t)r0 + (int64_t)rb * W;
            const bool live = r < N;
            const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(packed3 + (live ? r : 0) * row_bytes), (short)0, live ? row_bytes : 0, (int)kB3Word3);
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int c = lane + kWave * j;
                w[rb][j] = b3_load16(res, c < nchunk ? (uint32_t)(16 * c) : kB3OutOfRange);
            }
        }
#pragma unroll
        for (int rb = 0; rb < kB3Batch; ++rb) {
            const int64_t r = (int64_t)r0 + (int64_t)rb * W;
            if (r >= N) break;  // wave-uniform
            int s = 0;
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const uint32_t ws[4] = {w[rb][j].x, w[rb][j].y, w[rb][j].z, w[rb][j].w};
                uint32_t fifth[16];
#pragma unroll
                for (int b = 0; b < 16; ++b) {
                    const uint2 e = lut[(ws[b / 4] >> (8 * (b % 4))) & 0xffu];
                    s = __builtin_amdgcn_sdot4((int)e.x, (int)xa[j][b], s, false);
                    fifth[b] = e.y;
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t f = fifth[4 * k] | (fifth[4 * k + 1] << 8) | (fifth[4 * k + 2] << 16) |
                                       (fifth[4 * k + 3] << 24);
                    s = __builtin_amdgcn_sdot4((int)f, (int)xb[j][k], s, false);
                }
            }
            s = wave_sum_dpp(s);
            if (lane == 0) {
                const int a = s - qs;
                y[r] = ((float)a * sx) * dw;
                if (acc_out != nullptr) acc_out[r] = a;
            }
        }
    }
}

template <int CH>
hipError_t launch_b3(const int8_t* xq, const float* x_scale, const int32_t* x_qsum, const uint8_t* packed3,
                     const float* w_scale, int64_t N, int64_t K, int row_bytes, float* y, int32_t* acc,
                     hipStream_t stream) {
    const int64_t waves = std::min<int64_t>((N + kB3Batch - 1) / kB3Batch, kB3MaxWaves);
    const int64_t blocks = (waves + kB3Threads / kWave - 1) / (kB3Threads / kWave);
    return launch_kernel(base3_gemv_kernel<CH>, dim3((unsigned)blocks), dim3(kB3Threads), 0, stream, xq, x_scale,
                         x_qsum, packed3, w_scale, (int)N, (int)K, row_bytes, y, acc);
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
