// gemv.hip - bandwidth-bound decode contraction for M <= 4 tokens.
//
// The ternary matmul needs only integer additions (Hugging Face 1.58-bit
// write-up, section 계산 패러다임), and at decode the packed weights are the only
// large stream, so the kernel is bound by HBM bandwidth on those bytes: each
// weight is read once, 2 bits per weight, with 128-bit loads, and unpacked in
// registers (section 추론 최적화 및 커스텀 커널: weights unpacked on the fly
// inside the matmul).
//
// Mapping: one wavefront owns a run of consecutive output rows.  Lane l owns
// the 16-byte packed chunks l, l+64, ... of every row (64 weights per chunk), so
// a wave reads 1 KiB of a row per load instruction, fully coalesced.  The
// matching 64 activation bytes per chunk stay in registers for all rows.
//
// Unpack: a packed word holds weights 16g..16g+15; with the field of weight
// 16g+4i+b at bits 8b+2i, (word & (3 << 2i) per byte) gives the four codes
// (q+1) of weights 16g+4i..16g+4i+3 times 4^i, in byte order, which
// v_dot4_i32_i8 multiplies with the activation dword 4g+i.  Slots i = 0, 1, 2
// need only the mask (codes times 1, 4, 16 fit a signed byte); slot 3 is shifted
// down first.  The four slot sums are combined exactly as s0 + s1/4 + s2/16 + s3.
// The offset code q + 1 is corrected at the end: sum q x = sum (q+1) x - sum x.
#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

constexpr int kGemvThreads = 256;
constexpr int kGemvRowBatch = 4;  // rows whose loads are in flight together

// Sum of v over the 64 lanes, returned wave-uniform.  Four DPP steps give every
// lane the sum of its 16-lane row; the four row sums are read out to scalars.
__device__ __forceinline__ int wave_sum_dpp(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// MT tokens, CH chunks per lane per row (K <= CH * 4096).
template <int MT, int CH>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ x_qsum, const uint8_t* __restrict__ packed,
    const float* __restrict__ w_scale, int N, int K, int rows_per_wave, float* __restrict__ y,
    int32_t* __restrict__ acc_out) {
    const int lane = threadIdx.x % kWave;
    const int wave = (int)((blockIdx.x * (int64_t)kGemvThreads + threadIdx.x) / kWave);
    const int64_t row0 = (int64_t)wave * rows_per_wave;
    if (row0 >= N) return;  // wave-uniform; no workgroup barrier in this kernel
    const int64_t row1 = min((int64_t)N, row0 + rows_per_wave);
    const int nchunk = K / 64;
    const int64_t row_bytes = K / 4;

    // Activation bytes of my chunks: chunk c covers x[64c .. 64c+63].
    uint32_t xv[MT][CH][16];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = lane + kWave * j;
            const uint4* p = reinterpret_cast<const uint4*>(xq + (int64_t)t * K + 64 * (int64_t)c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint4 a = make_uint4(0, 0, 0, 0);
                if (c < nchunk) a = p[q];
                xv[t][j][4 * q] = a.x;
                xv[t][j][4 * q + 1] = a.y;
                xv[t][j][4 * q + 2] = a.z;
                xv[t][j][4 * q + 3] = a.w;
            }
        }
    }

    int my_acc[MT];  // lane r keeps the accumulator of row row0 + r
#pragma unroll
    for (int t = 0; t < MT; ++t) my_acc[t] = 0;

    for (int64_t row = row0; row < row1; row += kGemvRowBatch) {
        uint4 w[kGemvRowBatch][CH];
#pragma unroll
        for (int rb = 0; rb < kGemvRowBatch; ++rb) {
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int c = lane + kWave * j;
                w[rb][j] = make_uint4(0, 0, 0, 0);
                if (row + rb < row1 && c < nchunk)
                    w[rb][j] = *reinterpret_cast<const uint4*>(packed + (row + rb) * row_bytes +
                                                               16 * (int64_t)c);
            }
        }
#pragma unroll
        for (int rb = 0; rb < kGemvRowBatch; ++rb) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                int s0 = 0, s1 = 0, s2 = 0, s3 = 0;
#pragma unroll
                for (int j = 0; j < CH; ++j) {
                    const uint32_t ws[4] = {w[rb][j].x, w[rb][j].y, w[rb][j].z, w[rb][j].w};
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t word = ws[d];
                        s0 = dot4(word & 0x03030303u, xv[t][j][4 * d + 0], s0);
                        s1 = dot4(word & 0x0C0C0C0Cu, xv[t][j][4 * d + 1], s1);
                        s2 = dot4(word & 0x30303030u, xv[t][j][4 * d + 2], s2);
                        s3 = dot4((word >> 6) & 0x03030303u, xv[t][j][4 * d + 3], s3);
                    }
                }
                const int total = wave_sum_dpp(s0 + (s1 >> 2) + (s2 >> 4) + s3);
                if (lane == (int)(row + rb - row0)) my_acc[t] = total;
            }
        }
    }

    const int64_t r = row0 + lane;
    if (r < row1) {
        const float d_w = w_scale[0];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int a = my_acc[t] - x_qsum[t];
            if (acc_out != nullptr) acc_out[(int64_t)t * N + r] = a;
            y[(int64_t)t * N + r] = ((float)a * x_scale[t]) * d_w;
        }
    }
}

constexpr int kMaxXRegsChunks = 8;  // MT * CH limit: 16 * MT * CH activation VGPRs

template <int MT, int CH>
hipError_t launch_mt_ch(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                        const uint8_t* packed, const float* w_scale, int64_t N, int64_t K,
                        float* y, int32_t* acc, hipStream_t stream) {
    // Aim for ~8 waves per CU on 256 CUs, at most 64 rows per wave.
    const int64_t target_waves = 2048;
    int64_t rpw = (N + target_waves - 1) / target_waves;
    if (rpw < 1) rpw = 1;
    if (rpw > kWave) rpw = kWave;
    const int64_t waves = (N + rpw - 1) / rpw;
    const int64_t blocks = (waves + kGemvThreads / kWave - 1) / (kGemvThreads / kWave);
    hipLaunchKernelGGL((gemv_kernel<MT, CH>), dim3((unsigned)blocks), dim3(kGemvThreads), 0,
                       stream, xq, x_scale, x_qsum, packed, w_scale, (int)N, (int)K, (int)rpw, y,
                       acc);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(int ch, const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                     const uint8_t* packed, const float* w_scale, int64_t N, int64_t K, float* y,
                     int32_t* acc, hipStream_t stream) {
#define BITNET_GEMV_CH(C)                                                                      \
    if (ch <= C) {                                                                             \
        if constexpr (MT * C <= kMaxXRegsChunks)                                               \
            return launch_mt_ch<MT, C>(xq, x_scale, x_qsum, packed, w_scale, N, K, y, acc,     \
                                       stream);                                                \
        return hipErrorInvalidValue;                                                           \
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

int chunks_per_lane(int64_t K) { return (int)((K / 64 + kWave - 1) / kWave); }

// The chunk counts instantiated: 1, 2, 3, 4, 6, 8 (larger counts are not supported).
int rounded_ch(int ch) { return ch <= 4 ? ch : (ch <= 6 ? 6 : (ch <= 8 ? 8 : ch)); }

}  // namespace

bool gemv_supported(int64_t M, int64_t K) {
    if (M < 1 || M > 4) return false;
    return M * rounded_ch(chunks_per_lane(K)) <= kMaxXRegsChunks;
}

hipError_t launch_gemv(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                       const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                       int64_t K, float* y, int32_t* acc, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    const int ch = chunks_per_lane(K);
    switch (M) {
        case 1: return launch_mt<1>(ch, xq, x_scale, x_qsum, packed, w_scale, N, K, y, acc, stream);
        case 2: return launch_mt<2>(ch, xq, x_scale, x_qsum, packed, w_scale, N, K, y, acc, stream);
        case 3: return launch_mt<3>(ch, xq, x_scale, x_qsum, packed, w_scale, N, K, y, acc, stream);
        case 4: return launch_mt<4>(ch, xq, x_scale, x_qsum, packed, w_scale, N, K, y, acc, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bitnet
