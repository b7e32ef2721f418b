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
// Mapping: a wavefront owns up to 64 consecutive output rows, processed in
// batches of RB rows whose loads are all issued before any of them is used.
// Lane l owns the 16-byte packed chunks l, l+64, ... of every row (64 weights
// per chunk), so a wave reads 1 KiB of a row per load instruction, fully
// coalesced.  The matching 64 activation bytes per chunk stay in registers.
//
// Unpack: a packed word holds weights 16g..16g+15; with the field of weight
// 16g+4i+b at bits 8b+2i, (word & (3 << 2i) per byte) gives the four codes
// (q+1) of weights 16g+4i..16g+4i+3 times 4^i, in byte order, which
// v_dot4_i32_i8 multiplies with the activation dword 4g+i.  Slots i = 0, 1, 2
// need only the mask (codes times 1, 4, 16 fit a signed byte); slot 3 is shifted
// down first.  The four slot sums are combined exactly as s0 + s1/4 + s2/16 + s3.
// The offset code q + 1 is corrected at the end: sum q x = sum (q+1) x - sum x.
//
// Fused variant: each 256-thread workgroup first quantises the (<= 4) tokens
// itself (RMSNorm + absmax int8, the same arithmetic as quant_act.hip) from the
// bf16 input, which every workgroup reads from L2, and shares the codes through
// LDS; the weight loads of the first batch are issued right after the
// activation loads and stay in flight through that prologue.  This removes the
// separate quantisation launch from the decode critical path.
#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;
constexpr int kMaxXRegsChunks = 8;
// Fused decode launch shape: 256-thread workgroups, about 1024 waves in all
// (measured on the decode projections against 512- and 1024-thread
// workgroups and 2048 or 4096 waves).
constexpr int kFusedThreads = 256;
constexpr int kFusedWaves = 1024;  // MT * CH limit: 16 * MT * CH activation VGPRs

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Rows per batch: all loads of a batch are in flight together (4*RB*CH VGPRs).
template <int CH>
constexpr int rows_per_batch() {
    return CH == 1 ? 16 : (CH == 2 ? 8 : (CH <= 4 ? 4 : 2));
}

// MT tokens, CH 16-byte chunks per lane per row (K <= CH * 4096).
template <int MT, int CH>
struct GemvCore {
    static constexpr int RB = rows_per_batch<CH>();

    // Loads of rows [r, r + RB) (zero beyond row1 or past the last chunk).
    __device__ static __forceinline__ void load(uint4 (&w)[RB][CH], const uint8_t* packed,
                                                int64_t row_bytes, int nchunk, int64_t r,
                                                int64_t row1, int lane) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int c = lane + kWave * j;
                w[rb][j] = make_uint4(0, 0, 0, 0);
                if (r + rb < row1 && c < nchunk)
                    w[rb][j] = *reinterpret_cast<const uint4*>(packed + (r + rb) * row_bytes +
                                                               16 * (int64_t)c);
            }
        }
    }

    // Dot products of one batch; the wave total of row r + rb lands in lane
    // (r + rb - row0) of my_acc.
    __device__ static __forceinline__ void compute(const uint4 (&w)[RB][CH],
                                                   const uint32_t (&xv)[MT][CH][16], int64_t r,
                                                   int64_t row0, int64_t row1, int lane,
                                                   int (&my_acc)[MT]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (r + rb >= row1) break;  // wave-uniform: the batch's last rows may be past row1
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
                if (lane == (int)(r + rb - row0)) my_acc[t] = total;
            }
        }
    }

    // Process rows [row0, row1) of this wave, the first batch already loaded in w.
    __device__ static __forceinline__ void run(uint4 (&w)[RB][CH], const uint32_t (&xv)[MT][CH][16],
                                               const uint8_t* packed, int64_t row_bytes,
                                               int nchunk, int64_t row0, int64_t row1, int lane,
                                               int (&my_acc)[MT]) {
        for (int64_t r = row0; r < row1; r += RB) {
            if (r != row0) load(w, packed, row_bytes, nchunk, r, row1, lane);
            compute(w, xv, r, row0, row1, lane, my_acc);
        }
    }

    // Epilogue: lane i writes row row0 + i.
    __device__ static __forceinline__ void store(const int (&my_acc)[MT], const float* x_scale,
                                                 const int32_t* x_qsum, const RowScales& scales,
                                                 int64_t N, int64_t row0, int64_t row1, int lane,
                                                 float* y, int32_t* acc_out) {
        const int64_t r = row0 + lane;
        if (r < row1) {
            const float d_w = scales.of(r, scales.w_scale[0]);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int a = my_acc[t] - x_qsum[t];
                if (acc_out != nullptr) acc_out[(int64_t)t * N + r] = a;
                y[(int64_t)t * N + r] = ((float)a * x_scale[t]) * d_w;
            }
        }
    }
};

template <int MT, int CH>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ x_qsum, const uint8_t* __restrict__ packed,
    const RowScales scales, int N, int K, int rows_per_wave, float* __restrict__ y,
    int32_t* __restrict__ acc_out) {
    using G = GemvCore<MT, CH>;
    const int lane = threadIdx.x % kWave;
    const int wave = (int)((blockIdx.x * (int64_t)kGemvThreads + threadIdx.x) / kWave);
    const int64_t row0 = (int64_t)wave * rows_per_wave;
    if (row0 >= N) return;  // wave-uniform; no workgroup barrier in this kernel
    const int64_t row1 = min((int64_t)N, row0 + rows_per_wave);
    const int nchunk = K / 64;
    const int64_t row_bytes = K / 4;

    uint4 w[G::RB][CH];
    G::load(w, packed, row_bytes, nchunk, row0, row1, lane);

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

    int my_acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) my_acc[t] = 0;
    G::run(w, xv, packed, row_bytes, nchunk, row0, row1, lane, my_acc);
    G::store(my_acc, x_scale, x_qsum, scales, N, row0, row1, lane, y, acc_out);
}

// Fused RMSNorm + int8 quantisation + GEMV.  Every workgroup quantises the MT
// tokens (K <= CH * 4096) into LDS; workgroup 0 also writes the codes, scales
// and sums to global memory.
//
// Order matters for latency: the bf16 activations are loaded first and the
// weights second, so the prologue (which waits for its own loads, and loads
// complete in issue order) does not wait for the weights; the weight loads
// stay in flight through the prologue.  The prologue needs one workgroup
// reduction (absmax and sum of squares of every token together); each wave
// then sums the codes it reads back from LDS itself.
template <int MT, int CH, int NT>
__global__ __launch_bounds__(NT) void fused_decode_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ gain, float eps,
    const uint8_t* __restrict__ packed, const RowScales scales, int N, int K,
    int rows_per_wave, float* __restrict__ y, int8_t* __restrict__ xq_out,
    float* __restrict__ x_scale_out, int32_t* __restrict__ x_qsum_out,
    int32_t* __restrict__ acc_out) {
    using G = GemvCore<MT, CH>;
    constexpr int NW = NT / kWave;
    constexpr int XV = (CH * 512 + NT - 1) / NT;  // 8-value bf16 vectors per thread per token (K <= CH*4096)
    __shared__ __align__(16) int8_t codes[MT][CH * 4096];
    __shared__ float red_f[MT][NW];
    __shared__ double red_d[MT][NW];

    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wave_id = t / kWave;
    const int64_t row0 = ((int64_t)blockIdx.x * NW + wave_id) * rows_per_wave;
    const int64_t row1 = min((int64_t)N, row0 + rows_per_wave);
    const int nchunk = K / 64;
    const int64_t row_bytes = K / 4;
    const int nvec = K / 8;

    // 1. Activation loads, then weight loads (in flight through the prologue).
    uint4 raw[MT][XV];
#pragma unroll
    for (int tok = 0; tok < MT; ++tok) {
        const uint4* xr = reinterpret_cast<const uint4*>(x + (int64_t)tok * K);
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int v = t + NT * i;
            raw[tok][i] = v < nvec ? xr[v] : make_uint4(0, 0, 0, 0);
        }
    }
    uint4 w[G::RB][CH];
    G::load(w, packed, row_bytes, nchunk, row0, row1, lane);

    auto values = [&](int tok, int i, int v, float (&u)[8], bool with_gain) {
        const uint32_t ws[4] = {raw[tok][i].x, raw[tok][i].y, raw[tok][i].z, raw[tok][i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[2 * e] = bf16_lo(ws[e]);
            u[2 * e + 1] = bf16_hi(ws[e]);
        }
        if (with_gain && gain != nullptr) {
            const float4 g0 = reinterpret_cast<const float4*>(gain)[2 * v];
            const float4 g1 = reinterpret_cast<const float4*>(gain)[2 * v + 1];
            u[0] *= g0.x; u[1] *= g0.y; u[2] *= g0.z; u[3] *= g0.w;
            u[4] *= g1.x; u[5] *= g1.y; u[6] *= g1.z; u[7] *= g1.w;
        }
    };

    // 2. Per-token absmax of x*gain and sum of x^2: one workgroup reduction.
#pragma unroll
    for (int tok = 0; tok < MT; ++tok) {
        float amax = 0.f;
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int v = t + NT * i;
            if (v < nvec) {
                float u[8];
                values(tok, i, v, u, false);
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += (double)u[e] * (double)u[e];
                values(tok, i, v, u, true);
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(u[e]));
            }
        }
        amax = wave_max_dpp(amax);
        ss = wave_sum_dpp(ss);
        if (lane == 0) {
            red_f[tok][wave_id] = amax;
            red_d[tok][wave_id] = ss;
        }
    }
    __syncthreads();

    // 3. Codes into LDS; every thread derives the same scales.  The dequant
    // factor (which needs a double square root and division) is only computed
    // in the epilogue, off the path to the contraction.
    float tok_amax[MT];
#pragma unroll
    for (int tok = 0; tok < MT; ++tok) {
        float amax = red_f[tok][0];
#pragma unroll
        for (int wv = 1; wv < NW; ++wv) amax = fmaxf(amax, red_f[tok][wv]);
        tok_amax[tok] = amax;
        const bool zero = amax < kTinyAbsmax;
        const float scale = zero ? 0.f : 127.0f / amax;
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int v = t + NT * i;
            if (v < nvec) {
                float u[8];
                values(tok, i, v, u, true);
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int q0 = zero ? 0 : round_clamp(u[e] * scale, -128.f, 127.f);
                    const int q1 = zero ? 0 : round_clamp(u[4 + e] * scale, -128.f, 127.f);
                    lo |= (uint32_t)(q0 & 0xff) << (8 * e);
                    hi |= (uint32_t)(q1 & 0xff) << (8 * e);
                }
                *reinterpret_cast<uint2*>(&codes[tok][8 * v]) = make_uint2(lo, hi);
            }
        }
    }
    __syncthreads();

    // 4. Codes of my chunks into registers; the wave sums them itself.
    uint32_t xv[MT][CH][16];
    int tok_sum[MT];
#pragma unroll
    for (int tok = 0; tok < MT; ++tok) {
        int part = 0;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = lane + kWave * j;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint4 a = make_uint4(0, 0, 0, 0);
                if (c < nchunk) a = reinterpret_cast<const uint4*>(&codes[tok][64 * c])[q];
                xv[tok][j][4 * q] = a.x;
                xv[tok][j][4 * q + 1] = a.y;
                xv[tok][j][4 * q + 2] = a.z;
                xv[tok][j][4 * q + 3] = a.w;
                part = dot4(a.x, 0x01010101u, part);
                part = dot4(a.y, 0x01010101u, part);
                part = dot4(a.z, 0x01010101u, part);
                part = dot4(a.w, 0x01010101u, part);
            }
        }
        tok_sum[tok] = wave_sum_dpp(part);
    }

    auto dequant_scale = [&](int tok) {
        double ss = red_d[tok][0];
#pragma unroll
        for (int wv = 1; wv < NW; ++wv) ss += red_d[tok][wv];
        const double rstd = 1.0 / sqrt(ss / (double)K + (double)eps);
        return tok_amax[tok] < kTinyAbsmax ? 0.f : (float)(((double)tok_amax[tok] * rstd) / 127.0);
    };
    if (blockIdx.x == 0) {
        for (int tok = 0; tok < MT; ++tok) {
            for (int v = t; v < K / 16; v += NT)
                reinterpret_cast<uint4*>(xq_out + (int64_t)tok * K)[v] =
                    reinterpret_cast<const uint4*>(codes[tok])[v];
            if (t == 0) {
                x_scale_out[tok] = dequant_scale(tok);
                x_qsum_out[tok] = tok_sum[tok];
            }
        }
    }
    if (row0 >= N) return;  // after the last barrier: wave-uniform exit

    int my_acc[MT];
#pragma unroll
    for (int tok = 0; tok < MT; ++tok) my_acc[tok] = 0;
    G::run(w, xv, packed, row_bytes, nchunk, row0, row1, lane, my_acc);
    float tok_scale[MT];
#pragma unroll
    for (int tok = 0; tok < MT; ++tok) tok_scale[tok] = dequant_scale(tok);
    G::store(my_acc, tok_scale, tok_sum, scales, N, row0, row1, lane, y, acc_out);
}

// Rows per wave: spread the rows over about `target_waves` waves (at most 64).
int64_t rows_per_wave(int64_t N, int64_t target_waves) {
    int64_t rpw = (N + target_waves - 1) / target_waves;
    if (rpw < 1) rpw = 1;
    if (rpw > kWave) rpw = kWave;
    return rpw;
}

struct Args {
    const int8_t* xq;
    const float* x_scale;
    const int32_t* x_qsum;
    const uint16_t* x;
    const float* gain;
    float eps;
    const uint8_t* packed;
    RowScales scales;
    int64_t N, K;
    float* y;
    int8_t* xq_out;
    float* x_scale_out;
    int32_t* x_qsum_out;
    int32_t* acc;
    hipStream_t stream;
};

template <int MT, int CH>
struct Standalone {
    static hipError_t run(const Args& a) {
        const int64_t rpw = rows_per_wave(a.N, 2048);
        const int64_t blocks = ((a.N + rpw - 1) / rpw + kGemvWaves - 1) / kGemvWaves;
        return launch_kernel((gemv_kernel<MT, CH>), dim3((unsigned)blocks), dim3(kGemvThreads), 0,
                             a.stream, a.xq, a.x_scale, a.x_qsum, a.packed, a.scales, (int)a.N,
                             (int)a.K, (int)rpw, a.y, a.acc);
    }
};

template <int MT, int CH>
struct Fused {
    static constexpr int NT = kFusedThreads;
    static hipError_t run(const Args& a) {
        // Every workgroup repeats the quantisation, so about one workgroup
        // per CU; its prologue is split over NT threads.
        const int64_t rpw = rows_per_wave(a.N, kFusedWaves);
        const int64_t blocks = ((a.N + rpw - 1) / rpw + NT / kWave - 1) / (NT / kWave);
        return launch_kernel((fused_decode_kernel<MT, CH, NT>), dim3((unsigned)blocks),
                             dim3(NT), 0, a.stream, a.x, a.gain, a.eps, a.packed,
                             a.scales, (int)a.N, (int)a.K, (int)rpw, a.y, a.xq_out,
                             a.x_scale_out, a.x_qsum_out, a.acc);
    }
};

template <template <int, int> class L, int MT>
hipError_t dispatch_ch(int ch, const Args& a) {
#define BITNET_GEMV_CH(C)                                                  \
    if (ch <= C) {                                                         \
        if constexpr (MT * C <= kMaxXRegsChunks) return L<MT, C>::run(a); \
        return hipErrorInvalidValue;                                       \
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

template <template <int, int> class L>
hipError_t dispatch(int64_t M, int ch, const Args& a) {
    switch (M) {
        case 1: return dispatch_ch<L, 1>(ch, a);
        case 2: return dispatch_ch<L, 2>(ch, a);
        case 3: return dispatch_ch<L, 3>(ch, a);
        case 4: return dispatch_ch<L, 4>(ch, a);
        default: return hipErrorInvalidValue;
    }
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
                       const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                       int64_t K, float* y, int32_t* acc, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    Args a{};
    a.xq = xq, a.x_scale = x_scale, a.x_qsum = x_qsum, a.packed = packed, a.scales = scales;
    a.N = N, a.K = K, a.y = y, a.acc = acc, a.stream = stream;
    return dispatch<Standalone>(M, chunks_per_lane(K), a);
}

hipError_t launch_fused_decode(const uint16_t* x, const float* gain, float eps,
                               const uint8_t* packed, const RowScales& scales, int64_t M,
                               int64_t N, int64_t K, float* y, int8_t* xq, float* x_scale,
                               int32_t* x_qsum, int32_t* acc, hipStream_t stream) {
    Args a{};
    a.x = x, a.gain = gain, a.eps = eps, a.packed = packed, a.scales = scales;
    a.N = N, a.K = K, a.y = y, a.xq_out = xq, a.x_scale_out = x_scale, a.x_qsum_out = x_qsum;
    a.acc = acc, a.stream = stream;
    return dispatch<Fused>(M, chunks_per_lane(K), a);
}

}  // namespace bitnet
