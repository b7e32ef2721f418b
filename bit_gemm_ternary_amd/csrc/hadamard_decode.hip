// hadamard_decode.hip - one-token H-BitLinear forward in one launch: the
// Walsh-Hadamard transform of the token, its per-token absmax 4-bit codes and
// the ternary GEMV on signed 4-bit dot products.
//
// Follows the BitNet v2 summary ("초저용량 LLM의 진화: BitNet v2 파헤치기",
// section 방법론): an H-BitLinear layer transforms its input with a Hadamard
// matrix and quantises it to 4-bit per-token absmax codes before the ternary
// contraction (weights packed with the matching row transform).  The
// arithmetic is that of hadamard_quant.hip (transform, codes, d_x) followed by
// the nibble contraction of gemv.hip (v_dot8_i32_i4 on the weight fields of
// two packing slots per nibble lane), so codes and accumulators are
// bit-identical to those two launches.
//
// Layout: one workgroup per CU (256 threads up to K = 4096, 512 above).
// Every workgroup repeats the token's transform (K log2 K float32
// butterflies, E = K / threads values per thread), and every weight load of a
// wave's rows is issued before it, so the weight stream is in flight through
// the whole prologue.  Wave g of the W waves owns the RB rows g, g + W, ... (one
// register set, no per-row branch: rows past N load zeros and store nothing);
// lane l owns the 16-byte chunks l, l + 64, ... of every row.  Order of work:
//   1. the token's bf16 values (E contiguous per thread), the gain and d_w,
//      then every weight load;
//   2. sum of x^2 (exact float32 squares in four float32 chains, combined in
//      float64), the gain, the transform (LDS exchanges between its phases);
//   3. absmax and sum of squares over the workgroup, one barrier;
//   4. the codes into LDS (piece-major, below), with the code sums, one
//      barrier;
//   5. each lane's chunks of codes from LDS as nibble dwords (in a group of
//      16 codes, byte j holds code j low and code 8 + j high); workgroup 0
//      stores them and the token's d_x and code sum;
//   6. per row, the dot products over the lane's chunks, a wave sum, and the
//      store by lane rb.
#include "common.hpp"
#include "hadamard.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

using hadamard::Fwht;

constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer descriptor word 3 (gfx9 family)
constexpr uint32_t kOutOfRange = 0x80000000u;   // offset past every buffer used here: loads 0
constexpr int kMaxRecords = 0x7fffffff;
constexpr int kMinP = 10, kMaxP = 14;           // K = 1024 .. 16384
constexpr int kMaxWeightRegs = 16;              // RB * CH 16-byte weight vectors per lane

struct HArgs {
    const uint16_t* x;       // bf16 [K]
    const float* gain;       // [K] or NULL
    float eps;
    double sqrt_k;           // sqrt(K) as the host computes it (the transform's normalisation)
    const uint8_t* packed;   // [N][K/4]
    const float* w_scale;    // d_w at [0]
    int N;
    float* y;                // [N]
    uint8_t* xq4;            // [K/2] nibble codes, written by workgroup 0
    float* x_scale;          // d_x, written by workgroup 0
    int32_t* x_qsum;         // sum of the codes, written by workgroup 0
    int32_t* acc;            // [N] or NULL
};

// The codes in LDS piece-major: the 16-byte piece q of chunk c (codes
// 64c + 16q .. 64c + 16q + 15) at q * kPlane + 16 c.  A lane reading piece q
// of its own chunk then meets its 15 neighbours on 15 other 16-byte bank
// groups (chunk-major rows 64 bytes apart put four lanes on each group), and
// a plane stride of K / 4 + 64 bytes keeps the transform's grouped code stores
// on distinct banks as well (one exception, two-way, for the 8-code groups at
// K = 8192).  The address is a bit permutation of k plus the plane padding,
// additive over disjoint bits as store_codes requires.
template <int P>
struct PieceMajorCodes {
    static constexpr int kPlane = (1 << P) / 4 + 64;
    static constexpr int addr(int k) { return ((k >> 4) & 3) * kPlane + ((k >> 6) << 4) + (k & 15); }
};

template <int P>
constexpr int chunks_per_lane() {
    return ((1 << P) / 64 + kWave - 1) / kWave;
}

// Threads per workgroup: 256 (E = 4 .. 16 values per thread) up to K = 4096,
// 512 above (E = 16, 32), so that the transform, which every workgroup
// repeats, has two waves per SIMD to overlap its LDS exchanges with.
template <int P>
constexpr int threads_for() {
    return P >= 13 ? 512 : 256;
}

template <int P, int RB>
__global__ __launch_bounds__(threads_for<P>()) void hdecode_kernel(const HArgs a) {
    constexpr int NT = threads_for<P>();
    constexpr int K = 1 << P;
    constexpr int E = K / NT;
    using F = Fwht<P, E>;
    static_assert(F::B == NT, "one transform value set per thread");
    constexpr int NW = NT / kWave;
    constexpr int NCH = K / 64;                 // 16-byte chunks per packed row
    constexpr int CH = chunks_per_lane<P>();
    constexpr int ROW = K / 4;                  // bytes per packed row
    constexpr int XW = E / 2;                   // bf16 pairs per thread
    static_assert(RB >= 1 && RB * CH <= kMaxWeightRegs, "one register set of rows");
    __shared__ __align__(16) float lds[F::LDS_FLOATS];
    __shared__ float red_f[NW];
    __shared__ double red_d[NW];
    __shared__ int red_i[NW];

    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int g = (int)blockIdx.x * NW + wave;
    const int W = (int)gridDim.x * NW;
    const int N = a.N;

    // 1. Token, gain and d_w (vector loads: a scalar load would be waited for
    // at the first barrier with the LDS traffic), then every weight load.
    uint32_t xw[XW];
    if constexpr (E >= 8) {
        const uint4* p4 = reinterpret_cast<const uint4*>(a.x + t * E);
#pragma unroll
        for (int q = 0; q < E / 8; ++q) {
            const uint4 u = p4[q];
            xw[4 * q] = u.x;
            xw[4 * q + 1] = u.y;
            xw[4 * q + 2] = u.z;
            xw[4 * q + 3] = u.w;
        }
    } else {
        static_assert(E == 4, "E");
        const uint2 u = *reinterpret_cast<const uint2*>(a.x + t * E);
        xw[0] = u.x;
        xw[1] = u.y;
    }
    const bool has_gain = a.gain != nullptr;
    float gv[E];
    if (has_gain) {
        const float4* g4 = reinterpret_cast<const float4*>(a.gain + t * E);
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
            const float4 u = g4[q];
            gv[4 * q] = u.x;
            gv[4 * q + 1] = u.y;
            gv[4 * q + 2] = u.z;
            gv[4 * q + 3] = u.w;
        }
    }
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc((void*)a.w_scale, (short)0, 4,
                                                                         (int)kBufferWord3);
    const float dw0 = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(sres, 0, 0, 0));
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.packed + (int64_t)(g < N ? g : 0) * ROW), (short)0, kMaxRecords, (int)kBufferWord3);
    uint4 w[RB][CH];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = lane + kWave * j;
            const bool ok = (int64_t)g + (int64_t)rb * W < N && c < NCH;
            const v4i q = __builtin_amdgcn_raw_buffer_load_b128(
                wres, ok ? (uint32_t)(rb * W * ROW + 16 * c) : kOutOfRange, 0, 0);
            w[rb][j] = make_uint4((uint32_t)q[0], (uint32_t)q[1], (uint32_t)q[2], (uint32_t)q[3]);
        }
    // The weight loads stay ahead of the token's arithmetic (the scheduler
    // would otherwise sink them below the wait for the token).
    __builtin_amdgcn_sched_barrier(0);

    // 2. Sum of squares of x, the gain, the transform.
    float v[E];
    float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < XW; ++i) {
        v[2 * i] = bf16_lo(xw[i]);
        v[2 * i + 1] = bf16_hi(xw[i]);
    }
#pragma unroll
    for (int r = 0; r < E; ++r) sq[r % 4] = __fmaf_rn(v[r], v[r], sq[r % 4]);
    double ss = ((double)sq[0] + (double)sq[1]) + ((double)sq[2] + (double)sq[3]);
    if (has_gain) {
#pragma unroll
        for (int r = 0; r < E; ++r) v[r] *= gv[r];
    }
    F::template run<0>(v, lds, t);

    // 3. Absmax of the transform and the sum of squares over the workgroup.
    // The transform's last LDS read is behind a barrier, so `lds` is free.
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < E; ++r) amax = fmaxf(amax, fabsf(v[r]));
    amax = wave_max_dpp(amax);
    ss = wave_sum_dpp(ss);
    if (lane == 0) {
        red_f[wave] = amax;
        red_d[wave] = ss;
    }
    __syncthreads();
    amax = red_f[0];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) amax = fmaxf(amax, red_f[wv]);

    // 4. Codes rint(t * rn(7 / amax)), |t| <= amax so within [-7, 7]; a token
    // below the tiny absmax has scale 0 and all-zero codes.
    const float scale = amax < kTinyAbsmax ? 0.f : 7.0f / amax;
    int8_t* lds8 = reinterpret_cast<int8_t*>(lds);
    using CL = PieceMajorCodes<P>;
    static_assert(4 * CL::kPlane <= 4 * F::LDS_FLOATS, "the codes fit the transform's LDS");
    int qs = hadamard::store_codes<P, E, CL>(v, scale, lds8, t);
    qs = wave_sum_dpp(qs);
    if (lane == 0) red_i[wave] = qs;
    __syncthreads();

    // 5. Nibble dwords of my chunks: chunk c holds codes 64c .. 64c + 63, four
    // groups of 16; dwords 2d and 2d + 1 are group d's (codes 0-3 | 8-11 << 4)
    // and (codes 4-7 | 12-15 << 4), the order the weight fields come in.
    uint32_t xv[CH][8];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = lane + kWave * j;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint4 q = make_uint4(0, 0, 0, 0);
            if (c < NCH) q = *reinterpret_cast<const uint4*>(lds8 + d * CL::kPlane + 16 * c);
            xv[j][2 * d] = (q.x & 0x0F0F0F0Fu) | ((q.z & 0x0F0F0F0Fu) << 4);
            xv[j][2 * d + 1] = (q.y & 0x0F0F0F0Fu) | ((q.w & 0x0F0F0F0Fu) << 4);
        }
    }
    int tok_sum = red_i[0];
    double sum_sq = red_d[0];
#pragma unroll
    for (int wv = 1; wv < NW; ++wv) {
        tok_sum += red_i[wv];
        sum_sq += red_d[wv];
    }
    const float d_x = token_scale(amax, sum_sq, 1.0 / (double)K, a.eps, 1.0 / (7.0 * a.sqrt_k));
    if (blockIdx.x == 0 && wave == 0) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = lane + kWave * j;
            if (c < NCH) {
                uint4* dst = reinterpret_cast<uint4*>(a.xq4 + 32 * c);
                dst[0] = make_uint4(xv[j][0], xv[j][1], xv[j][2], xv[j][3]);
                dst[1] = make_uint4(xv[j][4], xv[j][5], xv[j][6], xv[j][7]);
            }
        }
        if (lane == 0) {
            a.x_scale[0] = d_x;
            a.x_qsum[0] = tok_sum;
        }
    }
    if (g >= N) return;  // after the last barrier: wave-uniform exit

    // 6. Rows.  The fields of slots 0 and 2 (w & 0x33333333) and of slots 1
    // and 3 ((w >> 2) & 0x33333333) are 4-bit lanes holding q + 1 for weights
    // 16g + j, 16g + 8 + j and 16g + 4 + j, 16g + 12 + j: the nibble order of
    // the group's two code dwords.  sum q x = sum (q + 1) x - sum x.
    int tot[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int s = 0;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const uint32_t ws[4] = {w[rb][j].x, w[rb][j].y, w[rb][j].z, w[rb][j].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                s = __builtin_amdgcn_sdot8((int)(ws[d] & 0x33333333u), (int)xv[j][2 * d], s, false);
                s = __builtin_amdgcn_sdot8((int)((ws[d] >> 2) & 0x33333333u), (int)xv[j][2 * d + 1], s, false);
            }
        }
        tot[rb] = wave_sum_dpp(s);
    }
    int mine = tot[0];
#pragma unroll
    for (int rb = 1; rb < RB; ++rb) mine = lane == rb ? tot[rb] : mine;
    if (lane < RB) {
        const int64_t r = (int64_t)g + (int64_t)lane * W;
        if (r < N) {
            const int acc = mine - tok_sum;
            if (a.acc != nullptr) a.acc[r] = acc;
            a.y[r] = ((float)acc * d_x) * dw0;
        }
    }
}

// Waves of one workgroup per CU (256 CUs).
template <int P>
constexpr int64_t chip_waves() {
    return 256 * (threads_for<P>() / kWave);
}

// RB = ceil(N / chip_waves) rows per wave over ceil(N / RB) waves (one
// workgroup per CU, or a few CUs idle), as long as a wave's rows fit one
// register set.
template <int P, int RB>
hipError_t launch_rb(const HArgs& a, hipStream_t stream) {
    constexpr int NW = threads_for<P>() / kWave;
    const int64_t waves = (a.N + RB - 1) / RB;
    const dim3 grid((unsigned)((waves + NW - 1) / NW));
    return launch_kernel((hdecode_kernel<P, RB>), grid, dim3(threads_for<P>()), 0, stream, a);
}

template <int P>
hipError_t launch_p(const HArgs& a, hipStream_t stream) {
    constexpr int CH = chunks_per_lane<P>();
    const int64_t rpw = (a.N + chip_waves<P>() - 1) / chip_waves<P>();
#define BITNET_HDECODE_RB(R) \
    if constexpr (R * CH <= kMaxWeightRegs) \
        if (rpw == R) return launch_rb<P, R>(a, stream);
    BITNET_HDECODE_RB(1) BITNET_HDECODE_RB(2) BITNET_HDECODE_RB(3) BITNET_HDECODE_RB(4)
    BITNET_HDECODE_RB(5) BITNET_HDECODE_RB(6) BITNET_HDECODE_RB(7) BITNET_HDECODE_RB(8)
    BITNET_HDECODE_RB(9) BITNET_HDECODE_RB(10) BITNET_HDECODE_RB(11) BITNET_HDECODE_RB(12)
    BITNET_HDECODE_RB(13) BITNET_HDECODE_RB(14) BITNET_HDECODE_RB(15) BITNET_HDECODE_RB(16)
#undef BITNET_HDECODE_RB
    return hipErrorNotSupported;
}

int log2_of_pow2(int64_t k) {
    int p = 0;
    while ((int64_t{1} << p) < k) ++p;
    return p;
}

}  // namespace

bool hadamard_decode_supported(int64_t N, int64_t K) {
    if (N < 1 || K < (1 << kMinP) || K > (1 << kMaxP) || (K & (K - 1)) != 0) return false;
    const int64_t ch = (K / 64 + kWave - 1) / kWave;
    const int64_t waves = K >= 8192 ? chip_waves<13>() : chip_waves<12>();
    return ((N + waves - 1) / waves) * ch <= kMaxWeightRegs;
}

hipError_t launch_hadamard_decode(const uint16_t* x, const float* gain, float eps, double sqrt_k,
                                  const uint8_t* packed, const float* w_scale, int64_t N, int64_t K,
                                  float* y, uint8_t* xq4, float* x_scale, int32_t* x_qsum,
                                  int32_t* acc, hipStream_t stream) {
    if (!hadamard_decode_supported(N, K)) return hipErrorNotSupported;
    HArgs a{};
    a.x = x, a.gain = gain, a.eps = eps, a.sqrt_k = sqrt_k, a.packed = packed, a.w_scale = w_scale;
    a.N = (int)N, a.y = y, a.xq4 = xq4, a.x_scale = x_scale, a.x_qsum = x_qsum, a.acc = acc;
    switch (log2_of_pow2(K)) {
        case 10: return launch_p<10>(a, stream);
        case 11: return launch_p<11>(a, stream);
        case 12: return launch_p<12>(a, stream);
        case 13: return launch_p<13>(a, stream);
        case 14: return launch_p<14>(a, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace bitnet
