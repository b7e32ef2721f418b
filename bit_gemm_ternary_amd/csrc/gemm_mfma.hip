// gemm_mfma.hip - compute-bound prefill contraction on int8 matrix cores.
//
// acc[m][n] = sum_k q_x[m][k] * q_w[n][k] in int32, y = acc * d_x[m] * d_w.
// The pages describe the contraction as integer additions (Hugging Face
// 1.58-bit write-up, section 계산 패러다임) done by kernels that unpack the
// packed weights on the fly (section 추론 최적화 및 커스텀 커널) over tiles held in
// fast on-chip memory (section 타일링 매트릭스 곱셈).  At prefill sizes the
// contraction is dense and MFMA-bound, so here it runs on
// v_mfma_i32_16x16x64_i8 with the weights' offset codes (q + 1, values 0..2)
// as the A operand and the int8 activations as the B operand; the offset is
// removed in the epilogue with the per-token code sums.
//
// Tiling: a workgroup computes a BN (weight rows) x BM (tokens) tile with
// WN x WM wavefronts, each owning (BN/WN) x (BM/WM) as 16x16 MFMA blocks.  Per
// K-stage of BK values the workgroup copies the packed weight tile (BK/4 bytes
// per row, 4x smaller than int8) and the int8 activation tile into LDS (double
// buffered, one barrier per stage); A fragments are unpacked from one packed
// dword per lane with shift/mask ((word >> 2i) & 0x03030303 is already in
// natural byte order), B fragments are one 16-byte LDS read per lane.
//
// MFMA operand layout used (16x16x64, wave64): lane l supplies row (l % 16) of
// A and column (l % 16) of B over the 16 K-values 16*(l/16) .. 16*(l/16)+15 of
// the 64-wide step (any K assignment shared by A and B gives the same sum);
// the result D[i][j] sits in lane j + 16*(i/4), element i % 4.
#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

template <int BN_, int BM_, int WN_, int WM_, int BK_>
struct GemmCfg {
    static constexpr int BN = BN_, BM = BM_, WN = WN_, WM = WM_, BK = BK_;
    static constexpr int NT = WN * WM * kWave;
    static constexpr int TN = BN / WN, TM = BM / WM;   // wave tile
    static constexpr int FN = TN / 16, FM = TM / 16;   // MFMA blocks per wave
    static constexpr int XS = BK + 16;                 // LDS row stride of the activation tile (bytes)
    static constexpr int WS = BK / 4 + 16;             // LDS row stride of the packed weight tile
    static constexpr int X_CHUNKS = BM * BK / 16;      // 16-byte chunks per stage
    static constexpr int W_CHUNKS = BN * BK / 64;
    static constexpr int X_LOADS = (X_CHUNKS + NT - 1) / NT;
    static constexpr int W_LOADS = (W_CHUNKS + NT - 1) / NT;
    static constexpr int LDS_X = BM * XS, LDS_W = BN * WS;
    static_assert(TN % 16 == 0 && TM % 16 == 0 && BK % 64 == 0, "tile shape");
};

__device__ __forceinline__ v4i unpack_codes(uint32_t w) {
    v4i r;
    r[0] = (int)(w & 0x03030303u);
    r[1] = (int)((w >> 2) & 0x03030303u);
    r[2] = (int)((w >> 4) & 0x03030303u);
    r[3] = (int)((w >> 6) & 0x03030303u);
    return r;
}

template <class C>
__global__ __launch_bounds__(C::NT) void gemm_kernel(
    const int8_t* __restrict__ X, const uint8_t* __restrict__ P, const float* __restrict__ x_scale,
    const int32_t* __restrict__ x_qsum, const float* __restrict__ w_scale, int M, int N, int K,
    float* __restrict__ y, int32_t* __restrict__ acc_out) {
    __shared__ __align__(16) int8_t lds_x[2][C::LDS_X];
    __shared__ __align__(16) uint8_t lds_w[2][C::LDS_W];

    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wave = t / kWave;
    const int wn = wave % C::WN, wm = wave / C::WN;
    const int64_t tiles_n = (N + C::BN - 1) / C::BN;
    const int64_t n0 = ((int64_t)blockIdx.x % tiles_n) * C::BN;
    const int64_t m0 = ((int64_t)blockIdx.x / tiles_n) * C::BM;
    const int64_t row_bytes = K / 4;

    uint4 rx[C::X_LOADS], rw[C::W_LOADS];

    // Global -> registers for the stage starting at k0 (zero outside M, N, K).
    auto load_stage = [&](int k0) {
#pragma unroll
        for (int i = 0; i < C::X_LOADS; ++i) {
            const int idx = t + i * C::NT;
            const int r = idx / (C::BK / 16), c = idx % (C::BK / 16);
            rx[i] = make_uint4(0, 0, 0, 0);
            if (idx < C::X_CHUNKS && m0 + r < M && k0 + 16 * c < K)
                rx[i] = *reinterpret_cast<const uint4*>(X + (m0 + r) * K + k0 + 16 * c);
        }
#pragma unroll
        for (int i = 0; i < C::W_LOADS; ++i) {
            const int idx = t + i * C::NT;
            const int r = idx / (C::BK / 64), c = idx % (C::BK / 64);
            rw[i] = make_uint4(0, 0, 0, 0);
            if (idx < C::W_CHUNKS && n0 + r < N && k0 + 64 * c < K)
                rw[i] = *reinterpret_cast<const uint4*>(P + (n0 + r) * row_bytes + k0 / 4 + 16 * c);
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < C::X_LOADS; ++i) {
            const int idx = t + i * C::NT;
            const int r = idx / (C::BK / 16), c = idx % (C::BK / 16);
            if (idx < C::X_CHUNKS) *reinterpret_cast<uint4*>(&lds_x[buf][r * C::XS + 16 * c]) = rx[i];
        }
#pragma unroll
        for (int i = 0; i < C::W_LOADS; ++i) {
            const int idx = t + i * C::NT;
            const int r = idx / (C::BK / 64), c = idx % (C::BK / 64);
            if (idx < C::W_CHUNKS) *reinterpret_cast<uint4*>(&lds_w[buf][r * C::WS + 16 * c]) = rw[i];
        }
    };

    v4i acc[C::FN][C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int nk = (K + C::BK - 1) / C::BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();

    const int frag_row = lane % 16;
    const int frag_grp = lane / 16;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_stage((kt + 1) * C::BK);
#pragma unroll
        for (int kk = 0; kk < C::BK; kk += 64) {
            v4i a[C::FN], b[C::FM];
#pragma unroll
            for (int i = 0; i < C::FN; ++i) {
                const int r = wn * C::TN + i * 16 + frag_row;
                const uint32_t word =
                    *reinterpret_cast<const uint32_t*>(&lds_w[buf][r * C::WS + kk / 4 + 4 * frag_grp]);
                a[i] = unpack_codes(word);
            }
#pragma unroll
            for (int j = 0; j < C::FM; ++j) {
                const int r = wm * C::TM + j * 16 + frag_row;
                b[j] = *reinterpret_cast<const v4i*>(&lds_x[buf][r * C::XS + kk + 16 * frag_grp]);
            }
#pragma unroll
            for (int i = 0; i < C::FN; ++i)
#pragma unroll
                for (int j = 0; j < C::FM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: D[n][m] -> y[m][n]; lane holds n = 4*(lane/16) + e, m = lane % 16.
    const float d_w = w_scale[0];
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
        const int64_t m = m0 + wm * C::TM + j * 16 + frag_row;
        if (m >= M) continue;
        const int32_t qs = x_qsum[m];
        const float sx = x_scale[m];
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
            const int64_t nb = n0 + wn * C::TN + i * 16 + 4 * frag_grp;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t n = nb + e;
                if (n < N) {
                    const int a = acc[i][j][e] - qs;
                    if (acc_out != nullptr) acc_out[m * N + n] = a;
                    y[m * N + n] = ((float)a * sx) * d_w;
                }
            }
        }
    }
}

template <class C>
hipError_t launch_cfg(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                      const uint8_t* packed, const float* w_scale, int64_t M, int64_t N, int64_t K,
                      float* y, int32_t* acc, hipStream_t stream) {
    const int64_t tiles = ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
    return launch_kernel(gemm_kernel<C>, dim3((unsigned)tiles), dim3(C::NT), 0, stream, xq, packed, x_scale, x_qsum,
                       w_scale, (int)M, (int)N, (int)K, y, acc);
}

using CfgLarge = GemmCfg<128, 128, 2, 2, 128>;   // wave tile 64 x 64
using CfgMid = GemmCfg<128, 64, 2, 2, 128>;      // wave tile 64 x 32
using CfgSkinny = GemmCfg<64, 16, 4, 1, 128>;    // wave tile 16 x 16

}  // namespace

hipError_t launch_gemm(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                       const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                       int64_t K, float* y, int32_t* acc, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    if (M <= 16)
        return launch_cfg<CfgSkinny>(xq, x_scale, x_qsum, packed, w_scale, M, N, K, y, acc, stream);
    if (M <= 64)
        return launch_cfg<CfgMid>(xq, x_scale, x_qsum, packed, w_scale, M, N, K, y, acc, stream);
    return launch_cfg<CfgLarge>(xq, x_scale, x_qsum, packed, w_scale, M, N, K, y, acc, stream);
}

}  // namespace bitnet
