// pack.hip - absmean ternary weight quantisation and 2-bit packing.
//
// Follows the weight rule of the Hugging Face 1.58-bit fine-tuning write-up
// ("LLM을 1.58비트로 파인튜닝", section 양자화 메커니즘: symmetric per-tensor
// scale equal to the reciprocal of the mean absolute weight; scale, round,
// clamp to [-1, 1]) and its packing of ternary weights into int8 tensors
// (section 주요 결과).  Offline: runs once per layer.
//
// Steps (each one launch, all on the caller's stream):
//   [hadamard] rows <- Walsh-Hadamard transform of the rows (float32);
//   row_abssum: r[n] = sum_k |w[n][k]| in float64, k ascending (one lane per row);
//   finalize:   S = sum_n r[n] (n ascending), gamma = S / (N K), s_w, d_w;
//   ternarize:  q = clamp(rint(w * s_w), -1, 1); 16 weights -> one 32-bit word.
// The fixed summation order makes s_w bit-identical to a sequential float64 sum.
#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

constexpr int kRowsPerWave = 64;
constexpr int kTileK = 64;
constexpr int kSumThreads = 256;

// Lane l of each wave sums row (wave_row0 + l).  The wave stages 64x64 float
// tiles through LDS (row stride 65 floats: conflict-free column reads) so the
// HBM reads stay coalesced while each lane still adds its own row in order.
__global__ __launch_bounds__(kSumThreads) void row_abssum_kernel(const float* __restrict__ src,
                                                                  int64_t N, int K,
                                                                  double* __restrict__ row_sum) {
    __shared__ float tile[kSumThreads / kWave][kRowsPerWave][kTileK + 1];
    const int lane = threadIdx.x % kWave;
    const int w = threadIdx.x / kWave;
    const int64_t row0 = ((int64_t)blockIdx.x * (kSumThreads / kWave) + w) * kRowsPerWave;
    if (row0 >= N) return;  // wave-uniform; this kernel has no workgroup barrier
    float(*T)[kTileK + 1] = tile[w];
    double acc = 0.0;
    const int sub_row = lane / 16;  // 4 rows per load instruction
    const int col4 = (lane % 16) * 4;
    for (int k0 = 0; k0 < K; k0 += kTileK) {
#pragma unroll
        for (int i = 0; i < kRowsPerWave / 4; ++i) {
            const int r = 4 * i + sub_row;
            const int64_t row = row0 + r;
            float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
            if (row < N) a = *reinterpret_cast<const float4*>(src + row * K + k0 + col4);
            T[r][col4] = a.x;
            T[r][col4 + 1] = a.y;
            T[r][col4 + 2] = a.z;
            T[r][col4 + 3] = a.w;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll 8
        for (int k = 0; k < kTileK; ++k) acc += fabs((double)T[lane][k]);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
    if (row0 + lane < N) row_sum[row0 + lane] = acc;
}

// One thread: total in row order, then the two float32 scales.
__global__ void finalize_scale_kernel(const double* __restrict__ row_sum, int64_t N, int64_t K,
                                      int hadamard, double sqrt_k, float* __restrict__ w_scale) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    double S = 0.0;
    for (int64_t n = 0; n < N; ++n) S += row_sum[n];
    const double gamma = S / ((double)N * (double)K);
    float s_w = 0.f, d_w = 0.f;
    if (gamma != 0.0) {
        s_w = (float)(1.0 / gamma);
        d_w = hadamard ? (float)(gamma / sqrt_k) : (float)gamma;
    }
    w_scale[0] = d_w;
    w_scale[1] = s_w;
}

// One thread per packed 32-bit word (16 weights).  Weight 16g + 4i + b goes to
// bits 8b + 2i of word g, as q + 1.
__global__ __launch_bounds__(256) void ternarize_pack_kernel(const float* __restrict__ src,
                                                             int64_t words,
                                                             const float* __restrict__ w_scale,
                                                             uint32_t* __restrict__ packed) {
    const float s_w = w_scale[1];
    for (int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; wi < words;
         wi += (int64_t)gridDim.x * blockDim.x) {
        // Rows are contiguous and K % 16 == 0, so word wi covers src[16 wi .. 16 wi + 15].
        const float4* s4 = reinterpret_cast<const float4*>(src + 16 * wi);
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 a = s4[i];
            v[4 * i] = a.x;
            v[4 * i + 1] = a.y;
            v[4 * i + 2] = a.z;
            v[4 * i + 3] = a.w;
        }
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = e / 4, b = e % 4;
            const int q = round_clamp(v[e] * s_w, -1.f, 1.f);
            word |= (uint32_t)(q + 1) << (8 * b + 2 * i);
        }
        packed[wi] = word;
    }
}

}  // namespace

size_t pack_workspace_bytes(int64_t N, int64_t K, int hadamard) {
    const size_t sums = ((size_t)N * sizeof(double) + 255) / 256 * 256;
    return sums + (hadamard ? (size_t)N * (size_t)K * sizeof(float) : 0);
}

hipError_t launch_pack_weights(const float* W, int64_t N, int64_t K, int hadamard, double sqrt_k,
                               uint8_t* packed, float* w_scale, void* workspace,
                               hipStream_t stream) {
    double* row_sum = reinterpret_cast<double*>(workspace);
    const float* src = W;
    if (hadamard) {
        float* rot = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                              pack_workspace_bytes(N, K, 0));
        hipError_t e = launch_fwht_rows_f32(W, rot, N, K, stream);
        if (e != hipSuccess) return e;
        src = rot;
    }
    const int64_t rows_per_block = (kSumThreads / kWave) * kRowsPerWave;
    hipLaunchKernelGGL(row_abssum_kernel, dim3((unsigned)((N + rows_per_block - 1) / rows_per_block)),
                       dim3(kSumThreads), 0, stream, src, N, (int)K, row_sum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(finalize_scale_kernel, dim3(1), dim3(64), 0, stream, row_sum, N, K,
                       hadamard, sqrt_k, w_scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t words = N * K / 16;
    const int64_t blocks = (words + 255) / 256;
    hipLaunchKernelGGL(ternarize_pack_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                       dim3(256), 0, stream, src, words, w_scale,
                       reinterpret_cast<uint32_t*>(packed));
    return hipGetLastError();
}

}  // namespace bitnet
