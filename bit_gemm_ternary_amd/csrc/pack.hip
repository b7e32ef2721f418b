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
//   finalize:   S = sum_n r[n] (n ascending, one wavefront), gamma = S / (N K), s_w, d_w;
//   ternarize:  q = clamp(rint(w * s_w), -1, 1); 16 weights -> one 32-bit word.
// The fixed summation order makes s_w bit-identical to a sequential float64 sum.
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

// Library-owned scratch of bitnet_pack_weights_noalloc (row sums, and the
// rotated rows of the Hadamard path), one copy per GPU the library runs on,
// held until the process ends.  Host code never uses this name as an address:
// its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[bitnet::kNoAllocScratchBytes];

namespace bitnet {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kBufferWord3 = 0x00020000u;   // gfx9-family raw buffer descriptor word 3
constexpr int kSumCols = 64;                     // floats of each row per LDS stage (256 B)
constexpr int kSumStages = 4;                    // stage buffers: three in flight, one summed
constexpr int kSumLoads = kSumCols * 4 / 16;     // 1 KiB LDS loads per stage (4 rows each)

// Row sums in float64, k ascending: one wavefront per workgroup, lane l owns
// row 64 * blockIdx.x + l.  Each stage (64 floats of the 64 rows, 16 KiB) is
// copied from HBM into LDS by 1 KiB buffer_load ... lds instructions (four
// 256-byte row segments each, whole memory sectors), three stages in flight
// while the fourth is summed.  The 16-byte piece p of row r sits at slot
// p ^ (r & 15) of its segment, so when every lane reads the same piece of its
// own row, 16 consecutive lanes hit 16 distinct bank groups.  The order of the
// additions is the row's natural order, whatever the staging.
__global__ __launch_bounds__(kWave) void row_abssum_kernel(const float* __restrict__ src, int64_t N,
                                                          int K, double* __restrict__ row_sum) {
    __shared__ __align__(16) float tile[kSumStages][kWave * kSumCols];
    const int lane = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * kWave;
    const int rows = (int)min((int64_t)kWave, N - row0);
    // The resource covers this block's rows only: rows past N read zeros.
    const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src + row0 * K), (short)0, rows * K * (int)sizeof(float), (int)kBufferWord3);
    const int nk = K / kSumCols;
    auto issue = [&](int j) {
        float* dst = tile[j % kSumStages];
#pragma unroll
        for (int i = 0; i < kSumLoads; ++i) {
            const int r = 4 * i + lane / 16;
            const int piece = (lane % 16) ^ (r & 15);
            const int off = (r * K + j * kSumCols + 4 * piece) * (int)sizeof(float);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_void*)&dst[i * 4 * kSumCols], 16, off,
                                                     0, 0, 0);
        }
    };
    double acc = 0.0;
    auto sum = [&](int j) {
        const float* T = tile[j % kSumStages] + lane * kSumCols;
#pragma unroll
        for (int p = 0; p < kSumCols / 4; ++p) {
            // (an ext_vector read: with a float4 struct read the compiler adds a
            // wait for every outstanding LDS load before it)
            const f4 v = *reinterpret_cast<const f4*>(T + 4 * (p ^ (lane & 15)));
            acc += fabs((double)v[0]);
            acc += fabs((double)v[1]);
            acc += fabs((double)v[2]);
            acc += fabs((double)v[3]);
        }
    };
    for (int j = 0; j < kSumStages - 1 && j < nk; ++j) issue(j);
    int j = 0;
    for (; j + kSumStages - 1 < nk; ++j) {
        // Buffer (j - 1) % kSumStages was read in the previous iteration: its
        // reads have returned before the loads of stage j + 3 overwrite it.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(j + kSumStages - 1);
        // Stage j has landed once at most the three later stages' loads are
        // outstanding (loads complete in order).
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kSumStages - 1) * kSumLoads) : "memory");
        sum(j);
    }
    // The last stages (at most three), nothing more to issue.
    static_assert(kSumStages == 4, "tail below drains three stages");
    if (nk - j == 3) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kSumLoads) : "memory");
        sum(j++);
    }
    if (nk - j == 2) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSumLoads) : "memory");
        sum(j++);
    }
    if (nk - j == 1) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        sum(j);
    }
    if (lane < rows) row_sum[row0 + lane] = acc;
}

// One wavefront: S = sum of the row sums in row order, then the two float32
// scales.  The additions form one dependent chain, run by lane 0 from LDS
// (reads issued ahead of the adds, so the chain waits only on the float64 add
// latency); meanwhile the whole wave loads the next 2048 row sums into
// registers and stores them to the other LDS buffer after the chain.
constexpr int kScaleChunk = 2048;   // row sums per LDS buffer (16 KiB)

__global__ __launch_bounds__(kWave) void finalize_scale_kernel(const double* __restrict__ row_sum,
                                                               int64_t N, int64_t K, int hadamard,
                                                               double sqrt_k,
                                                               float* __restrict__ w_scale) {
    constexpr int PER_LANE = kScaleChunk / kWave;
    __shared__ double buf[2][kScaleChunk];
    const int lane = threadIdx.x;
    double nxt[PER_LANE];
    auto load = [&](int64_t c0) {
#pragma unroll
        for (int j = 0; j < PER_LANE; ++j) {
            const int64_t n = c0 + lane + kWave * j;
            nxt[j] = n < N ? row_sum[n] : 0.0;
        }
    };
    auto store = [&](int b) {
#pragma unroll
        for (int j = 0; j < PER_LANE; ++j) buf[b][lane + kWave * j] = nxt[j];
    };
    load(0);
    store(0);
    __syncthreads();
    double S = 0.0;
    for (int64_t c0 = 0; c0 < N; c0 += kScaleChunk) {
        const int b = (int)((c0 / kScaleChunk) & 1);
        const bool more = c0 + kScaleChunk < N;
        if (more) load(c0 + kScaleChunk);
        if (lane == 0) {
            const int cnt = (int)min((int64_t)kScaleChunk, N - c0);
            int i = 0;
            for (; i + 16 <= cnt; i += 16) {
#pragma unroll
                for (int e = 0; e < 16; ++e) S += buf[b][i + e];
            }
            for (; i < cnt; ++i) S += buf[b][i];
        }
        if (more) store(b ^ 1);
        __syncthreads();
    }
    if (lane != 0) return;
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

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

}  // namespace

hipError_t noalloc_scratch(int device, void** ptr) {
    if (device < 0 || device >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[device] == nullptr) {
        // The device address of this GPU's copy of the array; the caller has
        // made `device` current.
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
}

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
    hipLaunchKernelGGL(row_abssum_kernel, dim3((unsigned)((N + kWave - 1) / kWave)), dim3(kWave), 0,
                       stream, src, N, (int)K, row_sum);
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
