// dequant.hip - the dequantisation epilogue as a kernel of its own:
// y[m][n] = acc[m][n] * d_x[m] * d_w, for int32 accumulators that were formed
// elsewhere.
//
// Follows the Hugging Face 1.58-bit fine-tuning write-up ("LLM을 1.58비트로
// 파인튜닝", section 양자화 메커니즘: the integer result is rescaled by both
// scales) and the quantization primer (endplan.ai, section 그러면 크기를 더
// 못줄이나요?: dequantise by the factors).  Its use is the row-parallel shard:
// each GPU contracts a K slice into int32 partial sums, the partials are added
// exactly (an integer all-reduce), and this kernel applies the scales once, in
// the order of the contraction kernels' own epilogue ((acc * d_x) * d_w), so
// the outputs equal the unsharded ones for equal d_x.
//
// HBM-bound: 4MN bytes read, 4MN written.  Grid-stride over 4-element groups
// (16-byte loads and stores when N % 4 == 0 and the pointers are aligned).
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

template <bool VEC>
__global__ __launch_bounds__(256) void dequant_kernel(const int32_t* __restrict__ acc,
                                                      const float* __restrict__ x_scale,
                                                      const float* __restrict__ w_scale, int64_t M,
                                                      int64_t N, float* __restrict__ y) {
    const float dw = w_scale[0];
    const int64_t total = M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if constexpr (VEC) {
        const int64_t groups = total / 4;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < groups; i += stride) {
            const int64_t e = 4 * i;
            const float dx = x_scale[e / N];   // N % 4 == 0: a group stays in one token's row
            const int4 a = reinterpret_cast<const int4*>(acc)[i];
            reinterpret_cast<float4*>(y)[i] = make_float4(((float)a.x * dx) * dw, ((float)a.y * dx) * dw,
                                                          ((float)a.z * dx) * dw, ((float)a.w * dx) * dw);
        }
    } else {
        for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride)
            y[e] = ((float)acc[e] * x_scale[e / N]) * dw;
    }
}

}  // namespace

hipError_t launch_dequant(const int32_t* acc, const float* x_scale, const float* w_scale, int64_t M,
                          int64_t N, float* y, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const bool vec = N % 4 == 0 && (uintptr_t)acc % 16 == 0 && (uintptr_t)y % 16 == 0;
    const int64_t items = vec ? M * N / 4 : M * N;
    // Enough workgroups to fill the chip a few times over, at most one item per thread.
    const int64_t blocks = std::min<int64_t>((items + 255) / 256, 256 * 8);
    if (vec)
        return launch_kernel((dequant_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, stream, acc, x_scale,
                             w_scale, M, N, y);
    return launch_kernel((dequant_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, stream, acc, x_scale,
                         w_scale, M, N, y);
}

}  // namespace bitnet
