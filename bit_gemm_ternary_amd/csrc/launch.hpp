// launch.hpp - host-side launchers of the gfx950 kernels (internal interface
// between the C ABI in api.cpp and the kernel translation units).
//
// Every launcher assumes its arguments were validated by api.cpp (shapes,
// alignment, non-NULL pointers) and only enqueues work on `stream`; it returns
// the status of hipGetLastError() after its launches.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bitnet {

// Timing events armed by bitnet_set_kernel_events() for the next kernel launched
// on this thread; returns them and disarms (both NULL when none are armed).
void take_kernel_events(hipEvent_t* start, hipEvent_t* stop);

// Launch `kernel` on `stream`; when timing events are armed, through
// hipExtLaunchKernelGGL so that the events are stamped by the kernel's own
// dispatch (start and end of execution) rather than by separate markers.
template <typename F, typename... Args>
hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t stream,
                         Args... args) {
    hipEvent_t ev_start = nullptr, ev_stop = nullptr;
    take_kernel_events(&ev_start, &ev_stop);
    if (ev_start != nullptr || ev_stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, ev_start, ev_stop, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
    return hipGetLastError();
}

// --- weight quantisation / packing (pack.hip) ------------------------------
// Workspace layout: [row sums: N doubles, padded to 256 B][rotated W: N*K floats
// when hadamard].
size_t pack_workspace_bytes(int64_t N, int64_t K, int hadamard);
hipError_t launch_pack_weights(const float* W, int64_t N, int64_t K, int hadamard,
                               double sqrt_k, uint8_t* packed, float* w_scale, void* workspace,
                               hipStream_t stream);
// Bytes of the library-owned scratch that bitnet_pack_weights_noalloc uses in
// place of a workspace (one array per device, in pack.hip).
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
// Device address of that array on `device`, which must be the current device;
// looked up once per device and kept.
hipError_t noalloc_scratch(int device, void** ptr);

// --- activation quantisation (quant_act.hip, hadamard_quant.hip) ------------
hipError_t launch_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M, int64_t K,
                            int8_t* xq, float* x_scale, int32_t* x_qsum, hipStream_t stream);
// Row-parallel shards (quant_act.hip): per token, the absmax of x * gain and
// the float64 sum of x^2 over this K slice; then the codes of the slice from
// the whole token's absmax and sum of squares (after the cross-shard maximum
// and sum), d_x with the mean over k_total values, and the slice's code sum.
hipError_t launch_token_stats(const uint16_t* x, const float* gain, int64_t M, int64_t K, float* amax,
                              double* sumsq, hipStream_t stream);
hipError_t launch_quant_act_with_stats(const uint16_t* x, const float* gain, float eps, int64_t M,
                                       int64_t K, int64_t k_total, const float* amax,
                                       const double* sumsq, int8_t* xq, float* x_scale,
                                       int32_t* x_qsum, hipStream_t stream);
// y = acc * d_x[m] * d_w for int32 accumulators [M][N] (dequant.hip).
hipError_t launch_dequant(const int32_t* acc, const float* x_scale, const float* w_scale, int64_t M,
                          int64_t N, float* y, hipStream_t stream);
hipError_t launch_hadamard_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M,
                                     int64_t K, double sqrt_k, int8_t* xq, float* x_scale,
                                     int32_t* x_qsum, hipStream_t stream);
// The same codes written as 6-bit E3M2 floats, 24 bytes per 32 values
// (xq6: [M][K / 4 * 3] bytes), in the order the FP4 x FP6 contraction reads.
hipError_t launch_hadamard_quant_act_f6(const uint16_t* x, const float* gain, float eps,
                                        int64_t M, int64_t K, double sqrt_k, uint8_t* xq6,
                                        float* x_scale, int32_t* x_qsum, hipStream_t stream);
// The same codes as packed 4-bit two's complement, two per byte
// (xq4: [M][K / 2] bytes; byte 8g + j holds code 16g + j in its low nibble and
// code 16g + 8 + j in its high nibble).
hipError_t launch_hadamard_quant_act_i4(const uint16_t* x, const float* gain, float eps,
                                        int64_t M, int64_t K, double sqrt_k, uint8_t* xq4,
                                        float* x_scale, int32_t* x_qsum, hipStream_t stream);
// One token through the H-BitLinear layer in one launch (hadamard_decode.hip):
// the codes of launch_hadamard_quant_act_i4 (xq4 [K/2], x_scale, x_qsum,
// written by the first workgroup) and the contraction of launch_gemv_i4 with
// one weight group (y, acc [N]).  K a power of two in [1024, 16384] and
// ceil(N / V) * ceil(K / 4096) <= 16 for N >= 1, with V = 1024 waves up to
// K = 4096 and 2048 above; hipErrorNotSupported outside that domain
// (hadamard_decode_supported), launching nothing.
bool hadamard_decode_supported(int64_t N, int64_t K);
hipError_t launch_hadamard_decode(const uint16_t* x, const float* gain, float eps, double sqrt_k,
                                  const uint8_t* packed, const float* w_scale, int64_t N, int64_t K,
                                  float* y, uint8_t* xq4, float* x_scale, int32_t* x_qsum,
                                  int32_t* acc, hipStream_t stream);
// Row-wise unnormalised Walsh-Hadamard transform of float32 [N][K] (K = 2^p,
// 256 <= K <= 32768), used for the weight pre-rotation.
hipError_t launch_fwht_rows_f32(const float* src, float* dst, int64_t N, int64_t K,
                                hipStream_t stream);

// --- contraction (gemv.hip, gemm_mfma.hip) ----------------------------------
// Dequantisation multipliers of the weight rows: one (d_w, s_w) pair per group
// of consecutive rows.  A single matrix is one group; projections that share
// their input (q|k|v, gate|up) are stacked row-wise as several groups and
// contracted in one launch.
constexpr int kMaxRowGroups = 8;
struct RowScales {
    const float* w_scale;          // device [groups][2]: (d_w, s_w) per group
    int groups;                    // 1 .. kMaxRowGroups
    int64_t end[kMaxRowGroups];    // exclusive last row of each group; end[groups-1] = N

    // d_w of weight row n (0 <= n < N); dw0 = w_scale[0], loaded once by the
    // caller before it stores anything (the outputs may not be assumed apart
    // from w_scale, so a load here would be repeated after every store).
    __device__ __forceinline__ float of(int64_t n, float dw0) const {
        if (groups == 1) return dw0;
        int g = 0;
#pragma unroll
        for (int i = 0; i < kMaxRowGroups - 1; ++i) g += (i < groups - 1 && n >= end[i]) ? 1 : 0;
        return w_scale[2 * g];
    }
};

inline RowScales single_group(const float* w_scale, int64_t N) {
    RowScales r{};
    r.w_scale = w_scale;
    r.groups = 1;
    r.end[0] = N;
    return r;
}

// True if the register-resident GEMV handles this (M, K).
bool gemv_supported(int64_t M, int64_t K);
hipError_t launch_gemv(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                       const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                       int64_t K, float* y, int32_t* acc, hipStream_t stream);
// Fused RMSNorm + int8 quantisation + GEMV (requires gemv_supported(M, K)).
hipError_t launch_fused_decode(const uint16_t* x, const float* gain, float eps,
                               const uint8_t* packed, const RowScales& scales, int64_t M,
                               int64_t N, int64_t K, float* y, int8_t* xq, float* x_scale,
                               int32_t* x_qsum, int32_t* acc, hipStream_t stream);
hipError_t launch_gemm(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                       const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                       int64_t K, float* y, int32_t* acc, hipStream_t stream);
// The contraction with packed 4-bit codes (launch_hadamard_quant_act_i4
// layout): the register-resident GEMV on v_dot8_i32_i4 when gemv_supported(M,
// K), and the int8 matrix-core tiles (codes expanded to 16 q) for any M.
hipError_t launch_gemv_i4(const uint8_t* xq4, const float* x_scale, const int32_t* x_qsum,
                          const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                          int64_t K, float* y, int32_t* acc, hipStream_t stream);
hipError_t launch_gemm_i4(const uint8_t* xq4, const float* x_scale, const int32_t* x_qsum,
                          const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                          int64_t K, float* y, int32_t* acc, hipStream_t stream);
// The contraction with 6-bit E3M2 activation codes (bitnet_hadamard_quant_act_f6
// layout) on the FP4 x FP6 matrix core; any M.
hipError_t launch_gemm_f6(const uint8_t* xq6, const float* x_scale, const int32_t* x_qsum,
                          const uint8_t* packed, const RowScales& scales, int64_t M, int64_t N,
                          int64_t K, float* y, int32_t* acc, hipStream_t stream);

// --- backward under the straight-through estimator (backward.hip) --------
// p[0 .. count) = 0 by a kernel (no memset node if the caller captures a graph).
hipError_t launch_zero_f32(float* p, int64_t count, hipStream_t stream);

// Base-3 packing (five ternary weights per byte) and its one-token GEMV.
constexpr int kBase3MaxChunks = 4;  // 16-byte chunks per lane: K <= 4 * 64 * 80 = 20480
int64_t base3_row_bytes(int64_t K);
bool base3_gemv_supported(int64_t K);
hipError_t launch_pack_base3(const uint8_t* packed, int64_t N, int64_t K, uint8_t* packed3, hipStream_t stream);
hipError_t launch_base3_gemv(const int8_t* xq, const float* x_scale, const int32_t* x_qsum, const uint8_t* packed3,
                             const float* w_scale, int64_t N, int64_t K, float* y, int32_t* acc,
                             hipStream_t stream);
// packed [N][K/4] -> packed_t [K][N/4] (N, K multiples of 64).
hipError_t launch_transpose_packed(const uint8_t* packed, int64_t N, int64_t K, uint8_t* packed_t,
                                   hipStream_t stream);
// grad_n [M][K] = d_w * grad_y (bf16 [M][N]) @ q_w, with q_w read from packed_t.
hipError_t launch_backward_input(const uint16_t* grad_y, const uint8_t* packed_t, const float* w_scale,
                                 int64_t M, int64_t N, int64_t K, float* grad_n, hipStream_t stream);
// grad_w [N][K] = sum_m grad_y[m][n] d_x[m] q_x[m][k]; workspace of
// backward_weight_workspace_bytes(M, N, K) bytes, 16-byte aligned.
size_t backward_weight_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_backward_weight(const uint16_t* grad_y, const int8_t* xq, const float* x_scale,
                                  int64_t M, int64_t N, int64_t K, float* grad_w, void* workspace,
                                  hipStream_t stream);
// RMSNorm backward: grad_x [M][K], optional grad_gain [K] (workspace of
// rmsnorm_backward_workspace_bytes(M, K) bytes when grad_gain is requested).
size_t rmsnorm_backward_workspace_bytes(int64_t M, int64_t K);
hipError_t launch_rmsnorm_backward(const uint16_t* x, const float* gain, float eps, const float* grad_n,
                                   int64_t M, int64_t K, float* grad_x, float* grad_gain, void* workspace,
                                   hipStream_t stream);

// The layer at warm-up blend factor lambda (blend.hip): workspace of
// blend_workspace_bytes(M, K) bytes, 16-byte aligned (blended activations,
// int8 codes, scales and sums).
size_t blend_workspace_bytes(int64_t M, int64_t K);
hipError_t launch_linear_forward_blend(const uint16_t* x, const float* gain, float eps, const float* W,
                                       const uint8_t* packed, const float* w_scale, float lambda, int64_t M,
                                       int64_t N, int64_t K, float* y, void* workspace, hipStream_t stream);

// Plain read of `bytes` bytes (a multiple of 16) of device memory; a word is
// written to sink only on a data pattern that does not occur in practice.
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace bitnet
