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

// --- activation quantisation (quant_act.hip, hadamard_quant.hip) ------------
hipError_t launch_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M, int64_t K,
                            int8_t* xq, float* x_scale, int32_t* x_qsum, hipStream_t stream);
hipError_t launch_hadamard_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M,
                                     int64_t K, double sqrt_k, int8_t* xq, float* x_scale,
                                     int32_t* x_qsum, hipStream_t stream);
// Row-wise unnormalised Walsh-Hadamard transform of float32 [N][K] (K = 2^p,
// 256 <= K <= 32768), used for the weight pre-rotation.
hipError_t launch_fwht_rows_f32(const float* src, float* dst, int64_t N, int64_t K,
                                hipStream_t stream);

// --- contraction (gemv.hip, gemm_mfma.hip) ----------------------------------
// True if the register-resident GEMV handles this (M, K).
bool gemv_supported(int64_t M, int64_t K);
hipError_t launch_gemv(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                       const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                       int64_t K, float* y, int32_t* acc, hipStream_t stream);
// Fused RMSNorm + int8 quantisation + GEMV (requires gemv_supported(M, K)).
hipError_t launch_fused_decode(const uint16_t* x, const float* gain, float eps,
                               const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                               int64_t K, float* y, int8_t* xq, float* x_scale, int32_t* x_qsum,
                               int32_t* acc, hipStream_t stream);
hipError_t launch_gemm(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                       const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                       int64_t K, float* y, int32_t* acc, hipStream_t stream);

}  // namespace bitnet
