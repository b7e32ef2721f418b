// api.cpp - the C ABI declared in include/bitnet.h: argument validation (before
// any HIP call), kernel selection and launch on the caller's stream, and
// thread-local error reporting.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>

#include "../../include/bitnet.h"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

// Disarms the timing events when an entry point returns, launched or not.
struct DisarmEvents {
    ~DisarmEvents() { g_ev_start = g_ev_stop = nullptr; }
};

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return BITNET_OK;
    return fail(BITNET_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kMaxRows = 2147483647;  // 2^31 - 1
constexpr int64_t kMinK = 64, kMaxK = 65536;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int check_k(int64_t K, const char* fn) {
    if (K < kMinK || K > kMaxK || K % 64 != 0)
        return fail(BITNET_ERR_SHAPE, "%s: K=%lld must be a multiple of 64 in [64, 65536]", fn,
                    (long long)K);
    return BITNET_OK;
}

int check_hadamard_k(int64_t K, const char* fn) {
    if (!is_pow2(K) || K < 256 || K > 32768)
        return fail(BITNET_ERR_UNSUPPORTED,
                    "%s: the Hadamard transform needs K a power of two in [256, 32768], got %lld",
                    fn, (long long)K);
    return BITNET_OK;
}

int check_eps(float eps, const char* fn) {
    if (!std::isfinite(eps) || eps < 0.f)
        return fail(BITNET_ERR_VALUE, "%s: eps must be finite and >= 0", fn);
    return BITNET_OK;
}

int validate_quant(const uint16_t* x, const float* gain, float eps, int64_t M, int64_t K,
                   int8_t* xq, float* x_scale, int32_t* x_qsum, bool hadamard, const char* fn) {
    if (M < 0 || M > kMaxRows) return fail(BITNET_ERR_SHAPE, "%s: M=%lld out of range", fn, (long long)M);
    int s = check_k(K, fn);
    if (s != BITNET_OK) return s;
    if (hadamard && (s = check_hadamard_k(K, fn)) != BITNET_OK) return s;
    if ((s = check_eps(eps, fn)) != BITNET_OK) return s;
    if (M == 0) return BITNET_OK;
    if (!x || !xq || !x_scale || !x_qsum)
        return fail(BITNET_ERR_NULL, "%s: x, xq, x_scale and x_qsum must not be NULL", fn);
    if (!aligned(x, 16) || !aligned(xq, 16) || (gain && !aligned(gain, 16)))
        return fail(BITNET_ERR_ALIGN, "%s: x, xq and gain must be 16-byte aligned", fn);
    if (!aligned(x_scale, 4) || !aligned(x_qsum, 4))
        return fail(BITNET_ERR_ALIGN, "%s: x_scale and x_qsum must be 4-byte aligned", fn);
    return BITNET_OK;
}

}  // namespace

namespace bitnet {
void take_kernel_events(hipEvent_t* start, hipEvent_t* stop) {
    *start = g_ev_start;
    *stop = g_ev_stop;
    g_ev_start = g_ev_stop = nullptr;
}
}  // namespace bitnet

extern "C" {

int bitnet_set_kernel_events(void* start_event, void* stop_event) {
    g_ev_start = (hipEvent_t)start_event;
    g_ev_stop = (hipEvent_t)stop_event;
    return BITNET_OK;
}

size_t bitnet_pack_weights_workspace_bytes(int64_t N, int64_t K, int hadamard) {
    if (N < 1 || N > kMaxRows || K < kMinK || K > kMaxK) return 0;
    return bitnet::pack_workspace_bytes(N, K, hadamard ? 1 : 0);
}

int bitnet_pack_weights(const float* W, int64_t N, int64_t K, int hadamard, uint8_t* packed,
                        float* w_scale, void* workspace, size_t workspace_bytes, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_pack_weights";
    if (N < 1 || N > kMaxRows) return fail(BITNET_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
    int s = check_k(K, fn);
    if (s != BITNET_OK) return s;
    if (hadamard != 0 && hadamard != 1) return fail(BITNET_ERR_VALUE, "%s: hadamard must be 0 or 1", fn);
    if (hadamard && (s = check_hadamard_k(K, fn)) != BITNET_OK) return s;
    if (!W || !packed || !w_scale || !workspace)
        return fail(BITNET_ERR_NULL, "%s: W, packed, w_scale and workspace must not be NULL", fn);
    if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(workspace, 16) || !aligned(w_scale, 4))
        return fail(BITNET_ERR_ALIGN, "%s: W, packed and workspace must be 16-byte aligned", fn);
    const size_t need = bitnet::pack_workspace_bytes(N, K, hadamard);
    if (workspace_bytes < need)
        return fail(BITNET_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn,
                    workspace_bytes, need);
    const double sqrt_k = std::sqrt((double)K);
    return hip_status(bitnet::launch_pack_weights(W, N, K, hadamard, sqrt_k, packed, w_scale,
                                                  workspace, (hipStream_t)stream),
                      fn);
}

static_assert(BITNET_NOALLOC_SCRATCH_BYTES == bitnet::kNoAllocScratchBytes,
              "the header's scratch size is the library's");

int bitnet_pack_weights_noalloc(const float* W, int64_t N, int64_t K, int hadamard, uint8_t* packed,
                                float* w_scale, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_pack_weights_noalloc";
    if (N < 1 || N > kMaxRows) return fail(BITNET_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
    int s = check_k(K, fn);
    if (s != BITNET_OK) return s;
    if (hadamard != 0 && hadamard != 1) return fail(BITNET_ERR_VALUE, "%s: hadamard must be 0 or 1", fn);
    if (hadamard && (s = check_hadamard_k(K, fn)) != BITNET_OK) return s;
    if (!W || !packed || !w_scale)
        return fail(BITNET_ERR_NULL, "%s: W, packed and w_scale must not be NULL", fn);
    if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(w_scale, 4))
        return fail(BITNET_ERR_ALIGN, "%s: W and packed must be 16-byte aligned", fn);
    const size_t need = bitnet::pack_workspace_bytes(N, K, hadamard);
    if (need > bitnet::kNoAllocScratchBytes)
        return fail(BITNET_ERR_WORKSPACE,
                    "%s: N=%lld K=%lld hadamard=%d needs %zu bytes of scratch; the library's static "
                    "scratch holds %zu (use bitnet_pack_weights with a workspace)",
                    fn, (long long)N, (long long)K, hadamard, need, bitnet::kNoAllocScratchBytes);
    int device = -1;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return hip_status(e, fn);
    if (stream != nullptr) {
        int stream_device = -1;
        e = hipStreamGetDevice((hipStream_t)stream, &stream_device);
        if (e != hipSuccess) return hip_status(e, fn);
        if (stream_device != device)
            return fail(BITNET_ERR_VALUE, "%s: the stream belongs to device %d, the current device is %d",
                        fn, stream_device, device);
    }
    void* scratch = nullptr;
    e = bitnet::noalloc_scratch(device, &scratch);
    if (e != hipSuccess) return hip_status(e, fn);
    return hip_status(bitnet::launch_pack_weights(W, N, K, hadamard, std::sqrt((double)K), packed, w_scale,
                                                  scratch, (hipStream_t)stream),
                      fn);
}

int bitnet_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M, int64_t K,
                     int8_t* xq, float* x_scale, int32_t* x_qsum, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_quant_act";
    int s = validate_quant(x, gain, eps, M, K, xq, x_scale, x_qsum, false, fn);
    if (s != BITNET_OK || M == 0) return s;
    return hip_status(bitnet::launch_quant_act(x, gain, eps, M, K, xq, x_scale, x_qsum,
                                               (hipStream_t)stream),
                      fn);
}

int bitnet_hadamard_quant_act(const uint16_t* x, const float* gain, float eps, int64_t M,
                              int64_t K, int8_t* xq, float* x_scale, int32_t* x_qsum,
                              void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_hadamard_quant_act";
    int s = validate_quant(x, gain, eps, M, K, xq, x_scale, x_qsum, true, fn);
    if (s != BITNET_OK || M == 0) return s;
    return hip_status(bitnet::launch_hadamard_quant_act(x, gain, eps, M, K, std::sqrt((double)K), xq,
                                                        x_scale, x_qsum, (hipStream_t)stream),
                      fn);
}

int bitnet_hadamard_quant_act_f6(const uint16_t* x, const float* gain, float eps, int64_t M,
                                 int64_t K, uint8_t* xq6, float* x_scale, int32_t* x_qsum,
                                 void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_hadamard_quant_act_f6";
    int s = validate_quant(x, gain, eps, M, K, reinterpret_cast<int8_t*>(xq6), x_scale, x_qsum,
                           true, fn);
    if (s != BITNET_OK || M == 0) return s;
    return hip_status(bitnet::launch_hadamard_quant_act_f6(x, gain, eps, M, K, std::sqrt((double)K),
                                                           xq6, x_scale, x_qsum,
                                                           (hipStream_t)stream),
                      fn);
}

int bitnet_hadamard_quant_act_i4(const uint16_t* x, const float* gain, float eps, int64_t M,
                                 int64_t K, uint8_t* xq4, float* x_scale, int32_t* x_qsum,
                                 void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_hadamard_quant_act_i4";
    int s = validate_quant(x, gain, eps, M, K, reinterpret_cast<int8_t*>(xq4), x_scale, x_qsum,
                           true, fn);
    if (s != BITNET_OK || M == 0) return s;
    return hip_status(bitnet::launch_hadamard_quant_act_i4(x, gain, eps, M, K, std::sqrt((double)K),
                                                           xq4, x_scale, x_qsum,
                                                           (hipStream_t)stream),
                      fn);
}

int bitnet_linear_forward_i4(const uint8_t* xq4, const float* x_scale, const int32_t* x_qsum,
                             const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                             int64_t K, float* y, int32_t* acc, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_linear_forward_i4";
    if (M < 0 || M > kMaxRows || N < 0 || N > kMaxRows)
        return fail(BITNET_ERR_SHAPE, "%s: M=%lld or N=%lld out of range", fn, (long long)M, (long long)N);
    int s = check_k(K, fn);
    if (s != BITNET_OK) return s;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!xq4 || !x_scale || !x_qsum || !packed || !w_scale || !y)
        return fail(BITNET_ERR_NULL, "%s: only acc may be NULL", fn);
    if (!aligned(xq4, 16) || !aligned(packed, 16))
        return fail(BITNET_ERR_ALIGN, "%s: xq4 and packed must be 16-byte aligned", fn);
    if (!aligned(x_scale, 4) || !aligned(x_qsum, 4) || !aligned(w_scale, 4) || !aligned(y, 4) ||
        (acc && !aligned(acc, 4)))
        return fail(BITNET_ERR_ALIGN, "%s: scales, sums, y and acc must be 4-byte aligned", fn);
    hipStream_t st = (hipStream_t)stream;
    const bitnet::RowScales scales = bitnet::single_group(w_scale, N);
    hipError_t e = bitnet::gemv_supported(M, K)
                       ? bitnet::launch_gemv_i4(xq4, x_scale, x_qsum, packed, scales, M, N, K, y, acc, st)
                       : bitnet::launch_gemm_i4(xq4, x_scale, x_qsum, packed, scales, M, N, K, y, acc, st);
    return hip_status(e, fn);
}

int bitnet_linear_forward_f6(const uint8_t* xq6, const float* x_scale, const int32_t* x_qsum,
                             const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                             int64_t K, float* y, int32_t* acc, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_linear_forward_f6";
    if (M < 0 || M > kMaxRows || N < 0 || N > kMaxRows)
        return fail(BITNET_ERR_SHAPE, "%s: M=%lld or N=%lld out of range", fn, (long long)M, (long long)N);
    int s = check_k(K, fn);
    if (s != BITNET_OK) return s;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!xq6 || !x_scale || !x_qsum || !packed || !w_scale || !y)
        return fail(BITNET_ERR_NULL, "%s: only acc may be NULL", fn);
    if (!aligned(xq6, 16) || !aligned(packed, 16))
        return fail(BITNET_ERR_ALIGN, "%s: xq6 and packed must be 16-byte aligned", fn);
    if (!aligned(x_scale, 4) || !aligned(x_qsum, 4) || !aligned(w_scale, 4) || !aligned(y, 4) ||
        (acc && !aligned(acc, 4)))
        return fail(BITNET_ERR_ALIGN, "%s: scales, sums, y and acc must be 4-byte aligned", fn);
    return hip_status(bitnet::launch_gemm_f6(xq6, x_scale, x_qsum, packed,
                                             bitnet::single_group(w_scale, N), M, N, K, y, acc,
                                             (hipStream_t)stream),
                      fn);
}

int bitnet_linear_forward(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                          const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                          int64_t K, float* y, int32_t* acc, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_linear_forward";
    if (M < 0 || M > kMaxRows || N < 0 || N > kMaxRows)
        return fail(BITNET_ERR_SHAPE, "%s: M=%lld or N=%lld out of range", fn, (long long)M, (long long)N);
    int s = check_k(K, fn);
    if (s != BITNET_OK) return s;
    if (M == 0 || N == 0) return BITNET_OK;
    if (!xq || !x_scale || !x_qsum || !packed || !w_scale || !y)
        return fail(BITNET_ERR_NULL, "%s: only acc may be NULL", fn);
    if (!aligned(xq, 16) || !aligned(packed, 16))
        return fail(BITNET_ERR_ALIGN, "%s: xq and packed must be 16-byte aligned", fn);
    if (!aligned(x_scale, 4) || !aligned(x_qsum, 4) || !aligned(w_scale, 4) || !aligned(y, 4) ||
        (acc && !aligned(acc, 4)))
        return fail(BITNET_ERR_ALIGN, "%s: scales, sums, y and acc must be 4-byte aligned", fn);
    hipStream_t st = (hipStream_t)stream;
    const bitnet::RowScales scales = bitnet::single_group(w_scale, N);
    hipError_t e = bitnet::gemv_supported(M, K)
                       ? bitnet::launch_gemv(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, st)
                       : bitnet::launch_gemm(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, st);
    return hip_status(e, fn);
}

namespace {

// Quantise x once, then contract it with every row group of `packed`.
int bitlinear_forward_rows(const uint16_t* x, const float* gain, float eps, const uint8_t* packed,
                           const bitnet::RowScales& scales, int64_t M, int64_t N, int64_t K,
                           int8_t* xq, float* x_scale, int32_t* x_qsum, float* y, int32_t* acc,
                           hipStream_t st, const char* fn) {
    if (bitnet::gemv_supported(M, K))
        return hip_status(bitnet::launch_fused_decode(x, gain, eps, packed, scales, M, N, K, y, xq,
                                                      x_scale, x_qsum, acc, st),
                          fn);
    hipError_t e = bitnet::launch_quant_act(x, gain, eps, M, K, xq, x_scale, x_qsum, st);
    if (e == hipSuccess)
        e = bitnet::launch_gemm(xq, x_scale, x_qsum, packed, scales, M, N, K, y, acc, st);
    return hip_status(e, fn);
}

}  // namespace

int bitnet_bitlinear_forward(const uint16_t* x, const float* gain, float eps,
                             const uint8_t* packed, const float* w_scale, int64_t M, int64_t N,
                             int64_t K, int8_t* xq, float* x_scale, int32_t* x_qsum, float* y,
                             int32_t* acc, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_bitlinear_forward";
    int s = validate_quant(x, gain, eps, M, K, xq, x_scale, x_qsum, false, fn);
    if (s != BITNET_OK) return s;
    if (N < 0 || N > kMaxRows) return fail(BITNET_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
    if (M == 0) return BITNET_OK;
    hipStream_t st = (hipStream_t)stream;
    if (N == 0)
        return hip_status(bitnet::launch_quant_act(x, gain, eps, M, K, xq, x_scale, x_qsum, st), fn);
    if (!packed || !w_scale || !y) return fail(BITNET_ERR_NULL, "%s: packed, w_scale and y must not be NULL", fn);
    if (!aligned(packed, 16)) return fail(BITNET_ERR_ALIGN, "%s: packed must be 16-byte aligned", fn);
    if (!aligned(w_scale, 4) || !aligned(y, 4) || (acc && !aligned(acc, 4)))
        return fail(BITNET_ERR_ALIGN, "%s: w_scale, y and acc must be 4-byte aligned", fn);
    return bitlinear_forward_rows(x, gain, eps, packed, bitnet::single_group(w_scale, N), M, N, K,
                                  xq, x_scale, x_qsum, y, acc, st, fn);
}

int bitnet_hadamard_bitlinear_forward(const uint16_t* x, const float* gain, float eps,
                                      const uint8_t* packed, const float* w_scale, int64_t M,
                                      int64_t N, int64_t K, uint8_t* xq4, float* x_scale,
                                      int32_t* x_qsum, float* y, int32_t* acc, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_hadamard_bitlinear_forward";
    int s = validate_quant(x, gain, eps, M, K, reinterpret_cast<int8_t*>(xq4), x_scale, x_qsum, true, fn);
    if (s != BITNET_OK) return s;
    if (N < 0 || N > kMaxRows) return fail(BITNET_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
    if (M == 0) return BITNET_OK;
    hipStream_t st = (hipStream_t)stream;
    const double sqrt_k = std::sqrt((double)K);
    if (N == 0)
        return hip_status(bitnet::launch_hadamard_quant_act_i4(x, gain, eps, M, K, sqrt_k, xq4, x_scale,
                                                               x_qsum, st),
                          fn);
    if (!packed || !w_scale || !y) return fail(BITNET_ERR_NULL, "%s: packed, w_scale and y must not be NULL", fn);
    if (!aligned(packed, 16)) return fail(BITNET_ERR_ALIGN, "%s: packed must be 16-byte aligned", fn);
    if (!aligned(w_scale, 4) || !aligned(y, 4) || (acc && !aligned(acc, 4)))
        return fail(BITNET_ERR_ALIGN, "%s: w_scale, y and acc must be 4-byte aligned", fn);
    if (M == 1 && bitnet::hadamard_decode_supported(N, K))
        return hip_status(bitnet::launch_hadamard_decode(x, gain, eps, sqrt_k, packed, w_scale, N, K, y, xq4,
                                                         x_scale, x_qsum, acc, st),
                          fn);
    hipError_t e = bitnet::launch_hadamard_quant_act_i4(x, gain, eps, M, K, sqrt_k, xq4, x_scale, x_qsum, st);
    if (e == hipSuccess) {
        const bitnet::RowScales scales = bitnet::single_group(w_scale, N);
        e = bitnet::gemv_supported(M, K)
                ? bitnet::launch_gemv_i4(xq4, x_scale, x_qsum, packed, scales, M, N, K, y, acc, st)
                : bitnet::launch_gemm_i4(xq4, x_scale, x_qsum, packed, scales, M, N, K, y, acc, st);
    }
    return hip_status(e, fn);
}

int bitnet_token_stats(const uint16_t* x, const float* gain, int64_t M, int64_t K, float* amax,
                       double* sumsq, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_token_stats";
    if (M < 0 || M > kMaxRows) return fail(BITNET_ERR_SHAPE, "%s: M=%lld out of range", fn, (long long)M);
    int s = check_k(K, fn);
    if (s != BITNET_OK || M == 0) return s;
    if (!x || !amax || !sumsq) return fail(BITNET_ERR_NULL, "%s: x, amax and sumsq must not be NULL", fn);
    if (!aligned(x, 16) || (gain && !aligned(gain, 16)))
        return fail(BITNET_ERR_ALIGN, "%s: x and gain must be 16-byte aligned", fn);
    if (!aligned(amax, 4) || !aligned(sumsq, 8))
        return fail(BITNET_ERR_ALIGN, "%s: amax must be 4-byte and sumsq 8-byte aligned", fn);
    return hip_status(bitnet::launch_token_stats(x, gain, M, K, amax, sumsq, (hipStream_t)stream), fn);
}

int bitnet_quant_act_with_stats(const uint16_t* x, const float* gain, float eps, int64_t M,
                                int64_t K, int64_t K_total, const float* amax, const double* sumsq,
                                int8_t* xq, float* x_scale, int32_t* x_qsum, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_quant_act_with_stats";
    int s = validate_quant(x, gain, eps, M, K, xq, x_scale, x_qsum, false, fn);
    if (s != BITNET_OK) return s;
    if (K_total < K || K_total > (int64_t{1} << 24))
        return fail(BITNET_ERR_SHAPE, "%s: K_total=%lld must lie in [K, 2^24]", fn, (long long)K_total);
    if (M == 0) return BITNET_OK;
    if (!amax || !sumsq) return fail(BITNET_ERR_NULL, "%s: amax and sumsq must not be NULL", fn);
    if (!aligned(amax, 4) || !aligned(sumsq, 8))
        return fail(BITNET_ERR_ALIGN, "%s: amax must be 4-byte and sumsq 8-byte aligned", fn);
    return hip_status(bitnet::launch_quant_act_with_stats(x, gain, eps, M, K, K_total, amax, sumsq, xq, x_scale,
                                                          x_qsum, (hipStream_t)stream),
                      fn);
}

int bitnet_dequant(const int32_t* acc, const float* x_scale, const float* w_scale, int64_t M, int64_t N,
                   float* y, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_dequant";
    if (M < 0 || M > kMaxRows || N < 0 || N > kMaxRows)
        return fail(BITNET_ERR_SHAPE, "%s: M=%lld or N=%lld out of range", fn, (long long)M, (long long)N);
    if (M == 0 || N == 0) return BITNET_OK;
    if (!acc || !x_scale || !w_scale || !y) return fail(BITNET_ERR_NULL, "%s: no argument may be NULL", fn);
    if (!aligned(acc, 4) || !aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(y, 4))
        return fail(BITNET_ERR_ALIGN, "%s: acc, x_scale, w_scale and y must be 4-byte aligned", fn);
    return hip_status(bitnet::launch_dequant(acc, x_scale, w_scale, M, N, y, (hipStream_t)stream), fn);
}

int bitnet_bitlinear_forward_grouped(const uint16_t* x, const float* gain, float eps,
                                     const uint8_t* packed, const float* w_scales,
                                     const int64_t* group_rows, int groups, int64_t M, int64_t K,
                                     int8_t* xq, float* x_scale, int32_t* x_qsum, float* y,
                                     int32_t* acc, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_bitlinear_forward_grouped";
    int s = validate_quant(x, gain, eps, M, K, xq, x_scale, x_qsum, false, fn);
    if (s != BITNET_OK) return s;
    if (groups < 1 || groups > bitnet::kMaxRowGroups)
        return fail(BITNET_ERR_SHAPE, "%s: groups=%d must be in [1, %d]", fn, groups,
                    bitnet::kMaxRowGroups);
    if (!group_rows) return fail(BITNET_ERR_NULL, "%s: group_rows must not be NULL", fn);
    bitnet::RowScales scales{};
    scales.w_scale = w_scales;
    scales.groups = groups;
    int64_t N = 0;
    for (int g = 0; g < groups; ++g) {
        if (group_rows[g] < 1 || group_rows[g] > kMaxRows - N)
            return fail(BITNET_ERR_SHAPE, "%s: group %d has %lld rows (each group needs >= 1, total <= 2^31-1)",
                        fn, g, (long long)group_rows[g]);
        N += group_rows[g];
        scales.end[g] = N;
    }
    if (M == 0) return BITNET_OK;
    if (!packed || !w_scales || !y)
        return fail(BITNET_ERR_NULL, "%s: packed, w_scales and y must not be NULL", fn);
    if (!aligned(packed, 16)) return fail(BITNET_ERR_ALIGN, "%s: packed must be 16-byte aligned", fn);
    if (!aligned(w_scales, 4) || !aligned(y, 4) || (acc && !aligned(acc, 4)))
        return fail(BITNET_ERR_ALIGN, "%s: w_scales, y and acc must be 4-byte aligned", fn);
    return bitlinear_forward_rows(x, gain, eps, packed, scales, M, N, K, xq, x_scale, x_qsum, y,
                                  acc, (hipStream_t)stream, fn);
}

namespace {

// Backward shapes: N and K multiples of 64 (whole 64 x 64 transpose tiles and
// 64-value reduction stages), M any token count.
int check_backward_nk(int64_t N, int64_t K, const char* fn) {
    int s = check_k(K, fn);
    if (s != BITNET_OK) return s;
    if (N < 64 || N > kMaxK || N % 64 != 0)
        return fail(BITNET_ERR_SHAPE, "%s: N=%lld must be a multiple of 64 in [64, 65536]", fn,
                    (long long)N);
    return BITNET_OK;
}

}  // namespace

int bitnet_transpose_packed(const uint8_t* packed, int64_t N, int64_t K, uint8_t* packed_t,
                            void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_transpose_packed";
    int s = check_backward_nk(N, K, fn);
    if (s != BITNET_OK) return s;
    if (!packed || !packed_t) return fail(BITNET_ERR_NULL, "%s: packed and packed_t must not be NULL", fn);
    if (!aligned(packed, 16) || !aligned(packed_t, 16))
        return fail(BITNET_ERR_ALIGN, "%s: packed and packed_t must be 16-byte aligned", fn);
    return hip_status(bitnet::launch_transpose_packed(packed, N, K, packed_t, (hipStream_t)stream), fn);
}

int bitnet_linear_backward_input(const uint16_t* grad_y, const uint8_t* packed_t, const float* w_scale,
                                 int64_t M, int64_t N, int64_t K, float* grad_n, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_linear_backward_input";
    if (M < 0 || M > kMaxRows) return fail(BITNET_ERR_SHAPE, "%s: M=%lld out of range", fn, (long long)M);
    int s = check_backward_nk(N, K, fn);
    if (s != BITNET_OK) return s;
    if (M == 0) return BITNET_OK;
    if (!grad_y || !packed_t || !w_scale || !grad_n)
        return fail(BITNET_ERR_NULL, "%s: no pointer may be NULL", fn);
    if (!aligned(grad_y, 16) || !aligned(packed_t, 16))
        return fail(BITNET_ERR_ALIGN, "%s: grad_y and packed_t must be 16-byte aligned", fn);
    if (!aligned(w_scale, 4) || !aligned(grad_n, 4))
        return fail(BITNET_ERR_ALIGN, "%s: w_scale and grad_n must be 4-byte aligned", fn);
    return hip_status(bitnet::launch_backward_input(grad_y, packed_t, w_scale, M, N, K, grad_n,
                                                    (hipStream_t)stream),
                      fn);
}

// dL/dW contracts over the tokens with operand rows of 2 M bf16 values; up to
// 2^21 tokens a 128-row tile of them spans at most 2^30 bytes.
constexpr int64_t kMaxBackwardWeightRows = int64_t(1) << 21;

size_t bitnet_linear_backward_weight_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || M > kMaxBackwardWeightRows || N < 64 || N > kMaxK || N % 64 != 0 || K < kMinK || K > kMaxK ||
        K % 64 != 0)
        return 0;
    return bitnet::backward_weight_workspace_bytes(M, N, K);
}

int bitnet_linear_backward_weight(const uint16_t* grad_y, const int8_t* xq, const float* x_scale,
                                  int64_t M, int64_t N, int64_t K, float* grad_w, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_linear_backward_weight";
    if (M < 0 || M > kMaxBackwardWeightRows)
        return fail(BITNET_ERR_SHAPE, "%s: M=%lld out of range [0, 2^21]", fn, (long long)M);
    int s = check_backward_nk(N, K, fn);
    if (s != BITNET_OK) return s;
    if (!grad_w) return fail(BITNET_ERR_NULL, "%s: grad_w must not be NULL", fn);
    if (!aligned(grad_w, 4)) return fail(BITNET_ERR_ALIGN, "%s: grad_w must be 4-byte aligned", fn);
    if (M == 0) {  // an empty sum: zero gradient
        return hip_status(bitnet::launch_zero_f32(grad_w, N * K, (hipStream_t)stream), fn);
    }
    if (!grad_y || !xq || !x_scale) return fail(BITNET_ERR_NULL, "%s: no input pointer may be NULL", fn);
    if (!aligned(grad_y, 16) || !aligned(xq, 16))
        return fail(BITNET_ERR_ALIGN, "%s: grad_y and xq must be 16-byte aligned", fn);
    if (!aligned(x_scale, 4)) return fail(BITNET_ERR_ALIGN, "%s: x_scale must be 4-byte aligned", fn);
    const size_t need = bitnet::backward_weight_workspace_bytes(M, N, K);
    if (!workspace || workspace_bytes < need)
        return fail(BITNET_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(BITNET_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
    return hip_status(bitnet::launch_backward_weight(grad_y, xq, x_scale, M, N, K, grad_w, workspace,
                                                     (hipStream_t)stream),
                      fn);
}

size_t bitnet_rmsnorm_backward_workspace_bytes(int64_t M, int64_t K) {
    if (M < 1 || M > kMaxRows || K < kMinK || K > kMaxK || K % 64 != 0) return 0;
    return bitnet::rmsnorm_backward_workspace_bytes(M, K);
}

int bitnet_rmsnorm_backward(const uint16_t* x, const float* gain, float eps, const float* grad_n,
                            int64_t M, int64_t K, float* grad_x, float* grad_gain, void* workspace,
                            size_t workspace_bytes, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_rmsnorm_backward";
    if (M < 0 || M > kMaxRows) return fail(BITNET_ERR_SHAPE, "%s: M=%lld out of range", fn, (long long)M);
    int s = check_k(K, fn);
    if (s != BITNET_OK) return s;
    if ((s = check_eps(eps, fn)) != BITNET_OK) return s;
    if (M == 0) {
        if (grad_gain)
            return hip_status(bitnet::launch_zero_f32(grad_gain, K, (hipStream_t)stream), fn);
        return BITNET_OK;
    }
    if (!x || !grad_n || !grad_x) return fail(BITNET_ERR_NULL, "%s: x, grad_n and grad_x must not be NULL", fn);
    if (!aligned(x, 4) || !aligned(grad_n, 4) || !aligned(grad_x, 4) || (gain && !aligned(gain, 4)) ||
        (grad_gain && !aligned(grad_gain, 4)))
        return fail(BITNET_ERR_ALIGN, "%s: arrays must be 4-byte aligned", fn);
    if (grad_gain) {
        const size_t need = bitnet::rmsnorm_backward_workspace_bytes(M, K);
        if (!workspace || workspace_bytes < need)
            return fail(BITNET_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 16)) return fail(BITNET_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
    }
    return hip_status(bitnet::launch_rmsnorm_backward(x, gain, eps, grad_n, M, K, grad_x, grad_gain,
                                                      workspace, (hipStream_t)stream),
                      fn);
}

size_t bitnet_linear_forward_blend_workspace_bytes(int64_t M, int64_t K) {
    if (M < 1 || M > kMaxRows || K < kMinK || K > kMaxK || K % 64 != 0) return 0;
    return bitnet::blend_workspace_bytes(M, K);
}

int bitnet_linear_forward_blend(const uint16_t* x, const float* gain, float eps, const float* W,
                                const uint8_t* packed, const float* w_scale, float lambda, int64_t M, int64_t N,
                                int64_t K, float* y, void* workspace, size_t workspace_bytes, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_linear_forward_blend";
    if (M < 0 || M > kMaxRows || N < 0 || N > kMaxRows)
        return fail(BITNET_ERR_SHAPE, "%s: M=%lld or N=%lld out of range", fn, (long long)M, (long long)N);
    int s = check_k(K, fn);
    if (s != BITNET_OK) return s;
    if ((s = check_eps(eps, fn)) != BITNET_OK) return s;
    if (!std::isfinite(lambda) || lambda < 0.f || lambda > 1.f)
        return fail(BITNET_ERR_VALUE, "%s: lambda must be in [0, 1]", fn);
    if (M == 0 || N == 0) return BITNET_OK;
    if (!x || !W || !packed || !w_scale || !y || !workspace)
        return fail(BITNET_ERR_NULL, "%s: only gain may be NULL", fn);
    if (!aligned(x, 16) || !aligned(W, 16) || !aligned(packed, 16) || !aligned(workspace, 16) ||
        (gain && !aligned(gain, 16)))
        return fail(BITNET_ERR_ALIGN, "%s: x, gain, W, packed and workspace must be 16-byte aligned", fn);
    if (!aligned(w_scale, 4) || !aligned(y, 4))
        return fail(BITNET_ERR_ALIGN, "%s: w_scale and y must be 4-byte aligned", fn);
    const size_t need = bitnet::blend_workspace_bytes(M, K);
    if (workspace_bytes < need)
        return fail(BITNET_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
    return hip_status(bitnet::launch_linear_forward_blend(x, gain, eps, W, packed, w_scale, lambda, M, N, K, y,
                                                          workspace, (hipStream_t)stream),
                      fn);
}

int bitnet_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_stream_read";
    if (bytes < 16 || bytes % 16 != 0 || bytes > ((size_t)1 << 40))
        return fail(BITNET_ERR_SHAPE, "%s: bytes=%zu must be a multiple of 16 in [16, 2^40]", fn, bytes);
    if (!buf || !sink) return fail(BITNET_ERR_NULL, "%s: buf and sink must not be NULL", fn);
    if (!aligned(buf, 16) || !aligned(sink, 4))
        return fail(BITNET_ERR_ALIGN, "%s: buf must be 16-byte and sink 4-byte aligned", fn);
    return hip_status(bitnet::launch_stream_read(buf, (int64_t)bytes, sink, (hipStream_t)stream), fn);
}

const char* bitnet_status_string(int status) {
    switch (status) {
        case BITNET_OK: return "ok";
        case BITNET_ERR_NULL: return "a required pointer is NULL";
        case BITNET_ERR_SHAPE: return "shape out of range";
        case BITNET_ERR_UNSUPPORTED: return "unsupported shape";
        case BITNET_ERR_ALIGN: return "misaligned pointer";
        case BITNET_ERR_WORKSPACE: return "workspace missing or too small";
        case BITNET_ERR_HIP: return "HIP error";
        case BITNET_ERR_VALUE: return "invalid scalar argument";
        default: return "unknown status";
    }
}

const char* bitnet_last_error(void) { return g_last_error; }

int bitnet_version(void) { return BITNET_ABI_VERSION; }

size_t bitnet_base3_row_bytes(int64_t K) {
    if (K < kMinK || K > kMaxK || K % 64 != 0) return 0;
    return (size_t)bitnet::base3_row_bytes(K);
}

int bitnet_pack_base3(const uint8_t* packed, int64_t N, int64_t K, uint8_t* packed3, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_pack_base3";
    if (N < 0 || N > kMaxRows) return fail(BITNET_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
    int s = check_k(K, fn);
    if (s != BITNET_OK) return s;
    if (N == 0) return BITNET_OK;
    if (!packed || !packed3) return fail(BITNET_ERR_NULL, "%s: packed and packed3 must not be NULL", fn);
    if (!aligned(packed, 16) || !aligned(packed3, 16))
        return fail(BITNET_ERR_ALIGN, "%s: packed and packed3 must be 16-byte aligned", fn);
    return hip_status(bitnet::launch_pack_base3(packed, N, K, packed3, (hipStream_t)stream), fn);
}

int bitnet_linear_forward_base3(const int8_t* xq, const float* x_scale, const int32_t* x_qsum,
                                const uint8_t* packed3, const float* w_scale, int64_t M, int64_t N, int64_t K,
                                float* y, int32_t* acc, void* stream) {
    DisarmEvents disarm;
    const char* fn = "bitnet_linear_forward_base3";
    if (M < 0 || N < 0 || N > kMaxRows)
        return fail(BITNET_ERR_SHAPE, "%s: M=%lld or N=%lld out of range", fn, (long long)M, (long long)N);
    int s = check_k(K, fn);
    if (s != BITNET_OK) return s;
    if (M > 1) return fail(BITNET_ERR_UNSUPPORTED, "%s: one token (M = 1) only, got M=%lld", fn, (long long)M);
    if (!bitnet::base3_gemv_supported(K))
        return fail(BITNET_ERR_UNSUPPORTED, "%s: K=%lld above 20480", fn, (long long)K);
    if (M == 0 || N == 0) return BITNET_OK;
    if (!xq || !x_scale || !x_qsum || !packed3 || !w_scale || !y)
        return fail(BITNET_ERR_NULL, "%s: only acc may be NULL", fn);
    if (!aligned(xq, 16) || !aligned(packed3, 16))
        return fail(BITNET_ERR_ALIGN, "%s: xq and packed3 must be 16-byte aligned", fn);
    if (!aligned(x_scale, 4) || !aligned(x_qsum, 4) || !aligned(w_scale, 4) || !aligned(y, 4) ||
        (acc && !aligned(acc, 4)))
        return fail(BITNET_ERR_ALIGN, "%s: scales, sums, y and acc must be 4-byte aligned", fn);
    return hip_status(bitnet::launch_base3_gemv(xq, x_scale, x_qsum, packed3, w_scale, N, K, y, acc,
                                                (hipStream_t)stream),
                      fn);
}

}  // extern "C"
