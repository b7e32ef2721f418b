// stream_read.hip - a plain read of a device buffer: the reference rate against
// which the bandwidth-bound kernels' GB/s are stated (what a simple streaming
// kernel reaches on this GPU), not part of the BitLinear computation.
#include "common.hpp"
#include "launch.hpp"

namespace bitnet {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;  // independent 16-byte loads in flight per thread

// Every 16-byte chunk is read once (grid-stride, kReadUnroll chunks per step);
// the XOR of the words read decides a store that never happens in practice, so
// no load can be dropped.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const v4i* __restrict__ src,
                                                                  int64_t chunks,
                                                                  uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kReadThreads;
    int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kReadUnroll - 1) * stride < chunks; i += kReadUnroll * stride) {
        v4i v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
    }
    for (; i < chunks; i += stride) {
        const v4i v = src[i];
        acc ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    const int64_t chunks = bytes / 16;
    // Eight workgroups per CU on 256 CUs, or fewer for small buffers.
    const int64_t want = (chunks + kReadThreads * kReadUnroll - 1) / (kReadThreads * kReadUnroll);
    const unsigned blocks = (unsigned)(want < 2048 ? (want > 0 ? want : 1) : 2048);
    return launch_kernel(stream_read_kernel, dim3(blocks), dim3(kReadThreads), 0, stream,
                         reinterpret_cast<const v4i*>(src), chunks, sink);
}

}  // namespace bitnet
