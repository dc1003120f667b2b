// Cache warm of a device range ("DeepSeek V4 Decode Optimization" sec. 4.5:
// a warm is a cache hint with no destination; it pays when the range fits the
// cache, lands before its consumer needs it, and overlaps work that leaves
// HBM idle). The kernel reads every 16 bytes of the range once with ordinary
// loads, so the lines are allocated on the way (the 256 MB memory-side cache
// and the XCD's L2), and discards the data: no value anywhere changes.
#include "internal.h"

namespace moe {
namespace {

constexpr int kWarmThreads = 256;
constexpr int kWarmUnroll = 4;      // 16-byte loads in flight per thread and iteration
constexpr int kWarmMaxBlocks = 128;

__global__ __launch_bounds__(kWarmThreads) void warm_kernel(const uint4 *p, size_t n16) {
    const size_t stride = static_cast<size_t>(gridDim.x) * kWarmThreads * kWarmUnroll;
    uint32_t acc = 0;
    for (size_t i = static_cast<size_t>(blockIdx.x) * kWarmThreads * kWarmUnroll + threadIdx.x; i < n16;
         i += stride) {
        uint4 v[kWarmUnroll];
#pragma unroll
        for (int u = 0; u < kWarmUnroll; ++u) {
            const size_t j = i + static_cast<size_t>(u) * kWarmThreads;
            v[u] = j < n16 ? p[j] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kWarmUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // keep the loads: the value is consumed by an empty asm statement (no
    // memory access), so the compiler cannot drop them
    asm volatile("; warm %0" ::"v"(acc));
}

}  // namespace

hipError_t launch_warm(const void *ptr, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    const size_t per_block = static_cast<size_t>(kWarmThreads) * kWarmUnroll;
    const size_t blocks = (n16 + per_block - 1) / per_block;
    const dim3 grid(static_cast<unsigned>(blocks < kWarmMaxBlocks ? blocks : kWarmMaxBlocks));
    hipLaunchKernelGGL(warm_kernel, grid, dim3(kWarmThreads), 0, s, static_cast<const uint4 *>(ptr), n16);
    return hipGetLastError();
}

}  // namespace moe
