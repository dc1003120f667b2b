// Cache warm of a device range ("DeepSeek V4 Decode Optimization" sec. 4.5:
// a warm is a cache hint with no destination; it pays when the range fits the
// cache, lands before its consumer needs it, and overlaps work that leaves
// HBM idle). The kernel reads every 16 bytes of the range once with ordinary
// loads, so the lines are allocated on the way (the 256 MB memory-side cache
// and the XCD's L2), and discards the data: no value anywhere changes.
// The same file holds a read-bandwidth probe with the weight stream's access
// pattern, which measures the HBM read rate the device reaches.
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

// Read-bandwidth probe: the GEMMs' weight-stream pattern with nothing else.
// Each wave reads 1 KB contiguous per load instruction (lane l at byte 16 l)
// with non-temporal loads, kProbeUnroll loads in flight per wave, in a
// grid-stride loop over the range; the data is discarded the same way.
#ifndef MOE_PROBE_UNROLL
#define MOE_PROBE_UNROLL 8
#endif
#ifndef MOE_PROBE_BLOCKS_PER_CU
#define MOE_PROBE_BLOCKS_PER_CU 8
#endif
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = MOE_PROBE_UNROLL;
constexpr int kProbeBlocksPerCu = MOE_PROBE_BLOCKS_PER_CU;

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const v4u *p, size_t n16) {
    const int lane = threadIdx.x & (kWave - 1);
    const size_t wave = static_cast<size_t>(blockIdx.x) * (kProbeThreads / kWave) + threadIdx.x / kWave;
    const size_t waves = static_cast<size_t>(gridDim.x) * (kProbeThreads / kWave);
    constexpr size_t kWaveSpan = static_cast<size_t>(kWave) * kProbeUnroll;  // 16-byte units per wave pass
    uint32_t acc = 0;
    for (size_t base = wave * kWaveSpan; base < n16; base += waves * kWaveSpan) {
        v4u v[kProbeUnroll];
        if (base + kWaveSpan <= n16) {  // wave-uniform: a whole pass in range, no per-load checks
#pragma unroll
            for (int u = 0; u < kProbeUnroll; ++u)
                v[u] = __builtin_nontemporal_load(p + base + static_cast<size_t>(u) * kWave + lane);
        } else {
#pragma unroll
            for (int u = 0; u < kProbeUnroll; ++u) {
                const size_t j = base + static_cast<size_t>(u) * kWave + lane;
                v[u] = j < n16 ? __builtin_nontemporal_load(p + j) : v4u{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    asm volatile("; read probe %0" ::"v"(acc));
}

}  // namespace

hipError_t launch_read_probe(const void *ptr, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return hipErrorInvalidDevice;
    const size_t per_block = static_cast<size_t>(kProbeThreads) * kProbeUnroll;
    const size_t need = (n16 + per_block - 1) / per_block;
    const size_t cap = static_cast<size_t>(cus) * kProbeBlocksPerCu;
    const dim3 grid(static_cast<unsigned>(need < cap ? need : cap));
    hipLaunchKernelGGL(read_probe_kernel, grid, dim3(kProbeThreads), 0, s, static_cast<const v4u *>(ptr), n16);
    return hipGetLastError();
}

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
