// Cache warm of a device range ("DeepSeek V4 Decode Optimization" sec. 4.5:
// a warm is a cache hint with no destination; it pays when the range fits the
// cache, lands before its consumer needs it, and overlaps work that leaves
// HBM idle). The kernel reads every 16 bytes of the range once with ordinary
// loads, so the lines are allocated on the way (the 256 MB memory-side cache
// and the XCD's L2), and discards the data: no value anywhere changes.
// The same file holds a read-bandwidth probe with the weight stream's access
// pattern, which measures the HBM read rate the device reaches, and a probe
// that also writes, as a larger batch's GEMM writes its output rows while its
// weights stream.
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

// Read-and-write probe: the larger-batch GEMM's weight stream with its
// output writes and nothing else. Work item (block) i reads 256 KB: each of
// its two waves streams two 64 KB tiles in 1 KB steps (lane l at byte 16 l)
// through a ring of 8 non-temporal loads per tile, a step refilled as soon as
// it is consumed; then the block stores its share of the write range,
// [i * dst16 / items, (i + 1) * dst16 / items) in 16-byte units, as a GEMM
// block stores its rows after its K loop. Six blocks run per CU (the GEMM's
// residency), held there by LDS the kernel reserves and does not use.
constexpr int kRwThreads = 128;
constexpr size_t kRwItemBytes = 256 * 1024;
constexpr int kRwTile16 = 64 * 1024 / 16;  // 16-byte units per 64 KB tile
constexpr int kRwRing = 8;
constexpr int kRwBlocksPerCu = 6;

__global__ __launch_bounds__(kRwThreads) void rw_probe_kernel(const v4u *src, v4u *dst, size_t dst16,
                                                               unsigned items) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const size_t item = blockIdx.x;
    const v4u *ta = src + (item * 2 + wave) * 2 * kRwTile16;
    const v4u *tb = ta + kRwTile16;
    constexpr int kSteps = kRwTile16 / kWave;  // 64 steps of 1 KB per tile
    v4u ra[kRwRing], rb[kRwRing];
#pragma unroll
    for (int i = 0; i < kRwRing; ++i) {
        ra[i] = __builtin_nontemporal_load(ta + i * kWave + lane);
        rb[i] = __builtin_nontemporal_load(tb + i * kWave + lane);
    }
    v4u acc = {0, 0, 0, 0};
    for (int c = 0; c < kSteps / kRwRing; ++c) {
#pragma unroll
        for (int i = 0; i < kRwRing; ++i) {
            acc ^= ra[i] ^ rb[i];
            const int next = (c + 1) * kRwRing + i;
            if (next < kSteps) {
                ra[i] = __builtin_nontemporal_load(ta + next * kWave + lane);
                rb[i] = __builtin_nontemporal_load(tb + next * kWave + lane);
            }
            __builtin_amdgcn_sched_barrier(0);  // refill each slot right after its use
        }
    }
    const size_t w0 = item * dst16 / items, w1 = (item + 1) * dst16 / items;
    for (size_t j = w0 + threadIdx.x; j < w1; j += kRwThreads) dst[j] = acc;
}

}  // namespace

hipError_t launch_rw_probe(const void *src, size_t src_bytes, void *dst, size_t dst_bytes, hipStream_t s) {
    const size_t items = src_bytes / kRwItemBytes;
    if (items == 0) return hipSuccess;
    int dev = 0, lds = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        lds <= 0)
        return hipErrorInvalidDevice;
    // reserve a sixth of the CU's LDS per block (rounded down to 256 bytes):
    // six blocks fit, a seventh does not
    const unsigned pad = static_cast<unsigned>(lds / kRwBlocksPerCu) & ~255u;
    hipLaunchKernelGGL(rw_probe_kernel, dim3(static_cast<unsigned>(items)), dim3(kRwThreads), pad, s,
                       static_cast<const v4u *>(src), static_cast<v4u *>(dst), dst_bytes / 16,
                       static_cast<unsigned>(items));
    return hipGetLastError();
}

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
