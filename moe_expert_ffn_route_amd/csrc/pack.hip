// One-time weight re-layout into the order the GEMM kernels stream: for each
// (group, 16-row tile, 64-byte K step) one contiguous 1 KB block whose
// 16-byte lane slots hold exactly what MFMA lane l needs (row l % 16, bytes
// 16 * (l / 16) .. +16 of the step). A GEMM1 weight also reorders its tiles
// so that gate tile j and up tile j (the two tiles one GEMM1 work item
// streams) follow each other. The MI355X counterpart of the NZ weight format
// that "FusedDeepMoE Kernel 深度分析报告" sec. 5.3 / 8.1 prepares for its cube
// unit. Pure data movement: one thread per 16-byte slot, writes coalesced.
// FP4 weights take the same re-layout of their nibble-pair bytes (a 64-byte
// step is then 128 elements), followed by their block scales in lane order.
#include "internal.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void pack_kernel(const int8_t *__restrict__ src, int8_t *__restrict__ dst,
                                                   int64_t slots, int n, int k, int which) {
    const int64_t o = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (o >= slots) return;
    const int l = static_cast<int>(o & 63);
    const int64_t blk = o >> 6;                 // (g, tile position, step) block index
    const int64_t steps = k / 64;
    const int64_t s = blk % steps;
    const int64_t gt = blk / steps;             // g * (n / 16) + tile position
    const int64_t tiles = n / 16;
    const int64_t g = gt / tiles, pos = gt % tiles;
    // GEMM1: position 2j holds gate tile j, 2j + 1 up tile j
    const int64_t j = which == 1 ? (pos & 1) * (tiles / 2) + (pos >> 1) : pos;
    const int64_t row = j * 16 + (l & 15);
    const int64_t col = s * 64 + (l >> 4) * 16;
    const v4i v = *reinterpret_cast<const v4i *>(src + (g * n + row) * k + col);
    *reinterpret_cast<v4i *>(dst + o * 16) = v;
}

// E8M0 block scales of FP4 weights: for each (group, tile position, 128-element
// K step) 64 bytes, byte l the scale of row l % 16 of the tile for the 32
// elements 32 * (l / 16) .. +32 of the step, which is the byte the scaled
// MFMA takes from lane l. One thread per byte.
__global__ __launch_bounds__(256) void pack_scale_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                         int64_t bytes, int n, int k, int which) {
    const int64_t o = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (o >= bytes) return;
    const int l = static_cast<int>(o & 63);
    const int64_t blk = o >> 6;
    const int64_t steps = k / 128;
    const int64_t s = blk % steps;
    const int64_t gt = blk / steps;
    const int64_t tiles = n / 16;
    const int64_t g = gt / tiles, pos = gt % tiles;
    const int64_t j = which == 1 ? (pos & 1) * (tiles / 2) + (pos >> 1) : pos;
    const int64_t row = j * 16 + (l & 15);
    dst[o] = src[(g * n + row) * (k / 32) + 4 * s + (l >> 4)];
}

}  // namespace

hipError_t launch_pack_mx(const uint8_t *data, const uint8_t *bscale, uint8_t *dst, int64_t groups, int n, int k,
                          int which, hipStream_t s) {
    // elements: the int8 re-layout of the [groups, n, k / 2] byte tensor
    const hipError_t e = launch_pack(reinterpret_cast<const int8_t *>(data), reinterpret_cast<int8_t *>(dst),
                                     groups, n, k / 2, which, s);
    if (e != hipSuccess) return e;
    const int64_t bytes = groups * static_cast<int64_t>(n) * (k / 32);
    if (bytes == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_scale_kernel, dim3(static_cast<unsigned>((bytes + 255) / 256)), dim3(256), 0, s, bscale,
                       dst + groups * static_cast<int64_t>(n) * (k / 2), bytes, n, k, which);
    return hipGetLastError();
}

hipError_t launch_pack(const int8_t *src, int8_t *dst, int64_t groups, int n, int k, int which, hipStream_t s) {
    const int64_t slots = groups * static_cast<int64_t>(n) * k / 16;
    if (slots == 0) return hipSuccess;
    const int64_t blocks = (slots + 255) / 256;
    hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, src, dst, slots, n, k, which);
    return hipGetLastError();
}

}  // namespace moe
