// Weighted top-k combine ("FusedDeepMoE Kernel 深度分析报告" sec. 4.2,
// LocalWindowCopy): for each token, an fp32 sum that starts at zero and adds,
// for k = 0..K-1 in order, the expert's bf16 row (cast to fp32) times the
// routing weight (unless the weight was folded into the row's GEMM2 row
// scale: then the rows are summed as they are); one round-to-nearest-even
// cast to bf16 at the end. Pairs
// that were dropped (inactive token, non-local expert, bad id) contribute
// nothing, so such tokens get zero rows. The sum order is fixed per element,
// so the result is deterministic.
//
// Grid = tokens x (H / 1024): each thread owns 8 consecutive channels and
// issues the 16-byte loads of all K rows (z is in pair order) together with
// the pairs' kept flags before it sums them, so a token costs one memory
// round trip. It also clears the shared-expert rows of
// inactive tokens, which GEMM2 never writes.
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 128;
constexpr int kChannels = kThreads * 8;  // channels per block

__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
    const int t = blockIdx.x;
    const int c = blockIdx.y * kChannels + threadIdx.x * 8;
    if (c >= a.H) return;
    const int32_t *rop = a.row_of_pair + static_cast<size_t>(t) * a.K;
    const float *wt = a.scales + static_cast<size_t>(t) * a.K;
    // z holds pair p = t*K + k at row p (written only for kept pairs): all K
    // rows are loaded at once, alongside the row_of_pair entries that say
    // which of them are kept (z has T*K rows, so every load is in bounds)
    uint4 raw[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        raw[k] = make_uint4(0, 0, 0, 0);
        if (k < a.K)
            raw[k] = *reinterpret_cast<const uint4 *>(a.z + (static_cast<size_t>(t) * a.K + k) * a.H + c);
    }
    float sum[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sum[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        if (k < a.K && rop[k] >= 0) {
            const float wk = wt[k];
            const uint32_t v[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float m0 = bf16_to_f32(static_cast<uint16_t>(v[i] & 0xFFFFu));
                float m1 = bf16_to_f32(static_cast<uint16_t>(v[i] >> 16));
                if (!a.fused) {
                    m0 = m0 * wk;
                    m1 = m1 * wk;
                }
                sum[2 * i] = sum[2 * i] + m0;
                sum[2 * i + 1] = sum[2 * i + 1] + m1;
            }
        }
    }
    uint4 o;
    o.x = f32_to_bf16(sum[0]) | (static_cast<uint32_t>(f32_to_bf16(sum[1])) << 16);
    o.y = f32_to_bf16(sum[2]) | (static_cast<uint32_t>(f32_to_bf16(sum[3])) << 16);
    o.z = f32_to_bf16(sum[4]) | (static_cast<uint32_t>(f32_to_bf16(sum[5])) << 16);
    o.w = f32_to_bf16(sum[6]) | (static_cast<uint32_t>(f32_to_bf16(sum[7])) << 16);
    *reinterpret_cast<uint4 *>(a.out + static_cast<size_t>(t) * a.H + c) = o;
    if (a.has_shared && a.mask && !a.mask[t])
        *reinterpret_cast<uint4 *>(a.share_out + static_cast<size_t>(t) * a.H + c) = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
    if (a.T <= 0) return hipSuccess;
    const dim3 grid(a.T, (a.H + kChannels - 1) / kChannels);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
