// Row quantisation kernels (the rule and its fp32 order are in rowquant.h;
// FP8 instantiations quantise to E4M3 for the FP4-weight variant):
//
//   requant_wave_kernel / requant_kernel  the SwiGLU output h of every
//                        grouped row ("FusedDeepMoE Kernel 深度分析报告"
//                        sec. 7.2);
//   dbg_gather_kernel    test support only: GEMM1's input rows in grouped-row
//                        order (the q_x / xs dump).
//
// Rows of up to 4096 elements take one wavefront each (in batches of more
// than 256 grouped rows), four to a workgroup, with no workgroup barrier: the
// row sits in the wave's registers between its amax and its quantisation.
// Longer rows take a workgroup of 256 threads each.
// Either way each row is read once. (x is quantised in the routing launch.)
#include "rowquant.h"

namespace moe {
namespace {

// GL > 0: group-wise scales ("DeepSeek V4 Decode Optimization" sec. 3.1), one
// per 4 * GL elements, a.ng of them per row.
template <bool FP8, int GL>
__global__ __launch_bounds__(kTPR) void requant_kernel(RequantArgs a) {
    __shared__ float s_part[kTPR / kWave];
    const int r = blockIdx.x;
    const int nrows = a.meta[kMetaP] + (a.has_shared ? a.meta[kMetaTAct] : 0);
    if (r >= nrows) return;
    const int n = a.row_group[r] < a.E_loc ? a.I : a.I_s;
    quant_f32_row<FP8, GL>(a.h + static_cast<size_t>(r) * a.imax, n, a.eps, a.q + static_cast<size_t>(r) * a.imax,
                           a.scale + static_cast<size_t>(r) * a.ng, true, 0, threadIdx.x, s_part);
    if (a.scale2 && threadIdx.x == 0) {  // the thread that wrote scale[r]
        const float hs = a.scale[r];
        a.scale2[r] = r < a.meta[kMetaP] ? hs * a.route_w[a.sorted_pair[r]] : hs;
    }
}

constexpr int kRowsPerBlock = 4;  // one wavefront per row

// Grouped row of this wavefront (wave-uniform, so its index loads are scalar).
__device__ __forceinline__ int wave_row() {
    return blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

// NCH 16-byte chunks of fp32 per lane: rows of up to NCH * 256 values.
template <int NCH, bool FP8, int GL>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void requant_wave_kernel(RequantArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int r = wave_row();
    if (r >= a.rows_max) return;
    const int P = a.meta[kMetaP], t_act = a.meta[kMetaTAct];
    const int g = a.row_group[r];
    const float *src = a.h + static_cast<size_t>(r) * a.imax;
    float4 v[NCH];
    auto load = [&] {
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int i = (lane + j * kWave) * 4;
            if (i < a.imax) v[j] = *reinterpret_cast<const float4 *>(src + i);
        }
    };
    // With load_early the row is fetched together with the row count (every
    // h row is inside the workspace, so the read is in bounds even for a row
    // that turns out to be unused); otherwise only rows in use are read.
    if (a.load_early) load();
    const int nrows = P + (a.has_shared ? t_act : 0);
    if (r >= nrows) return;
    if (!a.load_early) load();
    const int n = g < a.E_loc ? a.I : a.I_s;
    int8_t *dst = a.q + static_cast<size_t>(r) * a.imax;
    if constexpr (GL > 0) {
        // one scale per group of 4 * GL elements, each in GL neighbouring lanes
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int i = (lane + j * kWave) * 4;
            if (j * kWave * 4 >= n) break;  // uniform
            const float mj = i < n ? fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w)))
                                   : 0.0f;
            const float ap = fmaxf(segment_max<GL>(mj), a.eps);
            const float inv = 1.0f / ap;
            if (i < n) {
                *reinterpret_cast<uint32_t *>(dst + i) = quant4<FP8>(v[j].x, v[j].y, v[j].z, v[j].w, inv);
                if ((lane & (GL - 1)) == 0)
                    a.scale[static_cast<size_t>(r) * a.ng + i / (4 * GL)] = ap * (1.0f / kQMax<FP8>);
            }
        }
        return;
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int i = (lane + j * kWave) * 4;
        if (i < n) m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    }
    const float ap = fmaxf(wave_max(m), a.eps);
    const float inv = 1.0f / ap;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int i = (lane + j * kWave) * 4;
        if (i < n) *reinterpret_cast<uint32_t *>(dst + i) = quant4<FP8>(v[j].x, v[j].y, v[j].z, v[j].w, inv);
    }
    if (lane == 0) {
        const float hs = ap * (1.0f / kQMax<FP8>);
        a.scale[r] = hs;
        if (a.scale2) a.scale2[r] = r < P ? hs * a.route_w[a.sorted_pair[r]] : hs;
    }
}

// Debug dump of GEMM1's input rows in grouped-row order: row r is copied from
// where GEMM1 reads it (the token's or the pair's row).
__global__ __launch_bounds__(256) void dbg_gather_kernel(GemmArgs g, const int32_t *row_group, const int32_t *meta,
                                                          int has_shared, int8_t *dst_q, float *dst_xs) {
    const int r = blockIdx.x;
    const int nrows = meta[kMetaP] + (has_shared ? meta[kMetaTAct] : 0);
    if (r >= nrows) return;
    const bool routed = row_group[r] < g.E_loc;
    const size_t src = routed ? g.idx_r[r] : g.row_token[r];
    const int8_t *qs = (routed ? g.A_r : g.A_s) + src * g.H;
    if (dst_q)
        for (int i = threadIdx.x * 16; i < g.H; i += 256 * 16)
            *reinterpret_cast<uint4 *>(dst_q + static_cast<size_t>(r) * g.H + i) =
                *reinterpret_cast<const uint4 *>(qs + i);
    if (dst_xs && static_cast<int>(threadIdx.x) < g.a_ng)  // a_ng <= H / 64 <= 256 scales per row
        dst_xs[static_cast<size_t>(r) * g.a_ng + threadIdx.x] =
            (routed ? g.a_scale_r : g.a_scale_s)[src * g.a_ng + threadIdx.x];
}

// Rows of up to MOE_REQUANT_WAVE_MAX values take one wavefront each, longer
// rows one 256-thread workgroup each. Batches expected to use at most
// MOE_REQUANT_BLOCK_ROWS grouped rows (decode, or an expert-parallel share of
// a larger batch) also take a workgroup per row: with so few rows the chip is
// mostly idle, and four times the threads per row shorten each row's chain of
// loads and conversions (measured on MI355X at T = 8, 80 rows of 2048: 4.9 ->
// 4.6 us INT8, 5.5 -> 4.6 us FP8).
#ifndef MOE_REQUANT_WAVE_MAX
#define MOE_REQUANT_WAVE_MAX 4096
#endif
#ifndef MOE_REQUANT_BLOCK_ROWS
#define MOE_REQUANT_BLOCK_ROWS 256
#endif

template <bool FP8, int GL>
hipError_t launch_requant_fmt(const RequantArgs &a, dim3 wgrid, dim3 wblk, hipStream_t s) {
    const bool wave = a.rows_expected > MOE_REQUANT_BLOCK_ROWS;
    if (wave && a.imax <= 8 * 256 && a.imax <= MOE_REQUANT_WAVE_MAX)
        hipLaunchKernelGGL((requant_wave_kernel<8, FP8, GL>), wgrid, wblk, 0, s, a);
    else if (wave && a.imax <= 16 * 256 && a.imax <= MOE_REQUANT_WAVE_MAX)
        hipLaunchKernelGGL((requant_wave_kernel<16, FP8, GL>), wgrid, wblk, 0, s, a);
    else
        hipLaunchKernelGGL((requant_kernel<FP8, GL>), dim3(a.rows_max), dim3(kTPR), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_requant(const RequantArgs &a, hipStream_t s) {
    if (a.rows_max <= 0) return hipSuccess;
    const dim3 wgrid((a.rows_max + kRowsPerBlock - 1) / kRowsPerBlock), wblk(kRowsPerBlock * kWave);
    if (a.fp8) return launch_requant_fmt<true, 0>(a, wgrid, wblk, s);
    switch (a.gl) {
        case 16: return launch_requant_fmt<false, 16>(a, wgrid, wblk, s);
        case 32: return launch_requant_fmt<false, 32>(a, wgrid, wblk, s);
        case 64: return launch_requant_fmt<false, 64>(a, wgrid, wblk, s);
        default: return launch_requant_fmt<false, 0>(a, wgrid, wblk, s);
    }
}

hipError_t launch_dbg_gather(const GemmArgs &g1, const int32_t *row_group, const int32_t *meta, int has_shared,
                             int rows_max, int8_t *dst_q, float *dst_xs, hipStream_t s) {
    if (rows_max <= 0) return hipSuccess;
    hipLaunchKernelGGL(dbg_gather_kernel, dim3(rows_max), dim3(256), 0, s, g1, row_group, meta, has_shared, dst_q,
                       dst_xs);
    return hipGetLastError();
}

}  // namespace moe
