// Row quantisation kernels (the rule and its fp32 order are in rowquant.h):
//
//   smooth_quant_kernel  GEMM1 input for groups with smooth scales: grouped
//                        row r = x[row_token[r]] * smooth[expert of r]
//                        ("FusedDeepMoE Kernel 深度分析报告" sec. 1.2
//                        expert_smooth_scales / share_smooth_scales), so the
//                        quantisation is per (token, expert) pair;
//   requant_kernel       the SwiGLU output h of every grouped row (sec. 7.2);
//   dbg_gather_kernel    test support only: writes the per-row q_x / xs dump
//                        for rows whose GEMM1 input is the per-token row.
//
// Rows of up to 4096 elements take one
// wavefront each, four to a workgroup, with no workgroup barrier: the row
// sits in the wave's registers between its amax and its quantisation. Longer
// rows take a workgroup of 256 threads each. Either way each row is read once.
#include "rowquant.h"

namespace moe {
namespace {

__global__ __launch_bounds__(kTPR) void smooth_quant_kernel(QuantArgs a) {
    __shared__ float s_part[kTPR / kWave];
    const int r = blockIdx.x;
    const int nrows = a.meta[kMetaP] + (a.has_shared ? a.meta[kMetaTAct] : 0);
    if (r >= nrows) return;
    const int g = a.row_group[r];
    const float *sm = g < a.E_loc ? (a.smooth ? a.smooth + static_cast<size_t>(g) * a.H : nullptr) : a.share_smooth;
    if (!sm) return;  // this group reads the per-token rows
    const size_t t = a.row_token[r];
    quant_bf16_row(a.x + t * a.H, sm, a.H, a.eps, a.q + static_cast<size_t>(r) * a.H, a.scale + r, true, 0,
                   threadIdx.x, s_part);
}

__global__ __launch_bounds__(kTPR) void requant_kernel(RequantArgs a) {
    __shared__ float s_part[kTPR / kWave];
    const int r = blockIdx.x;
    const int nrows = a.meta[kMetaP] + (a.has_shared ? a.meta[kMetaTAct] : 0);
    if (r >= nrows) return;
    const int n = a.row_group[r] < a.E_loc ? a.I : a.I_s;
    quant_f32_row(a.h + static_cast<size_t>(r) * a.imax, n, a.eps, a.q + static_cast<size_t>(r) * a.imax,
                  a.scale + r, true, 0, threadIdx.x, s_part);
}

constexpr int kRowsPerBlock = 4;  // one wavefront per row

// Grouped row of this wavefront (wave-uniform, so its index loads are scalar).
__device__ __forceinline__ int wave_row() {
    return blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

// NCH 16-byte chunks of fp32 per lane: rows of up to NCH * 256 values.
template <int NCH>
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
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int i = (lane + j * kWave) * 4;
        if (i < n) m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    }
    const float ap = fmaxf(wave_max(m), a.eps);
    const float inv = 1.0f / ap;
    int8_t *dst = a.q + static_cast<size_t>(r) * a.imax;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int i = (lane + j * kWave) * 4;
        if (i < n) *reinterpret_cast<uint32_t *>(dst + i) = quant4(v[j].x, v[j].y, v[j].z, v[j].w, inv);
    }
    if (lane == 0) a.scale[r] = ap * (1.0f / 127.0f);
}

// NCH 16-byte chunks of bf16 per lane: rows of up to NCH * 512 values.
template <int NCH>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void smooth_quant_wave_kernel(QuantArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int r = wave_row();
    if (r >= a.rows_max) return;
    const int nrows = a.meta[kMetaP] + (a.has_shared ? a.meta[kMetaTAct] : 0);
    const int g = a.row_group[r];
    const size_t t = a.row_token[r];
    if (r >= nrows) return;
    const float *sm = g < a.E_loc ? (a.smooth ? a.smooth + static_cast<size_t>(g) * a.H : nullptr) : a.share_smooth;
    if (!sm) return;  // this group reads the per-token rows
    const uint16_t *src = a.x + t * a.H;
    float v[NCH][8];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int i = (lane + j * kWave) * 8;
        if (i < a.H) {
            const uint4 raw = *reinterpret_cast<const uint4 *>(src + i);
            const float4 s0 = *reinterpret_cast<const float4 *>(sm + i);
            const float4 s1 = *reinterpret_cast<const float4 *>(sm + i + 4);
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
            const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[j][2 * e] = bf16_to_f32(static_cast<uint16_t>(w[e] & 0xFFFFu)) * sc[2 * e];
                v[j][2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(w[e] >> 16)) * sc[2 * e + 1];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[j][e]));
        }
    }
    const float ap = fmaxf(wave_max(m), a.eps);
    const float inv = 1.0f / ap;
    int8_t *dst = a.q + static_cast<size_t>(r) * a.H;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int i = (lane + j * kWave) * 8;
        if (i < a.H) {
            const uint32_t lo = quant4(v[j][0], v[j][1], v[j][2], v[j][3], inv);
            const uint32_t hi = quant4(v[j][4], v[j][5], v[j][6], v[j][7], inv);
            *reinterpret_cast<uint2 *>(dst + i) = make_uint2(lo, hi);
        }
    }
    if (lane == 0) a.scale[r] = ap * (1.0f / 127.0f);
}

struct GatherArgs {
    const int8_t *q_tok;
    const float *xs_tok;
    const int8_t *q_rows;
    const float *xs_rows;
    const int32_t *row_token;
    const int32_t *row_group;
    const int32_t *meta;
    int E_loc, routed_by_token, shared_by_token, has_shared, H;
    int8_t *dst_q;
    float *dst_xs;
};

__global__ __launch_bounds__(256) void dbg_gather_kernel(GatherArgs a) {
    const int r = blockIdx.x;
    const int nrows = a.meta[kMetaP] + (a.has_shared ? a.meta[kMetaTAct] : 0);
    if (r >= nrows) return;
    const bool routed = a.row_group[r] < a.E_loc;
    const bool by_tok = routed ? a.routed_by_token : a.shared_by_token;
    const size_t src = by_tok ? static_cast<size_t>(a.row_token[r]) : static_cast<size_t>(r);
    const int8_t *qs = by_tok ? a.q_tok : a.q_rows;
    if (a.dst_q)
        for (int i = threadIdx.x * 16; i < a.H; i += 256 * 16)
            *reinterpret_cast<uint4 *>(a.dst_q + static_cast<size_t>(r) * a.H + i) =
                *reinterpret_cast<const uint4 *>(qs + src * a.H + i);
    if (a.dst_xs && threadIdx.x == 0) a.dst_xs[r] = by_tok ? a.xs_tok[src] : a.xs_rows[src];
}

}  // namespace

hipError_t launch_quant(const QuantArgs &a, hipStream_t s) {
    if (a.rows_max <= 0) return hipSuccess;
    const dim3 wgrid((a.rows_max + kRowsPerBlock - 1) / kRowsPerBlock), wblk(kRowsPerBlock * kWave);
    if (a.H <= 8 * 512)
        hipLaunchKernelGGL(smooth_quant_wave_kernel<8>, wgrid, wblk, 0, s, a);
    else
        hipLaunchKernelGGL(smooth_quant_kernel, dim3(a.rows_max), dim3(kTPR), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_requant(const RequantArgs &a, hipStream_t s) {
    if (a.rows_max <= 0) return hipSuccess;
    const dim3 wgrid((a.rows_max + kRowsPerBlock - 1) / kRowsPerBlock), wblk(kRowsPerBlock * kWave);
    if (a.imax <= 8 * 256)
        hipLaunchKernelGGL(requant_wave_kernel<8>, wgrid, wblk, 0, s, a);
    else if (a.imax <= 16 * 256)
        hipLaunchKernelGGL(requant_wave_kernel<16>, wgrid, wblk, 0, s, a);
    else
        hipLaunchKernelGGL(requant_kernel, dim3(a.rows_max), dim3(kTPR), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_dbg_gather(const int8_t *q_tok, const float *xs_tok, const int8_t *q_rows, const float *xs_rows,
                             const int32_t *row_token, const int32_t *row_group, const int32_t *meta, int E_loc,
                             int routed_by_token, int shared_by_token, int has_shared, int H, int rows_max,
                             int8_t *dst_q, float *dst_xs, hipStream_t s) {
    if (rows_max <= 0) return hipSuccess;
    GatherArgs a{q_tok, xs_tok, q_rows, xs_rows, row_token, row_group, meta, E_loc, routed_by_token,
                 shared_by_token, has_shared, H, dst_q, dst_xs};
    hipLaunchKernelGGL(dbg_gather_kernel, dim3(rows_max), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
