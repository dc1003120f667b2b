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
// One workgroup of 256 threads per row; each row is read once.
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
    hipLaunchKernelGGL(smooth_quant_kernel, dim3(a.rows_max), dim3(kTPR), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_requant(const RequantArgs &a, hipStream_t s) {
    if (a.rows_max <= 0) return hipSuccess;
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
