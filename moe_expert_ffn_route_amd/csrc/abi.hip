// C ABI of libmoe_w8a8: argument validation, workspace carve-up and the
// stream-ordered launch sequence of the expert block
//   route + quantisation of x -> GEMM1 (+dequant, SwiGLU)
//         -> requant -> GEMM2 (+dequant to bf16) -> combine
// which is the unfused five-op chain of "FusedDeepMoE Kernel 深度分析报告"
// sec. 9.3 with the dequant/SwiGLU/quant fused into the GEMMs' epilogues
// (sec. 6.1, 6.2, 7.2). Nothing here allocates or synchronises.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/moe_w8a8.h"
#include "internal.h"

using namespace moe;

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t up256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

moe_status_t check_dims(const moe_w8a8_dims_t *d) {
    if (!d) return MOE_ERR_INVALID_ARG;
    if (d->num_tokens < 0 || d->hidden <= 0 || d->inter <= 0 || d->share_inter < 0 || d->topk <= 0 ||
        d->moe_expert_num <= 0 || d->ep_rank_size <= 0 || d->ep_rank_id < 0 ||
        d->ep_rank_id >= d->ep_rank_size || d->moe_expert_num % d->ep_rank_size != 0)
        return MOE_ERR_INVALID_ARG;
    if (!(d->amax_eps > 0.0f) || !isfinite(d->amax_eps)) return MOE_ERR_INVALID_ARG;
    if (d->quant_mode != 1 && d->quant_mode != 2) return MOE_ERR_UNSUPPORTED;
    if (d->topk > kMaxTopK || d->num_tokens > kMaxTokens) return MOE_ERR_UNSUPPORTED;
    if (d->moe_expert_num / d->ep_rank_size > kMaxLocalExperts) return MOE_ERR_UNSUPPORTED;
    if (d->hidden % 256 || d->inter % 256 || d->share_inter % 256) return MOE_ERR_UNSUPPORTED;
    if (d->hidden > 16384 || d->inter > 16384 || d->share_inter > 16384) return MOE_ERR_UNSUPPORTED;
    if (d->weight_layout != MOE_WEIGHT_ROW_MAJOR && d->weight_layout != MOE_WEIGHT_PACKED) return MOE_ERR_INVALID_ARG;
    if (d->fuse_route_scale != 0 && d->fuse_route_scale != 1) return MOE_ERR_INVALID_ARG;
    if (d->requant_in_epilogue != 0 && d->requant_in_epilogue != 1) return MOE_ERR_INVALID_ARG;
    if (d->weight_format != MOE_WEIGHT_INT8 && d->weight_format != MOE_WEIGHT_MXFP4) return MOE_ERR_INVALID_ARG;
    if (d->weight_format == MOE_WEIGHT_MXFP4 && d->weight_layout != MOE_WEIGHT_PACKED) return MOE_ERR_UNSUPPORTED;
    if (d->quant_mode == 2) {
        const int g = d->quant_group;
        if (g != 64 && g != 128 && g != 256) return MOE_ERR_UNSUPPORTED;  // each divides H, I, I_s
        if (d->weight_format != MOE_WEIGHT_INT8 || d->fuse_route_scale) return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

// Activation scales per row of x (H / G) and of h (max(I, I_s) / G) with
// group-wise scales (quant_mode 2), else 1.
int groups_x(const moe_w8a8_dims_t *d) { return d->quant_mode == 2 ? d->hidden / d->quant_group : 1; }
int groups_h(const moe_w8a8_dims_t *d) {
    const int imax = d->inter > d->share_inter ? d->inter : d->share_inter;
    return d->quant_mode == 2 ? imax / d->quant_group : 1;
}

Layout make_layout(const moe_w8a8_dims_t *d) {
    Layout L;
    const size_t T = d->num_tokens, K = d->topk, H = d->hidden;
    const size_t TK = T * K;
    const size_t E = d->moe_expert_num / d->ep_rank_size;
    const bool shared = d->share_inter > 0;
    L.imax = d->inter > d->share_inter ? d->inter : d->share_inter;
    L.rows_max = static_cast<int>(TK + T);
    const size_t nonempty = E < TK ? E : TK;
    // rows per GEMM work item: 16 for decode batches; 256 (tall items) when
    // the routed experts average kTallMinRows rows or more; 32 otherwise.
    // FP4 weights (gemm_mx.hip) and group-wise scales (gemm.hip, gemm_wide.hip): 32 when the
    // local experts can average 16 rows or more (T*K / ep_rank_size >=
    // 16 * E_loc), else 16 (measured on MI355X with FP4 weights: 32-row items
    // take the T = 512 layer from 996 to 859 us but slow the skewed T = 64
    // layer from 305 to 328 us).
    // (the routed rows this rank can expect are T*K / ep_rank_size, as for
    // the other item-size rules)
    const bool tall = T >= kTallMinRows && TK / d->ep_rank_size >= static_cast<size_t>(kTallMinRows) * E;
    const bool mx = d->weight_format == MOE_WEIGHT_MXFP4;
    const bool grp = d->quant_mode == 2;
    const bool two_tiles = T > kChunkRowsSmall && TK / d->ep_rank_size >= static_cast<size_t>(kTileN) * E;
    L.chunk_rows = T <= kChunkRowsSmall ? kChunkRowsSmall
                   : mx || grp          ? (two_tiles ? 2 * kTileN : kChunkRowsSmall)
                   : tall               ? kChunkRowsTall
                                        : kChunkRowsLarge;
    const size_t cr = L.chunk_rows;
    L.max_chunks = static_cast<int>(nonempty + TK / cr + (shared ? (T + cr - 1) / cr : 0));
    const size_t R = L.rows_max;
    size_t o = 0;
    L.meta = o;        o = up256(o + sizeof(int32_t) * kMetaWords);
    L.offsets = o;     o = up256(o + sizeof(int32_t) * (E + 2));
    L.sorted_pair = o; o = up256(o + sizeof(int32_t) * TK);
    L.row_of_pair = o; o = up256(o + sizeof(int32_t) * TK);
    L.row_token = o;   o = up256(o + sizeof(int32_t) * R);
    L.row_group = o;   o = up256(o + sizeof(int32_t) * R);
    L.chunks = o;      o = up256(o + sizeof(int4) * L.max_chunks);
    L.q_tok = o;       o = up256(o + T * H);
    const size_t ngx = groups_x(d), ngh = groups_h(d);
    L.xs_tok = o;      o = up256(o + sizeof(float) * T * ngx);
    L.q_sm = o;        o = up256(o + R * H);  // per-pair rows [0, T*K), per-token shared rows after
    L.s_sm = o;        o = up256(o + sizeof(float) * R * ngx);
    L.h = o;           o = up256(o + sizeof(float) * R * L.imax);
    L.q_h = o;         o = up256(o + R * L.imax);
    L.hs = o;          o = up256(o + sizeof(float) * R * ngh);
    L.hs2 = o;         o = up256(o + sizeof(float) * R);  // GEMM2 row scales with the routing weight folded in
    L.z = o;           o = up256(o + sizeof(uint16_t) * TK * H);
    L.fin_count = o;   o = up256(o + sizeof(int32_t) * L.max_chunks);  // GEMM1 arrivals per chunk
    L.total = o;
    return L;
}

}  // namespace

extern "C" moe_status_t moe_w8a8_workspace_size(const moe_w8a8_dims_t *dims, size_t *bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARG;
    const moe_status_t st = check_dims(dims);
    if (st != MOE_OK) return st;
    *bytes = make_layout(dims).total;
    return MOE_OK;
}

extern "C" moe_status_t moe_w8a8_pack_weights(const int8_t *src, int8_t *dst, int64_t groups, int32_t n, int32_t k,
                                              int32_t which, void *stream) {
    if (!src || !dst || groups < 0 || n <= 0 || k <= 0 || n % 32 || k % 64) return MOE_ERR_INVALID_ARG;
    if (which != MOE_PACK_GMM1 && which != MOE_PACK_GMM2) return MOE_ERR_INVALID_ARG;
    if (!aligned(src, 16) || !aligned(dst, 16)) return MOE_ERR_INVALID_ARG;
    const uint64_t bytes = static_cast<uint64_t>(groups) * n * k;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < d0 + bytes && d0 < s0 + bytes) return MOE_ERR_INVALID_ARG;  // overlap
    if (bytes / 16 / 256 >= (1ull << 31)) return MOE_ERR_UNSUPPORTED;
    return launch_pack(src, dst, groups, n, k, which, static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK
                                                                                                  : MOE_ERR_HIP;
}

extern "C" moe_status_t moe_w8a8_packed_mx_bytes(int64_t groups, int32_t n, int32_t k, size_t *bytes) {
    if (!bytes || groups < 0 || n <= 0 || k <= 0 || n % 32 || k % 128) return MOE_ERR_INVALID_ARG;
    *bytes = static_cast<size_t>(groups) * n * (k / 2 + k / 32);
    return MOE_OK;
}

extern "C" moe_status_t moe_w8a8_pack_weights_mx(const uint8_t *data, const uint8_t *block_scale, uint8_t *dst,
                                                 int64_t groups, int32_t n, int32_t k, int32_t which, void *stream) {
    size_t bytes = 0;
    if (!data || !block_scale || !dst || moe_w8a8_packed_mx_bytes(groups, n, k, &bytes) != MOE_OK)
        return MOE_ERR_INVALID_ARG;
    if (which != MOE_PACK_GMM1 && which != MOE_PACK_GMM2) return MOE_ERR_INVALID_ARG;
    if (!aligned(data, 16) || !aligned(dst, 16)) return MOE_ERR_INVALID_ARG;
    const uint64_t nd = static_cast<uint64_t>(groups) * n * (k / 2), ns = static_cast<uint64_t>(groups) * n * (k / 32);
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst), a0 = reinterpret_cast<uintptr_t>(data),
                    b0 = reinterpret_cast<uintptr_t>(block_scale);
    if ((a0 < d0 + bytes && d0 < a0 + nd) || (b0 < d0 + bytes && d0 < b0 + ns)) return MOE_ERR_INVALID_ARG;
    if (nd / 16 / 256 >= (1ull << 31)) return MOE_ERR_UNSUPPORTED;
    return launch_pack_mx(data, block_scale, dst, groups, n, k, which, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

extern "C" moe_status_t moe_w8a8_warm(const void *ptr, size_t bytes, void *stream) {
    if (bytes == 0) return MOE_OK;
    if (!ptr || !aligned(ptr, 16) || bytes % 16) return MOE_ERR_INVALID_ARG;
    return launch_warm(ptr, bytes, static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status_t moe_w8a8_read_probe(const void *ptr, size_t bytes, void *stream) {
    if (bytes == 0) return MOE_OK;
    if (!ptr || !aligned(ptr, 16) || bytes % 16) return MOE_ERR_INVALID_ARG;
    return launch_read_probe(ptr, bytes, static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status_t moe_w8a8_read_write_probe(const void *src, size_t src_bytes, void *dst, size_t dst_bytes,
                                                  void *stream) {
    if (src_bytes % (256 * 1024) || dst_bytes % 16 || dst_bytes > src_bytes) return MOE_ERR_INVALID_ARG;
    if (src_bytes == 0) return MOE_OK;
    if (!src || !aligned(src, 16) || src_bytes / (256 * 1024) > 0x7FFFFFFFu) return MOE_ERR_INVALID_ARG;
    if (dst_bytes > 0) {
        if (!dst || !aligned(dst, 16)) return MOE_ERR_INVALID_ARG;
        const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
        if (s0 < d0 + dst_bytes && d0 < s0 + src_bytes) return MOE_ERR_INVALID_ARG;  // overlap
    }
    return launch_rw_probe(src, src_bytes, dst, dst_bytes, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MOE_OK
               : MOE_ERR_HIP;
}

extern "C" const char *moe_w8a8_status_string(moe_status_t s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument (NULL or misaligned pointer, or inconsistent sizes)";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_SCRATCH_LIMIT:
            return "the call needs more scratch than moe_w8a8_forward_noalloc's built-in buffer holds "
                   "(use moe_w8a8_forward with a workspace)";
    }
    return "unknown status";
}

// Host-side checks of a forward call's sizes and pointers (not the
// workspace): nothing is launched unless this returns MOE_OK.
static moe_status_t check_call(const moe_w8a8_dims_t *d, const void *x, const int32_t *expert_ids,
                               const float *expert_scales, const int8_t *gmm1_weight, const float *gmm1_weight_scale,
                               const int8_t *gmm2_weight, const float *gmm2_weight_scale,
                               const int8_t *share_gmm1_weight, const float *share_gmm1_weight_scale,
                               const int8_t *share_gmm2_weight, const float *share_gmm2_weight_scale,
                               const float *expert_smooth_scales, const float *share_smooth_scales, void *output,
                               void *share_output, int32_t *expert_token_nums) {
    const moe_status_t st = check_dims(d);
    if (st != MOE_OK) return st;
    const bool shared = d->share_inter > 0;
    const int n_share_ptrs = (share_gmm1_weight != nullptr) + (share_gmm1_weight_scale != nullptr) +
                             (share_gmm2_weight != nullptr) + (share_gmm2_weight_scale != nullptr);
    const bool need_tok = d->num_tokens > 0;
    if ((need_tok && (!x || !expert_ids || !expert_scales || !output)) || !gmm1_weight || !gmm1_weight_scale ||
        !gmm2_weight || !gmm2_weight_scale || !expert_token_nums)
        return MOE_ERR_INVALID_ARG;
    if (shared ? (n_share_ptrs != 4 || (need_tok && !share_output)) : (n_share_ptrs != 0 || share_smooth_scales))
        return MOE_ERR_INVALID_ARG;
    const void *a16[] = {x, output, gmm1_weight, gmm2_weight, share_gmm1_weight, share_gmm2_weight,
                         expert_smooth_scales, share_smooth_scales, shared ? share_output : nullptr};
    for (const void *p : a16)
        if (p && !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
    const void *a4[] = {expert_ids, expert_scales, gmm1_weight_scale, gmm2_weight_scale,
                        share_gmm1_weight_scale, share_gmm2_weight_scale, expert_token_nums};
    for (const void *p : a4)
        if (p && !aligned(p, 4)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

// The block on a caller-given workspace (both forward entry points).
static moe_status_t forward_impl(const moe_w8a8_dims_t *d, const void *x, const int32_t *expert_ids,
                                 const float *expert_scales, const int8_t *gmm1_weight, const float *gmm1_weight_scale,
                                 const int8_t *gmm2_weight, const float *gmm2_weight_scale,
                                 const int8_t *share_gmm1_weight, const float *share_gmm1_weight_scale,
                                 const int8_t *share_gmm2_weight, const float *share_gmm2_weight_scale,
                                 const float *expert_smooth_scales, const float *share_smooth_scales,
                                 const uint8_t *x_active_mask, void *output, void *share_output,
                                 int32_t *expert_token_nums, void *workspace, size_t workspace_bytes,
                                 const moe_w8a8_debug_t *dbg, void *stream) {
    const moe_status_t st = check_call(d, x, expert_ids, expert_scales, gmm1_weight, gmm1_weight_scale, gmm2_weight,
                                       gmm2_weight_scale, share_gmm1_weight, share_gmm1_weight_scale,
                                       share_gmm2_weight, share_gmm2_weight_scale, expert_smooth_scales,
                                       share_smooth_scales, output, share_output, expert_token_nums);
    if (st != MOE_OK) return st;
    const bool shared = d->share_inter > 0;
    const Layout L = make_layout(d);
    if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MOE_ERR_INVALID_ARG;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    auto I32 = [&](size_t off) { return reinterpret_cast<int32_t *>(ws + off); };
    int32_t *meta = I32(L.meta);
    const int T = d->num_tokens, K = d->topk, H = d->hidden;
    const int E = d->moe_expert_num / d->ep_rank_size;
    const moe_w8a8_debug_t nodbg = {};
    const moe_w8a8_debug_t &D = dbg ? *dbg : nodbg;
    auto mark = [&](int i) {
        return !D.stage_events || !D.stage_events[i] ||
               hipEventRecord(static_cast<hipEvent_t>(D.stage_events[i]), s) == hipSuccess;
    };
    if (!mark(0)) return MOE_ERR_HIP;
    auto kev = [&](int i) {
        return D.kernel_events ? static_cast<hipEvent_t>(D.kernel_events[i]) : static_cast<hipEvent_t>(nullptr);
    };

    // GEMM1 input rows: per token (quantised once, in the routing launch)
    // for groups without smooth scales, per grouped row otherwise
    const bool routed_tok = expert_smooth_scales == nullptr;
    const bool shared_tok = shared && share_smooth_scales == nullptr;

    RouteArgs ra;
    ra.ids = expert_ids;
    ra.mask = x_active_mask;
    ra.T = T;
    ra.K = K;
    ra.E_g = d->moe_expert_num;
    ra.E_loc = E;
    ra.base = d->ep_rank_id * E;
    ra.has_shared = shared;
    ra.chunk_rows = L.chunk_rows;
    ra.counts_out = expert_token_nums;
    ra.offsets = I32(L.offsets);
    ra.sorted_pair = I32(L.sorted_pair);
    ra.row_of_pair = I32(L.row_of_pair);
    ra.row_token = I32(L.row_token);
    ra.row_group = I32(L.row_group);
    ra.chunks = reinterpret_cast<int4 *>(ws + L.chunks);
    ra.meta = meta;
    ra.dbg_shared_token = D.shared_token;
    // requantisation in GEMM1's epilogue: where the decode GEMM runs (16-row
    // work items, INT8 weights, one scale per row)
    const bool fin = d->requant_in_epilogue && d->weight_format == MOE_WEIGHT_INT8 && d->quant_mode == 1 &&
                     L.chunk_rows == kChunkRowsSmall;
    ra.zero_words = fin ? I32(L.fin_count) : nullptr;
    ra.n_zero = fin ? L.max_chunks : 0;
    TokQuantArgs tq;
    tq.x = static_cast<const uint16_t *>(x);
    tq.mask = x_active_mask;
    tq.T = T;
    tq.H = H;
    tq.eps = d->amax_eps;
    tq.ids = expert_ids;
    tq.K = K;
    tq.E_g = d->moe_expert_num;
    tq.E_loc = E;
    tq.base = ra.base;
    tq.q_tok = (T > 0 && (routed_tok || shared_tok)) ? reinterpret_cast<int8_t *>(ws + L.q_tok) : nullptr;
    tq.s_tok = reinterpret_cast<float *>(ws + L.xs_tok);
    tq.smooth = T > 0 ? expert_smooth_scales : nullptr;
    tq.share_smooth = T > 0 && shared ? share_smooth_scales : nullptr;
    tq.q_sm = reinterpret_cast<int8_t *>(ws + L.q_sm);
    tq.s_sm = reinterpret_cast<float *>(ws + L.s_sm);
    const bool mx = d->weight_format == MOE_WEIGHT_MXFP4;
    const bool grp = d->quant_mode == 2;
    const int ngx = groups_x(d), ngh = groups_h(d);
    tq.fp8 = mx;
    tq.ng = ngx;
    tq.gl = grp ? d->quant_group / 8 : 0;
    if (launch_route_quant(ra, tq, s) != hipSuccess || !mark(1)) return MOE_ERR_HIP;

    // GEMM1's activation rows: per token (q_tok, index row_token) or per
    // (token, expert) pair (q_sm, index sorted_pair) for routed rows; per
    // token, plain (q_tok) or with the shared smooth scales (q_sm rows T*K..),
    // for shared rows
    auto gemm1_inputs = [&] {
        GemmArgs g = {};
        const size_t sh_row0 = static_cast<size_t>(T) * K;
        g.a_stride = H;
        g.H = H;
        g.E_loc = E;
        g.row_token = ra.row_token;
        g.A_r = routed_tok ? tq.q_tok : tq.q_sm;
        g.a_scale_r = routed_tok ? tq.s_tok : tq.s_sm;
        g.idx_r = routed_tok ? ra.row_token : ra.sorted_pair;
        g.A_s = shared_tok ? tq.q_tok : tq.q_sm + sh_row0 * H;
        g.a_scale_s = shared_tok ? tq.s_tok : tq.s_sm + sh_row0 * ngx;
        g.a_ng = ngx;
        g.gsteps = grp ? d->quant_group / 64 : 0;
        return g;
    };
    if (T > 0) {
        GemmArgs g1 = gemm1_inputs();
        g1.W = gmm1_weight;
        g1.Ws = gmm1_weight_scale;
        g1.W_sh = share_gmm1_weight;
        g1.Ws_sh = share_gmm1_weight_scale;
        g1.I = d->inter;
        g1.I_s = d->share_inter;
        g1.H = H;
        g1.E_loc = E;
        g1.imax = L.imax;
        g1.g_lo = 0;
        g1.g_hi = E + 1;
        g1.packed = d->weight_layout == MOE_WEIGHT_PACKED;
        g1.mt = L.chunk_rows / kTileN;
        // three INT8 kernels by chunk size: decode (gemm.hip), wide
        // (gemm_wide.hip) and tall (gemm_tall.hip) work items; group-wise
        // scales: gemm.hip (16-row items) or gemm_wide.hip (32-row items);
        // FP4 weights: gemm_mx.hip
        const bool tall = !mx && !grp && g1.mt == kTallTiles, wide = !mx && g1.mt == kWideTiles;
        // tile pairs per work item
        const int nw = tall ? kTallPairs : wide ? wide_tile_pairs() : (mx && g1.mt == 2) ? mx_wide_tile_pairs(1) : 1;
        const int nw2 = mx && g1.mt == 2 ? mx_wide_tile_pairs(2) : nw;
        g1.n_tiles = L.imax / kTileN / nw;
        g1.chunks = ra.chunks;
        g1.count_word = kMetaChunks;
        g1.meta = meta;
        g1.row_token = ra.row_token;
        g1.h = reinterpret_cast<float *>(ws + L.h);
        g1.dbg_acc = D.acc1;
        const bool fused = d->fuse_route_scale != 0;
        if (fin) {
            g1.fin_count = I32(L.fin_count);
            g1.fin_q = reinterpret_cast<int8_t *>(ws + L.q_h);
            g1.fin_scale = reinterpret_cast<float *>(ws + L.hs);
            g1.fin_scale2 = fused ? reinterpret_cast<float *>(ws + L.hs2) : nullptr;
            g1.fin_route_w = expert_scales;
            g1.fin_sorted_pair = ra.sorted_pair;
            g1.fin_eps = d->amax_eps;
        }
        const hipError_t e1 = mx     ? launch_gemm1_mx(g1, L.max_chunks, s, kev(0), kev(1))
                              : tall ? launch_gemm1_tall(g1, L.max_chunks, s, kev(0), kev(1))
                              : wide ? launch_gemm1_wide(g1, L.max_chunks, s, kev(0), kev(1))
                                     : launch_gemm1(g1, L.max_chunks, s, kev(0), kev(1));
        if (e1 != hipSuccess || !mark(2)) return MOE_ERR_HIP;

        RequantArgs rq;
        rq.h = g1.h;
        rq.row_group = ra.row_group;
        rq.meta = meta;
        rq.E_loc = E;
        rq.I = d->inter;
        rq.I_s = d->share_inter;
        rq.imax = L.imax;
        rq.has_shared = shared;
        rq.rows_max = L.rows_max;
        rq.load_early = d->ep_rank_size == 1;  // then nearly every grouped row is in use
        rq.rows_expected = static_cast<int>(static_cast<size_t>(T) * K / d->ep_rank_size) + (shared ? T : 0);
        rq.eps = d->amax_eps;
        rq.q = reinterpret_cast<int8_t *>(ws + L.q_h);
        rq.scale = reinterpret_cast<float *>(ws + L.hs);
        rq.scale2 = fused ? reinterpret_cast<float *>(ws + L.hs2) : nullptr;
        rq.route_w = expert_scales;
        rq.sorted_pair = ra.sorted_pair;
        rq.fp8 = mx;
        rq.ng = ngh;
        rq.gl = grp ? d->quant_group / 4 : 0;
        if ((!fin && launch_requant(rq, s) != hipSuccess) || !mark(3)) return MOE_ERR_HIP;

        GemmArgs g2 = g1;
        g2.A = rq.q;
        g2.a_stride = L.imax;
        g2.a_scale = fused ? rq.scale2 : rq.scale;
        g2.a_ng = ngh;
        g2.W = gmm2_weight;
        g2.Ws = gmm2_weight_scale;
        g2.W_sh = share_gmm2_weight;
        g2.Ws_sh = share_gmm2_weight_scale;
        g2.n_tiles = H / (2 * kTileN) / nw2;
        g2.h = nullptr;
        g2.fin_count = nullptr;
        g2.z = reinterpret_cast<uint16_t *>(ws + L.z);
        g2.zrow = ra.sorted_pair;  // routed z rows in pair order: combine reads row t*K + k
        g2.share_out = static_cast<uint16_t *>(share_output);
        g2.dbg_acc = D.acc2;
        g2.dbg_z = D.z;
        // the contraction length of GEMM2 is the group's intermediate size
        auto gemm2 = [&](int k_dim, hipEvent_t e0, hipEvent_t e1) {
            return mx     ? launch_gemm2_mx(g2, L.max_chunks, k_dim, s, e0, e1)
                   : tall ? launch_gemm2_tall(g2, L.max_chunks, k_dim, s, e0, e1)
                   : wide ? launch_gemm2_wide(g2, L.max_chunks, k_dim, s, e0, e1)
                          : launch_gemm2(g2, L.max_chunks, k_dim, s, e0, e1);
        };
        if (!shared || d->share_inter == d->inter) {
            if (gemm2(d->inter, kev(2), kev(3)) != hipSuccess) return MOE_ERR_HIP;
        } else {
            g2.g_hi = E;
            if (gemm2(d->inter, kev(2), nullptr) != hipSuccess) return MOE_ERR_HIP;
            g2.g_lo = E;
            g2.g_hi = E + 1;
            if (gemm2(d->share_inter, nullptr, kev(3)) != hipSuccess) return MOE_ERR_HIP;
        }
        if (!mark(4)) return MOE_ERR_HIP;

        CombineArgs ca;
        ca.z = g2.z;
        ca.row_of_pair = ra.row_of_pair;
        ca.scales = expert_scales;
        ca.mask = x_active_mask;
        ca.T = T;
        ca.K = K;
        ca.H = H;
        ca.has_shared = shared;
        ca.fused = fused;
        ca.out = static_cast<uint16_t *>(output);
        ca.share_out = static_cast<uint16_t *>(share_output);
        if (launch_combine(ca, s) != hipSuccess || !mark(5)) return MOE_ERR_HIP;
    } else {
        for (int i = 2; i < 6; ++i)
            if (!mark(i)) return MOE_ERR_HIP;
    }

    // optional intermediates that live in the workspace
    struct Copy { void *dst; size_t off, bytes; };
    const size_t R = L.rows_max, TK = static_cast<size_t>(T) * K;
    const Copy copies[] = {
        {D.sorted_pair, L.sorted_pair, sizeof(int32_t) * TK},
        {D.row_of_pair, L.row_of_pair, sizeof(int32_t) * TK},
        {D.group_offset, L.offsets, sizeof(int32_t) * (E + 1)},
        {D.num_rows, L.meta, sizeof(int32_t) * kMetaWords},
        {D.h, L.h, sizeof(float) * R * L.imax},
        {D.q_h, L.q_h, R * L.imax},
        {D.hs, L.hs, sizeof(float) * R * ngh},
    };
    if ((D.q_x || D.xs) &&
        launch_dbg_gather(gemm1_inputs(), I32(L.row_group), meta, shared, L.rows_max, D.q_x, D.xs, s) != hipSuccess)
        return MOE_ERR_HIP;
    for (const Copy &c : copies)
        if (c.dst && c.bytes && hipMemcpyAsync(c.dst, ws + c.off, c.bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return MOE_ERR_HIP;
    return MOE_OK;
}

extern "C" moe_status_t moe_w8a8_forward(const moe_w8a8_dims_t *d, const void *x, const int32_t *expert_ids,
                                         const float *expert_scales, const int8_t *gmm1_weight,
                                         const float *gmm1_weight_scale, const int8_t *gmm2_weight,
                                         const float *gmm2_weight_scale, const int8_t *share_gmm1_weight,
                                         const float *share_gmm1_weight_scale, const int8_t *share_gmm2_weight,
                                         const float *share_gmm2_weight_scale, const float *expert_smooth_scales,
                                         const float *share_smooth_scales, const uint8_t *x_active_mask,
                                         void *output, void *share_output, int32_t *expert_token_nums,
                                         void *workspace, size_t workspace_bytes, const moe_w8a8_debug_t *dbg,
                                         void *stream) {
    return forward_impl(d, x, expert_ids, expert_scales, gmm1_weight, gmm1_weight_scale, gmm2_weight,
                        gmm2_weight_scale, share_gmm1_weight, share_gmm1_weight_scale, share_gmm2_weight,
                        share_gmm2_weight_scale, expert_smooth_scales, share_smooth_scales, x_active_mask, output,
                        share_output, expert_token_nums, workspace, workspace_bytes, dbg, stream);
}

// ---------------------------------------------------------------------------
// The entry point that allocates nothing: the workspace is a device-resident
// array of this library. Each GPU the library runs on holds its own copy from
// module load until the process ends. In host code `scratch` names only a
// host-side stand-in for the symbol, never device memory: the array's device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is ever handed to kernels or copies.
static __device__ __align__(256) unsigned char scratch[MOE_W8A8_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch` array (null on failure).
void *scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        if (reinterpret_cast<uintptr_t>(p) % 256) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" moe_status_t moe_w8a8_forward_noalloc(
    const moe_w8a8_dims_t *d, const void *x, const int32_t *expert_ids, const float *expert_scales,
    const int8_t *gmm1_weight, const float *gmm1_weight_scale, const int8_t *gmm2_weight,
    const float *gmm2_weight_scale, const int8_t *share_gmm1_weight, const float *share_gmm1_weight_scale,
    const int8_t *share_gmm2_weight, const float *share_gmm2_weight_scale, const float *expert_smooth_scales,
    const float *share_smooth_scales, const uint8_t *x_active_mask, void *output, void *share_output,
    int32_t *expert_token_nums, const moe_w8a8_debug_t *dbg, void *stream) {
    const moe_status_t st = check_call(d, x, expert_ids, expert_scales, gmm1_weight, gmm1_weight_scale, gmm2_weight,
                                       gmm2_weight_scale, share_gmm1_weight, share_gmm1_weight_scale,
                                       share_gmm2_weight, share_gmm2_weight_scale, expert_smooth_scales,
                                       share_smooth_scales, output, share_output, expert_token_nums);
    if (st != MOE_OK) return st;
    if (make_layout(d).total > static_cast<size_t>(MOE_W8A8_NOALLOC_SCRATCH_BYTES)) return MOE_ERR_SCRATCH_LIMIT;
    void *ws = scratch_on_current_device();
    if (!ws) return MOE_ERR_HIP;
    return forward_impl(d, x, expert_ids, expert_scales, gmm1_weight, gmm1_weight_scale, gmm2_weight,
                        gmm2_weight_scale, share_gmm1_weight, share_gmm1_weight_scale, share_gmm2_weight,
                        share_gmm2_weight_scale, expert_smooth_scales, share_smooth_scales, x_active_mask, output,
                        share_output, expert_token_nums, ws, MOE_W8A8_NOALLOC_SCRATCH_BYTES, dbg, stream);
}
