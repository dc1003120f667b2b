// Internal definitions shared by the HIP sources of libmoe_w8a8 (not part of
// the public C ABI in include/moe_w8a8.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kMaxLocalExperts = 512;
constexpr int kRouteThreads = 1024;  // the routing kernel runs as one workgroup
constexpr int kRouteWaves = kRouteThreads / kWave;
// Grouped rows per GEMM work item (INT8 weights, one scale per row): one
// 16-row MFMA tile when T <= 16 (decode; gemm.hip), MOE_WIDE_MT tiles
// otherwise (gemm_wide.hip, which shares each chunk's activations across the
// waves of a workgroup), or tall items (below). Group-wise scales and FP4
// weights run 16-row items, or 32-row ones when the local experts can average
// 16 rows or more (group-wise: gemm.hip / gemm_wide.hip; FP4: gemm_mx.hip).
#ifndef MOE_WIDE_MT
#define MOE_WIDE_MT 2
#endif
constexpr int kWideTiles = MOE_WIDE_MT;
constexpr int kChunkRowsSmall = 16;
constexpr int kChunkRowsLarge = 16 * MOE_WIDE_MT;
// When the routed experts can average at least kTallMinRows rows (T * K /
// ep_rank_size >= kTallMinRows * E_loc), every group is cut into chunks of kChunkRowsTall rows
// instead: tall work items (gemm_tall.hip), each covering kTallPairs pairs of
// 16-row weight tiles with both operands staged through LDS.
#ifndef MOE_TALL_MIN_ROWS
#define MOE_TALL_MIN_ROWS 256
#endif
constexpr int kTallTiles = 16;
constexpr int kChunkRowsTall = 16 * kTallTiles;
#ifndef MOE_TBIG_PAIRS
#define MOE_TBIG_PAIRS 8
#endif
constexpr int kTallPairs = MOE_TBIG_PAIRS;
constexpr int kTallMinRows = MOE_TALL_MIN_ROWS;
constexpr int kTileN = 16;           // MFMA 16x16x64 output tile edge
// A chunk entry's third word holds its row count (<= 256) in the low bits and
// the number of chunks of its group above kChunkCountShift.
constexpr int kChunkCountShift = 9;
constexpr int kChunkRowsMask = (1 << kChunkCountShift) - 1;
static_assert(kChunkRowsLarge <= kChunkRowsMask && kChunkRowsTall <= kChunkRowsMask,
              "chunk rows must fit below the count bits");
constexpr int kMaxTopK = 16;
constexpr int kMaxTokens = 1 << 16;

// meta words written by the routing kernel
enum { kMetaP = 0, kMetaTAct = 1, kMetaBad = 2, kMetaChunks = 3, kMetaWords = 4 };

// Carve-up of the caller's workspace (byte offsets, 256-aligned).
struct Layout {
    int rows_max;    // T*K + T grouped-row capacity
    int max_chunks;  // upper bound of GEMM work items
    int chunk_rows;  // rows per GEMM work item
    int imax;        // max(I, I_s)
    size_t meta, offsets, sorted_pair, row_of_pair, row_token, row_group, chunks;
    size_t q_tok, xs_tok, q_sm, s_sm, h, q_h, hs, hs2, z, fin_count, total;
};

struct RouteArgs {
    const int32_t *ids;
    const uint8_t *mask;
    int T, K, E_g, E_loc, base, has_shared;
    int chunk_rows;        // rows per GEMM work item
    int32_t *counts_out;   // expert_token_nums [E_loc]
    int32_t *offsets;      // [E_loc + 2]
    int32_t *sorted_pair;  // [T*K]
    int32_t *row_of_pair;  // [T*K]
    int32_t *row_token;    // [rows_max]
    int32_t *row_group;    // [rows_max]
    int4 *chunks;          // [max_chunks] (group, first row, rows | count << kChunkCountShift, index)
    int32_t *meta;         // [kMetaWords]
    int32_t *dbg_shared_token;  // [T] or null
    int32_t *zero_words;   // [n_zero] counters of later launches of this call, cleared here (or null)
    int n_zero;
};

// Quantisation of x in the routing launch, which needs no routing result:
//   - per token (x[t]) into q_tok, for groups without smooth scales;
//   - per (token, expert) pair p = t * K + k (x[t] * smooth[e]) into rows
//     [0, T*K) of q_sm, for routed rows when expert smooth scales are given
//     (pairs that are not kept are skipped);
//   - per token (x[t] * share_smooth) into rows [T*K, T*K + T) of q_sm, for
//     the shared expert when its smooth scales are given.
struct TokQuantArgs {
    const uint16_t *x;     // bf16 [T, H]
    const uint8_t *mask;   // [T] or null
    const int32_t *ids;    // [T, K] global expert ids
    int T, K, H, E_g, E_loc, base;
    float eps;
    int8_t *q_tok;         // [T, H]; null = not needed
    float *s_tok;          // [T]
    const float *smooth;        // [E_loc, H] or null
    const float *share_smooth;  // [H] or null
    int8_t *q_sm;          // [T*K + T, H]
    float *s_sm;           // [T*K + T]
    int fp8;               // quantise to FP8 E4M3 codes instead of INT8
    int ng;                // scales per row: H / G with group-wise scales, else 1
    int gl;                // group-wise scales: lanes per group (G / 8), else 0
};

struct RequantArgs {
    const float *h;           // [rows_max, imax]
    const int32_t *row_group;
    const int32_t *meta;
    int E_loc, I, I_s, imax, has_shared, rows_max;
    int load_early;  // read each h row before the row count is known (all pairs local)
    int rows_expected;  // grouped rows the batch can use: T*K / ep_rank_size (+ T with a shared expert)
    float eps;
    int8_t *q;     // [rows_max, imax]
    float *scale;  // [rows_max]
    // fused route scale: scale2[r] = scale[r] * route_w[sorted_pair[r]] for
    // routed rows, scale[r] for shared rows (null: not fused)
    float *scale2;
    const float *route_w;        // [T*K]
    const int32_t *sorted_pair;  // [P]
    int fp8;                     // FP8 E4M3 codes instead of INT8
    int ng;                      // scale stride per row: Imax / G with group-wise scales, else 1
    int gl;                      // group-wise scales: lanes per group (G / 4), else 0
};

struct GemmArgs {
    // GEMM2 activations: grouped int8 rows (row r of A) and their scales
    const int8_t *A;
    int a_stride;
    const float *a_scale;
    // GEMM1 activations: routed row r reads row idx_r[r] of A_r (the token's
    // row of q_tok, or the pair's row of q_sm), a shared row reads row
    // row_token[r] of A_s
    const int8_t *A_r, *A_s;
    const float *a_scale_r, *a_scale_s;
    const int32_t *idx_r;
    // weights [E_loc, N, K] routed, [N, K] shared, and per-output-channel scales
    const int8_t *W;
    const float *Ws;
    const int8_t *W_sh;
    const float *Ws_sh;
    int I, I_s, H, E_loc, imax;
    int g_lo, g_hi;   // only chunks of groups in [g_lo, g_hi)
    int packed;       // weights in moe_w8a8_pack_weights order
    int gsteps;       // group-wise activation scales: 64-byte K steps per group (0: one scale per row)
    int a_ng;         // activation scales per row (1 without group-wise scales)
    int mt;           // 16-row MFMA tiles per chunk
    int n_tiles;      // work items per chunk along N
    const int4 *chunks;
    int count_word;   // meta word holding the number of chunks
    const int32_t *meta;
    const int32_t *row_token;
    // outputs
    float *h;              // GEMM1: [rows_max, imax]
    uint16_t *z;           // GEMM2 routed rows: [T*K, H] bf16, routed row r at row zrow[r] (its pair id)
    const int32_t *zrow;   // [P] pair id of routed row r (sorted_pair)
    uint16_t *share_out;   // GEMM2 shared rows: [T, H] bf16 indexed by token
    int32_t *dbg_acc;      // optional [rows_max, 2*imax] (GEMM1) / [rows_max, H] (GEMM2)
    uint16_t *dbg_z;       // optional [rows_max, H]
    // Requantisation in GEMM1's epilogue (decode kernel, INT8, one scale per
    // row): every N-tile block of a chunk publishes its h values with
    // agent-coherent stores and counts itself in fin_count[chunk]; the last
    // block to arrive quantises the chunk's rows (q_h, hs) as the requant
    // kernel would. No block waits for another. null: separate requant launch.
    int32_t *fin_count;           // [max_chunks], zeroed by the routing launch of the same call
    int8_t *fin_q;                // q_h [rows_max, imax]
    float *fin_scale;             // hs [rows_max]
    float *fin_scale2;            // fused route scale: hs * route weight (routed rows), else null
    const float *fin_route_w;     // [T*K]
    const int32_t *fin_sorted_pair;  // [P]
    float fin_eps;
};

struct CombineArgs {
    const uint16_t *z;
    const int32_t *row_of_pair;
    const float *scales;
    const uint8_t *mask;
    int T, K, H, has_shared;
    int fused;  // the routing weights are already in the z rows: only sum
    uint16_t *out;
    uint16_t *share_out;
};

hipError_t launch_route_quant(const RouteArgs &a, const TokQuantArgs &q, hipStream_t s);
hipError_t launch_requant(const RequantArgs &a, hipStream_t s);
// ev_start / ev_stop (may be null) are bound to the kernel launch itself.
hipError_t launch_gemm1(const GemmArgs &a, int max_chunks, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_gemm2(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t ev_start,
                        hipEvent_t ev_stop);
// Wide work items (gemm_wide.hip; a.mt = kWideTiles): n_tiles counts groups
// of wide_tile_pairs() pairs of 16-row weight tiles.
hipError_t launch_gemm1_wide(const GemmArgs &a, int max_chunks, hipStream_t s, hipEvent_t ev_start,
                             hipEvent_t ev_stop);
hipError_t launch_gemm2_wide(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t ev_start,
                             hipEvent_t ev_stop);
int wide_tile_pairs();
// Tall work items (gemm_tall.hip; a.mt = kTallTiles): n_tiles counts groups
// of kTallPairs pairs of 16-row weight tiles.
hipError_t launch_gemm1_tall(const GemmArgs &a, int max_chunks, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_gemm2_tall(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t ev_start,
                             hipEvent_t ev_stop);
// FP4-weight / FP8-activation GEMMs (gemm_mx.hip): work items of one or two
// 16-row tiles (a.mt = 1 or 2), weights from moe_w8a8_pack_weights_mx, A codes
// FP8 E4M3; k_dim % 256 == 0. dbg_acc receives fp32 bit patterns.
hipError_t launch_gemm1_mx(const GemmArgs &a, int max_chunks, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_gemm2_mx(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t ev_start,
                           hipEvent_t ev_stop);
// Tile pairs per work item of the two-tile (32-row) FP4-weight kernel, for
// GEMM1 (kind 1) or GEMM2 (kind 2).
int mx_wide_tile_pairs(int kind);
hipError_t launch_combine(const CombineArgs &a, hipStream_t s);
// Reads [ptr, ptr + bytes) once and discards it (a cache warm); bytes % 16 == 0.
hipError_t launch_warm(const void *ptr, size_t bytes, hipStream_t s);
hipError_t launch_read_probe(const void *ptr, size_t bytes, hipStream_t s);
hipError_t launch_rw_probe(const void *src, size_t src_bytes, void *dst, size_t dst_bytes, hipStream_t s);
hipError_t launch_pack(const int8_t *src, int8_t *dst, int64_t groups, int n, int k, int which, hipStream_t s);
hipError_t launch_pack_mx(const uint8_t *data, const uint8_t *bscale, uint8_t *dst, int64_t groups, int n, int k,
                          int which, hipStream_t s);
// debug only: the GEMM1 input rows of every grouped row (q_x / xs dump)
hipError_t launch_dbg_gather(const GemmArgs &g1, const int32_t *row_group, const int32_t *meta, int has_shared,
                             int rows_max, int8_t *dst_q, float *dst_xs, hipStream_t s);

// Position of 16-row tile t in a packed GEMM1 weight whose gate half holds
// `half` tiles: gate and up tiles alternate (gate j, up j, gate j + 1, ...),
// so the two tiles a GEMM1 work item streams lie side by side.
__host__ __device__ __forceinline__ size_t g1_tile_pos(int t, int half) {
    return t < half ? 2 * static_cast<size_t>(t) : 2 * static_cast<size_t>(t - half) + 1;
}

// bf16 helpers (round to nearest even)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// GEMM epilogues, one fp32 operation per step in this order (every GEMM
// kernel uses these, so all of them round alike):
//   dequant ("FusedDeepMoE Kernel 深度分析报告" sec. 6.1, 6.2):
//     y = (float(acc) * w_scale[n]) * row_scale[r];
//   SwiGLU (sec. 6.1): h = (y_g / (1 + exp(-y_g))) * y_u.
// The accumulator is int32 (INT8 GEMMs) or fp32 (FP4-weight GEMMs).
template <typename Acc>
__device__ __forceinline__ float dequant(Acc acc, float w_scale, float row_scale) {
    const float y = static_cast<float>(acc) * w_scale;
    return y * row_scale;
}
__device__ __forceinline__ float swiglu_y(float yg, float yu) {
    const float ex = expf(-yg);
    const float den = 1.0f + ex;
    const float sg = yg / den;
    return sg * yu;
}
template <typename Acc>
__device__ __forceinline__ float swiglu(Acc acc_g, Acc acc_u, float ws_g, float ws_u, float row_scale) {
    return swiglu_y(dequant(acc_g, ws_g, row_scale), dequant(acc_u, ws_u, row_scale));
}

}  // namespace moe
