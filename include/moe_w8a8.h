/*
 * moe_w8a8 -- fused W8A8 MoE expert block for AMD MI355X (gfx950).
 *
 * One call runs the expert block of a DeepSeek-style decode step on one GPU:
 *   1. dispatch grouping: per-local-expert token counts (expert_token_nums),
 *      their exclusive prefix sum and the stable (expert, token, k) row order;
 *   2. per-row dynamic INT8 quantisation of x (optionally times smooth scales);
 *   3. grouped INT8 GEMM1 (gate and up halves) with exact int32 accumulation;
 *   4. dequantisation by per-output-channel weight scale x per-row scale,
 *      SwiGLU, and per-row INT8 requantisation;
 *   5. grouped INT8 GEMM2 (down) and dequantisation to bf16;
 *   6. routing-weighted top-k combine into `output`, and the optional shared
 *      expert on every active token into `share_output`.
 * Options of the same call (moe_w8a8_dims_t): the routing weight folded into
 * GEMM2's row scale (fuse_route_scale), group-wise activation scales
 * (quant_mode 2), and FP4 weights with FP8 activations (weight_format).
 *
 * Passages that define the operation (pages, by title):
 *   "FusedDeepMoE Kernel 深度分析报告": sec. 1.2 (inputs, outputs, attributes),
 *     sec. 2.1 (tiling info: ep size/rank, experts per rank, bs, k, h, 2*inter),
 *     sec. 4.1 (dispatch: counts, prefix sum, quantisation fused in dispatch),
 *     sec. 4.2 (combine: fp32 sum over k of row x routing weight, one bf16 cast),
 *     sec. 6.1 (int32 -> fp32, x weight scale per column, x per-token scale,
 *               left half x/(1+exp(-x))), sec. 6.2 (same dequant, cast to bf16),
 *     sec. 7.2 (BlockQuant: scale = max|h|/127, q = rint(h*127/max)),
 *     sec. 9.4 (supported ranges).
 *   "DeepSeek V4 Decode Optimization" sec. 0: INT8 weights with FP32
 *     per-output-channel scales; activations quantised per token, amax
 *     floored by an eps and rescaled to 127; scales stay FP32.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers, row-major, owned by the caller; the
 *     library never frees or retains them. 16-byte alignment is required for
 *     x, output, share_output and every weight; the workspace must be 256-byte
 *     aligned.
 *   - Calls are stream-ordered and asynchronous: no host synchronisation, no
 *     allocation. The library keeps no state between calls, so calls are
 *     reentrant when each uses its own workspace; two calls in flight that
 *     share one workspace race.
 *   - Host-detectable errors (bad sizes, NULL required pointers, misaligned
 *     pointers, short workspace) return a negative status and launch nothing.
 *     A pair whose expert id lies outside [0, moe_expert_num) is dropped and
 *     counted in a diagnostics word (readable through moe_w8a8_debug_t).
 *     HIP launch failures return MOE_ERR_HIP; faults inside kernels surface at
 *     the caller's next synchronisation.
 */
#ifndef MOE_W8A8_H
#define MOE_W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define MOE_W8A8_API __attribute__((visibility("default")))
#else
#define MOE_W8A8_API
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* NULL / misaligned pointer, inconsistent sizes */
    MOE_ERR_UNSUPPORTED = -2, /* legal for the operator, outside what this library runs */
    MOE_ERR_WORKSPACE = -3,   /* workspace pointer NULL or workspace_bytes too small */
    MOE_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
    MOE_ERR_SCRATCH_LIMIT = -5 /* moe_w8a8_forward_noalloc: the call needs more
                                  than MOE_W8A8_NOALLOC_SCRATCH_BYTES of workspace */
} moe_status_t;

/* Sizes and attributes of one call (FusedDeepMoE sec. 1.2 attributes and the
 * sec. 2.1 tiling struct, minus the communication-only group_ep / global_bs). */
typedef struct {
    int32_t num_tokens;     /* T >= 0 rows of x; T == 0 is legal (all counts 0)     */
    int32_t hidden;         /* H > 0, multiple of 256                                */
    int32_t inter;          /* I > 0, multiple of 256; GEMM1 has 2*I outputs:        */
                            /*   gate = rows [0, I), up = rows [I, 2I) of gmm1_weight */
    int32_t share_inter;    /* I_s: shared-expert intermediate, multiple of 256;     */
                            /*   0 = no shared expert                                */
    int32_t topk;           /* K in [1, 16]                                          */
    int32_t moe_expert_num; /* E_g >= 1 global routed experts                        */
    int32_t ep_rank_size;   /* >= 1, divides E_g; E_loc = E_g / ep_rank_size <= 512  */
    int32_t ep_rank_id;     /* in [0, ep_rank_size): local experts are global ids    */
                            /*   [ep_rank_id*E_loc, (ep_rank_id+1)*E_loc)            */
    int32_t quant_mode;     /* 1 = per-token dynamic INT8; 2 = per token and group:  */
                            /*   one amax / scale per row and group of quant_group   */
                            /*   consecutive elements along the contraction, each    */
                            /*   group's int32 partial dequantised by its own scale  */
                            /*   and the groups summed in fp32 ("DeepSeek V4 Decode  */
                            /*   Optimization" sec. 3.1); see quant_group            */
    float amax_eps;         /* > 0: row amax floor (e.g. 1e-6)                       */
    int32_t weight_layout;  /* MOE_WEIGHT_ROW_MAJOR: the layouts listed at           */
                            /*   moe_w8a8_forward; MOE_WEIGHT_PACKED: all four       */
                            /*   weight tensors come from moe_w8a8_pack_weights      */
    int32_t fuse_route_scale; /* 0: combine multiplies each routed bf16 row by its   */
                            /*   routing weight (FusedDeepMoE sec. 4.2); 1: the     */
                            /*   weight is folded into the row's GEMM2 dequant scale */
                            /*   (fl(hs * w), "DeepSeek V4 Decode Optimization" sec. */
                            /*   2.3) and combine only sums; z rows then carry it    */
    int32_t weight_format;  /* MOE_WEIGHT_INT8: the W8A8 block above.               */
                            /*   MOE_WEIGHT_MXFP4: the FP8/FP4 variant of the expert */
                            /*   GEMMs ("FIFO Pipeline Analysis ... Mega MoE": FP8   */
                            /*   GEMMs, FP8 cast after SwiGLU, FP4 weights): x and h */
                            /*   are quantised per row to FP8 E4M3 (scale = a'/448, */
                            /*   q = e4m3((v*448)/a'), round to nearest even,        */
                            /*   saturating), the weights are OCP E2M1 with one E8M0 */
                            /*   scale per 32 k elements and keep their fp32         */
                            /*   per-channel scales, the GEMMs accumulate in fp32.   */
                            /*   Requires weight_layout == MOE_WEIGHT_PACKED (else   */
                            /*   MOE_ERR_UNSUPPORTED) with every weight tensor       */
                            /*   written by moe_w8a8_pack_weights_mx; the debug      */
                            /*   acc1 / acc2 dumps then hold fp32 bit patterns       */
    int32_t quant_group;    /* quant_mode 2: elements per group, 64, 128 or 256      */
                            /*   (so it divides H, I and I_s); INT8 weights only,    */
                            /*   not with fuse_route_scale (MOE_ERR_UNSUPPORTED      */
                            /*   otherwise). The debug                               */
                            /*   xs / hs dumps then hold H/G and max(I, I_s)/G       */
                            /*   scales per row, acc1 / acc2 the fp32 bits of the    */
                            /*   dequantised group sums. Ignored for quant_mode 1    */
    int32_t requant_in_epilogue; /* 0: h is requantised by a launch of its own.     */
                            /*   1: inside GEMM1's epilogue where the batch runs the */
                            /*   decode GEMM (T <= 16, INT8 weights, quant_mode 1):  */
                            /*   the last of a chunk's GEMM1 workgroups to finish    */
                            /*   quantises the chunk's rows, found by an arrival     */
                            /*   count per chunk that the same call's routing resets */
                            /*   ("FIFO Pipeline Analysis ... Mega MoE": the first   */
                            /*   GEMM's epilogue ends in the cast after SwiGLU, with */
                            /*   arrival counts; "FusedDeepMoE Kernel 深度分析报告"  */
                            /*   sec. 7: SwiGLU and quantisation fused). Results are */
                            /*   identical either way; other batches ignore it       */
} moe_w8a8_dims_t;

enum { MOE_WEIGHT_ROW_MAJOR = 0, MOE_WEIGHT_PACKED = 1 };
enum { MOE_WEIGHT_INT8 = 0, MOE_WEIGHT_MXFP4 = 1 };

/* Optional intermediates for testing (every field may be NULL; all are device
 * buffers written in stream order). Rows are "grouped rows": rows [0, P) are
 * the kept routed pairs in (local expert, token, k) order, rows [P, P+T_act)
 * the shared expert's rows, one per active token in token order. With
 * R = T*K + T rows of capacity and Imax = max(I, I_s):                       */
typedef struct {
    int32_t *sorted_pair;   /* [T*K]   pair id t*K+k of routed row r           */
    int32_t *row_of_pair;   /* [T*K]   routed row of pair t*K+k, -1 if dropped */
    int32_t *group_offset;  /* [E_loc+1] exclusive prefix sum of the counts    */
    int32_t *shared_token;  /* [T]     token of shared row P+i                 */
    int32_t *num_rows;      /* [4]     P, T_act, #ids out of range, #chunks    */
    int8_t  *q_x;           /* [R, H]  GEMM1 input codes                       */
    float   *xs;            /* [R]     their per-row dequant scale             */
    int32_t *acc1;          /* [R, 2*Imax] GEMM1 int32 accumulators            */
    float   *h;             /* [R, Imax] SwiGLU output (fp32)                  */
    int8_t  *q_h;           /* [R, Imax] GEMM2 input codes                     */
    float   *hs;            /* [R]     their per-row dequant scale             */
    int32_t *acc2;          /* [R, H]  GEMM2 int32 accumulators                */
    uint16_t *z;            /* [R, H]  bf16 GEMM2 output rows                  */
    void   **stage_events;  /* [6] caller-created hipEvent_t (NULL entries are
                               skipped), recorded on the stream before routing
                               and after each stage: routing with the
                               quantisation of x, GEMM1, requant, GEMM2,
                               combine                                        */
    void   **kernel_events; /* [4] caller-created hipEvent_t (NULL entries are
                               skipped) bound to the GEMM kernels themselves
                               (hipExtLaunchKernel): start and end of the GEMM1
                               launch, start of the first and end of the last
                               GEMM2 launch. Unlike stage_events they add no
                               marker between kernels, so their elapsed times
                               are the kernels' own durations.               */
} moe_w8a8_debug_t;

/* Workspace bytes that moe_w8a8_forward needs for these dims. The size depends
 * only on T, H, I, I_s, K, E_loc and the options. The workspace holds every
 * intermediate the launches of one call hand to each other, as FusedDeepMoE
 * sec. 2.2 (workspace layout) does: the grouped rows' quantised GEMM1 input and
 * its scales, the SwiGLU output, the quantised GEMM2 input and its scales, the
 * GEMM2 output rows before combine, and the per-expert counts, prefix sum and
 * row order; here also the GEMM work-item list and per-call counters. Returns
 * MOE_ERR_INVALID_ARG for NULL arguments and the same size errors as
 * moe_w8a8_forward. */
MOE_W8A8_API moe_status_t moe_w8a8_workspace_size(const moe_w8a8_dims_t *dims, size_t *bytes);

/*
 * The fused expert block (FusedDeepMoE sec. 1.2 signature; EP communication
 * left out: non-local pairs are dropped, so `output` holds this rank's
 * partial sum, exactly as one expert-parallel rank computes before combine).
 *
 *  x                  bf16 [T, H]   (x, expert_ids, expert_scales and output
 *                     may be NULL when T == 0)
 *  expert_ids         int32 [T, K] global expert ids
 *  expert_scales      fp32 [T, K] routing weights
 *  gmm1_weight        int8 [E_loc, 2I, H]  (output channel major, H contiguous)
 *  gmm1_weight_scale  fp32 [E_loc, 2I]
 *  gmm2_weight        int8 [E_loc, H, I]   (I contiguous)
 *  gmm2_weight_scale  fp32 [E_loc, H]
 *  share_gmm1_weight  int8 [2I_s, H], share_gmm1_weight_scale fp32 [2I_s]  } all four NULL
 *  share_gmm2_weight  int8 [H, I_s],  share_gmm2_weight_scale fp32 [H]     } iff I_s == 0
 *  expert_smooth_scales fp32 [E_loc, H] or NULL: x is multiplied by the row of
 *                     the pair's expert before quantisation
 *  share_smooth_scales  fp32 [H] or NULL (requires I_s > 0)
 *  x_active_mask      uint8 [T] (0 / non-0) or NULL = every token active
 *  output             bf16 [T, H]  sum over kept pairs (k ascending, fp32) of
 *                     expert row x routing weight, one bf16 rounding; rows of
 *                     inactive tokens or tokens with no kept pair are 0
 *  share_output       bf16 [T, H]  shared-expert output (unweighted), 0 on
 *                     inactive tokens; required iff I_s > 0, else ignored
 *  expert_token_nums  int32 [E_loc] kept pairs per local expert
 *  workspace          device scratch of >= moe_w8a8_workspace_size() bytes;
 *                     need not be zeroed; contents are undefined afterwards
 *  dbg                NULL in production; else intermediates (above)
 *  stream             hipStream_t to launch on (NULL = the default stream)
 *
 * Values: x, the routing weights, the weight scales and the smooth scales are
 * taken to be finite (the block the pages describe defines nothing else). A
 * NaN or infinity in a token's inputs makes that token's rows and outputs
 * unspecified; every row of the block is computed independently of the other
 * tokens, so the rest of the result is unaffected. Expert ids outside
 * [0, moe_expert_num) drop their pair (the routing diagnostics word counts
 * them); duplicated ids in one token's top-k are kept as separate pairs.
 */
MOE_W8A8_API moe_status_t moe_w8a8_forward(const moe_w8a8_dims_t *dims,
                              const void *x,
                              const int32_t *expert_ids,
                              const float *expert_scales,
                              const int8_t *gmm1_weight,
                              const float *gmm1_weight_scale,
                              const int8_t *gmm2_weight,
                              const float *gmm2_weight_scale,
                              const int8_t *share_gmm1_weight,
                              const float *share_gmm1_weight_scale,
                              const int8_t *share_gmm2_weight,
                              const float *share_gmm2_weight_scale,
                              const float *expert_smooth_scales,
                              const float *share_smooth_scales,
                              const uint8_t *x_active_mask,
                              void *output,
                              void *share_output,
                              int32_t *expert_token_nums,
                              void *workspace,
                              size_t workspace_bytes,
                              const moe_w8a8_debug_t *dbg,
                              void *stream);

/*
 * moe_w8a8_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Every other argument, the result and the
 * errors are those of moe_w8a8_forward; the call allocates nothing (no
 * hipMalloc, no hipFree, no allocating library routine).
 *
 * The workspace is a device array built into the library,
 * MOE_W8A8_NOALLOC_SCRATCH_BYTES bytes on each GPU the library runs on, held
 * from module load until the process ends. Its device address is looked up
 * on the first call on each device (the device that is current at the call,
 * which must be the stream's device). Calls whose workspace (see
 * moe_w8a8_workspace_size) would exceed it return MOE_ERR_SCRATCH_LIMIT and
 * launch nothing: at hidden 4096, intermediate 2048, top-8 with a shared
 * expert, batches of up to about 128 tokens fit.
 *
 * All calls on one GPU share that GPU's array, so two calls that may overlap
 * on one GPU (different streams, or different host threads without ordering)
 * race: order them on one stream, or use moe_w8a8_forward with a workspace
 * each. The array keeps the last call's contents; nothing needs to start at
 * zero (every index and counter the block uses is rebuilt by each call).
 */
#define MOE_W8A8_NOALLOC_SCRATCH_BYTES (32u << 20)
MOE_W8A8_API moe_status_t moe_w8a8_forward_noalloc(const moe_w8a8_dims_t *dims,
                              const void *x,
                              const int32_t *expert_ids,
                              const float *expert_scales,
                              const int8_t *gmm1_weight,
                              const float *gmm1_weight_scale,
                              const int8_t *gmm2_weight,
                              const float *gmm2_weight_scale,
                              const int8_t *share_gmm1_weight,
                              const float *share_gmm1_weight_scale,
                              const int8_t *share_gmm2_weight,
                              const float *share_gmm2_weight_scale,
                              const float *expert_smooth_scales,
                              const float *share_smooth_scales,
                              const uint8_t *x_active_mask,
                              void *output,
                              void *share_output,
                              int32_t *expert_token_nums,
                              const moe_w8a8_debug_t *dbg,
                              void *stream);

/*
 * Re-lay int8 weights once, at load time, into the order the GEMM kernels
 * stream (the MI355X counterpart of the NZ weight format that FusedDeepMoE
 * sec. 5.3 / 8.1 feeds its cube unit). Nothing is computed; bytes move.
 *
 *  src    int8 [groups, n, k], k contiguous (a gmm*_weight tensor: n = 2I, k = H
 *         for GEMM1; n = H, k = I for GEMM2; groups = E_loc, or 1 for a shared
 *         expert)
 *  which  MOE_PACK_GMM1 for a gmm1 tensor, MOE_PACK_GMM2 for a gmm2 tensor
 *  dst    int8, same size; for group g, tile position p and 64-byte k step s,
 *         the 1024 bytes at ((g*(n/16) + p)*(k/64) + s)*1024 hold, at byte
 *         16*l + b (l in [0,64), b in [0,16)), src[g][16j + l%16][64s +
 *         16*(l/16) + b], where j = p for GEMM2 and, for GEMM1 (gate tiles
 *         j < n/32, up tiles after them), j = p/2 for even p and n/32 + p/2
 *         for odd p: gate tile j and up tile j follow each other
 *  n % 32 == 0, k % 64 == 0; src and dst 16-byte aligned and not overlapping.
 *  Stream-ordered; returns MOE_ERR_INVALID_ARG for bad sizes, pointers or
 *  `which`.
 */
enum { MOE_PACK_GMM1 = 1, MOE_PACK_GMM2 = 2 };
MOE_W8A8_API moe_status_t moe_w8a8_pack_weights(const int8_t *src, int8_t *dst, int64_t groups, int32_t n,
                                                int32_t k, int32_t which, void *stream);

/*
 * FP4 weights for weight_format == MOE_WEIGHT_MXFP4, re-laid once at load time
 * (OCP microscaling formats: E2M1 elements, E8M0 scale 2^(e-127) per block of
 * 32 consecutive k elements of a weight row).
 *
 *  data         uint8 [groups, n, k/2]: element k' of row r in the low nibble
 *               of byte k'/2 when k' is even, the high nibble when odd
 *  block_scale  uint8 [groups, n, k/32] E8M0 exponents (255 = NaN: not allowed)
 *  which        MOE_PACK_GMM1 / MOE_PACK_GMM2 as for moe_w8a8_pack_weights
 *  dst          moe_w8a8_packed_mx_bytes(groups, n, k) bytes, 16-byte aligned:
 *               first the element blocks, exactly as moe_w8a8_pack_weights lays
 *               out a [groups, n, k/2] int8 tensor (one 1024-byte block per
 *               16-row tile and 128-element k step), then the scales: for group
 *               g, tile position p and k step s, the 64 bytes at
 *               D + ((g*(n/16) + p)*(k/128) + s)*64, D = groups*n*k/2, hold at
 *               byte l (l in [0,64)) block_scale[g][16j + l%16][4s + l/16], with
 *               j the tile of position p as in moe_w8a8_pack_weights
 *  n % 32 == 0, k % 128 == 0; no buffer may overlap dst. Stream-ordered.
 */
MOE_W8A8_API moe_status_t moe_w8a8_packed_mx_bytes(int64_t groups, int32_t n, int32_t k, size_t *bytes);
MOE_W8A8_API moe_status_t moe_w8a8_pack_weights_mx(const uint8_t *data, const uint8_t *block_scale, uint8_t *dst,
                                                   int64_t groups, int32_t n, int32_t k, int32_t which,
                                                   void *stream);

/*
 * Cache warm ("DeepSeek V4 Decode Optimization" sec. 4.5, inter-layer
 * eviction): read the device range [ptr, ptr + bytes) once on `stream` and
 * discard it, so that its lines sit in the 256 MB memory-side cache (and an
 * XCD's L2) when a later kernel reads them. A hint with no destination: no
 * value anywhere changes, and dropping the call changes no result. Meant for
 * the next layer's weights that every call touches (the shared expert's),
 * issued on a second stream while the current layer runs its latency-bound
 * launches; a range larger than the cache evicts itself. ptr 16-byte aligned,
 * bytes a multiple of 16 (MOE_ERR_INVALID_ARG otherwise); bytes == 0 is a
 * no-op. Stream-ordered, no allocation.
 */
MOE_W8A8_API moe_status_t moe_w8a8_warm(const void *ptr, size_t bytes, void *stream);

/*
 * Read-bandwidth probe, for measurement only: read the device range
 * [ptr, ptr + bytes) once on `stream` over the whole chip, with the access
 * pattern of the GEMMs' weight stream (each wave loads 1 KB contiguous per
 * instruction, non-temporal, eight loads in flight), and discard the data.
 * Timing it over a range larger than the 256 MB memory-side cache gives the
 * HBM read rate this device reaches, the measured counterpart of the
 * published peak that a memory-bound kernel's roofline fraction is set
 * against. No value anywhere changes. ptr 16-byte aligned, bytes a multiple
 * of 16 (MOE_ERR_INVALID_ARG otherwise); bytes == 0 is a no-op.
 * Stream-ordered, no allocation.
 */
MOE_W8A8_API moe_status_t moe_w8a8_read_probe(const void *ptr, size_t bytes, void *stream);

/*
 * Read-and-write probe, for measurement only: the larger-batch GEMMs' weight
 * stream together with their output writes. [src, src + src_bytes) is read in
 * work items of 256 KB (one two-wave workgroup each, six resident per CU;
 * each wave reads two 64 KB tiles in 1 KB steps through a ring of eight
 * non-temporal loads per tile), and every item then writes its equal share
 * of [dst, dst + dst_bytes) with 16-byte stores, as a GEMM workgroup writes
 * its output rows after its contraction. Timing it with a GEMM's own read and
 * write byte counts gives the rate that mix reaches on the device: writes to
 * HBM while the read stream saturates it cost several times their bytes.
 * src is not changed; dst receives arbitrary values. src 16-byte aligned,
 * src_bytes a multiple of 262144 (0 is a no-op); dst_bytes a multiple of 16
 * and at most src_bytes; dst 16-byte aligned and not overlapping src when
 * dst_bytes > 0 (MOE_ERR_INVALID_ARG otherwise). Stream-ordered, no
 * allocation.
 */
MOE_W8A8_API moe_status_t moe_w8a8_read_write_probe(const void *src, size_t src_bytes, void *dst, size_t dst_bytes,
                                                    void *stream);

/* Static description of a status code. Never NULL. */
MOE_W8A8_API const char *moe_w8a8_status_string(moe_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_W8A8_H */
