/*
 * CPU oracle of the W8A8 MoE expert block -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded C model of what the block computes, used to
 * check the GPU library. Only the tests, the smoke entry and the benchmark's
 * CPU-baseline leg may load it; the library never calls it and shares no code
 * with it.
 *
 * Sources (pages, by title):
 *  - "FusedDeepMoE Kernel 深度分析报告" (FusedDeepMoE):
 *      sec. 1.2 operator signature; sec. 4.1 dispatch (table + prefix-sum
 *      grouping, quantisation in dispatch); sec. 4.2 combine weighted top-k
 *      sum (LocalWindowCopy); sec. 6.1 dequant + SwiGLU epilogue; sec. 6.2
 *      dequant + bf16 cast epilogue; sec. 7.2 BlockQuant dynamic quantisation;
 *      sec. 9.1-9.3 math correspondence and the five-op SmallOps chain.
 *  - "DeepSeek V4 Decode Optimization": sec. 0 W8A8 contract (amax floored by
 *      an eps, scaled to the int8 maximum; scales stay fp32) and the rule
 *      that the golden uses the kernel's operation order and dtypes.
 *
 * Every floating-point step is one IEEE fp32 operation, round-to-nearest-even,
 * in the order written (build with -O2 -ffp-contract=off, no fast-math).
 * Integer accumulation is exact (int64).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t T;        /* tokens                                   */
    int32_t H;        /* hidden                                   */
    int32_t I;        /* routed intermediate (GEMM1 outputs 2*I)  */
    int32_t I_s;      /* shared intermediate, 0 = none            */
    int32_t K;        /* top-k                                    */
    int32_t E_g;      /* global routed experts                    */
    int32_t ep_size;  /* E_loc = E_g / ep_size                    */
    int32_t ep_rank;  /* local experts [ep_rank*E_loc, +E_loc)    */
    float eps;        /* amax floor                               */
    int32_t fuse_route_scale; /* 1: routing weight folded into the GEMM2
                                 row scale, combine only sums (DeepSeek V4
                                 Decode Optimization sec. 2.3)            */
    int32_t quant_group;      /* 0: one activation scale per row; G > 0: one
                                 per row and group of G consecutive elements
                                 along the contraction (DeepSeek V4 Decode
                                 Optimization sec. 3.1, the narrowed amax);
                                 G divides H, I and I_s                   */
} moe_oracle_dims;

/* Optional intermediates, indexed by grouped row: routed rows [0, P) in
 * (local expert, token, k) order, then shared-expert rows [P, P + T_act) in
 * token order. Row strides: q_x/acc2/z: H; acc1: 2*max(I, I_s);
 * h/q_h: max(I, I_s). Any pointer may be NULL. Only rows of the tokens that
 * forward() computes are written. With quant_group G > 0, xs holds H/G and hs
 * max(I, I_s)/G scales per row, and acc1 / acc2 the bits of the fp32
 * dequantised GEMM outputs (the group sums, before SwiGLU / the bf16 cast). */
typedef struct {
    int32_t *sorted_pair;   /* [T*K] pair id t*K+k per routed row          */
    int32_t *row_of_pair;   /* [T*K] routed row of a pair, -1 if dropped    */
    int32_t *offsets;       /* [E_loc+1] exclusive prefix of the counts     */
    int32_t *shared_token;  /* [T] token of shared row P+i                 */
    int32_t *num_rows;      /* [3] P, T_act, ids out of range              */
    int8_t  *q_x;           /* quantised GEMM1 input                        */
    float   *xs;            /* its per-row scale                            */
    int32_t *acc1;          /* GEMM1 int32 accumulators                     */
    float   *h;             /* SwiGLU output                                */
    int8_t  *q_h;           /* requantised GEMM2 input                      */
    float   *hs;            /* its per-row scale                            */
    int32_t *acc2;          /* GEMM2 int32 accumulators                     */
    uint16_t *z;            /* bf16 GEMM2 output rows                       */
} moe_oracle_trace;

/* bf16 <-> fp32 (bit patterns in uint16). */
float    moe_oracle_bf16_to_f32(uint16_t b);
uint16_t moe_oracle_f32_to_bf16(float f);

/* Dispatch grouping. Returns P (kept pairs). */
int32_t moe_oracle_route(const moe_oracle_dims *d, const int32_t *expert_ids,
                         const uint8_t *mask, int32_t *counts, int32_t *offsets,
                         int32_t *sorted_pair, int32_t *row_of_pair, int32_t *n_bad);

/* Per-row dynamic int8 quantisation of v[0..n). */
void moe_oracle_quant_row(const float *v, int32_t n, float eps, int8_t *q, float *scale);

/* C[m][n] = sum_k A[m][k] * B[n][k], exact. Returns 0, or -1 if a sum leaves int32. */
int32_t moe_oracle_gemm_i8(const int8_t *A, const int8_t *B, int32_t M, int32_t N,
                           int32_t Kd, int32_t *C);

/* Group-wise form (quant_group G): the row quantiser applied to each group of
 * G consecutive elements, one scale per group. */
void moe_oracle_quant_row_groups(const float *v, int32_t n, int32_t G, float eps, int8_t *q, float *scales);

/* One row through a GEMM with group-wise activation scales: for each output
 * n, each group's exact int32 partial acc_g = sum_{k in g} a[k] * B[n][k] is
 * dequantised by its own scale, p_g = fl(fl(float(acc_g) * wscale[n]) *
 * a_scales[g]), and y[n] is the fp32 sum of the p_g from zero, g ascending.
 * Returns 0, or -1 if a partial leaves int32. */
int32_t moe_oracle_gemm_i8_groups(const int8_t *a, const float *a_scales, const int8_t *B, const float *wscale,
                                  int32_t N, int32_t Kd, int32_t G, float *y);

/* SwiGLU of one dequantised GEMM1 row: h[j] = silu(y[j]) * y[n_half + j]. */
void moe_oracle_swiglu(const float *y, int32_t n_half, float *h);

/* --- FP4 weights / FP8 activations (the FP8/FP4 variant of the expert GEMMs,
 *     "FIFO Pipeline Analysis ... Mega MoE": FP8 GEMMs, FP8 cast after
 *     SwiGLU, FP4 weights). Formats are the OCP microscaling ones:
 *   E4M3 (activations): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 *     infinities, largest finite 448, code 0x7F / 0xFF NaN;
 *   E2M1 (weights): 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, values
 *     0, 0.5, 1, 1.5, 2, 3, 4, 6; two per byte, element 2j in the low nibble;
 *   E8M0 (weight block scales): 2^(e - 127), one per 32 consecutive K elements
 *     of a weight row (e = 255 is NaN and not used). */
uint8_t moe_oracle_f32_to_e4m3(float f);   /* round to nearest even, saturating at 448 */
float   moe_oracle_e4m3_to_f32(uint8_t c);
float   moe_oracle_e2m1_to_f32(uint8_t nibble);

/* Per-row dynamic FP8 quantisation of v[0..n): a' = max(max|v|, eps);
 * scale = a' * (1/448); q_i = e4m3((v_i * 448) * (1/a')). */
void moe_oracle_quant_row_fp8(const float *v, int32_t n, float eps, uint8_t *q, float *scale);

/* C[m][n] = sum_k e4m3(A[m][k]) * e2m1(B[n], k) * 2^(S[n][k/32] - 127): block
 * sums exact in int64, blocks combined in double, then one rounding to fp32.
 * A [M][Kd] codes, B [N][Kd/2] nibble pairs, S [N][Kd/32]; Kd % 32 == 0. */
void moe_oracle_gemm_mx(const uint8_t *A, const uint8_t *B, const uint8_t *S, int32_t M, int32_t N,
                        int32_t Kd, float *C);

/* Whole block. token_subset (n_subset entries, NULL = every token) selects
 * which output rows are computed; others are left untouched. Returns 0 or a
 * negative value on bad arguments. All pointers are host pointers. */
int32_t moe_oracle_forward(const moe_oracle_dims *d, const uint16_t *x,
                           const int32_t *expert_ids, const float *expert_scales,
                           const int8_t *w1, const float *w1s,
                           const int8_t *w2, const float *w2s,
                           const int8_t *sw1, const float *sw1s,
                           const int8_t *sw2, const float *sw2s,
                           const float *smooth, const float *share_smooth,
                           const uint8_t *mask,
                           const int32_t *token_subset, int32_t n_subset,
                           uint16_t *output, uint16_t *share_output,
                           int32_t *expert_token_nums, moe_oracle_trace *tr);

/* The same block with FP4 weights (E2M1 nibble pairs [.., N, K/2] plus E8M0
 * block scales [.., N, K/32]; the fp32 per-channel scales stay) and FP8 (E4M3)
 * activations: x and h are quantised to E4M3 per row, the GEMMs accumulate in
 * fp32 (exact here, then rounded once), everything else as in
 * moe_oracle_forward. Trace: q_x / q_h hold E4M3 codes, acc1 / acc2 the bits
 * of the fp32 accumulators. */
int32_t moe_oracle_forward_mx(const moe_oracle_dims *d, const uint16_t *x,
                              const int32_t *expert_ids, const float *expert_scales,
                              const uint8_t *w1, const uint8_t *w1b, const float *w1s,
                              const uint8_t *w2, const uint8_t *w2b, const float *w2s,
                              const uint8_t *sw1, const uint8_t *sw1b, const float *sw1s,
                              const uint8_t *sw2, const uint8_t *sw2b, const float *sw2s,
                              const float *smooth, const float *share_smooth,
                              const uint8_t *mask,
                              const int32_t *token_subset, int32_t n_subset,
                              uint16_t *output, uint16_t *share_output,
                              int32_t *expert_token_nums, moe_oracle_trace *tr);

#ifdef __cplusplus
}
#endif
#endif
