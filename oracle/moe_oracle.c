/*
 * CPU oracle of the W8A8 MoE expert block -- TEST INFRASTRUCTURE ONLY.
 * Loaded by the tests, the smoke entry and the benchmark's CPU-baseline leg;
 * never by the GPU library. Build: gcc -O2 -ffp-contract=off -fPIC -shared.
 *
 * It follows the unfused five-op decomposition of the pages (dispatch with
 * quantisation -> grouped GEMM1 -> dequant/SwiGLU/quant -> grouped GEMM2 ->
 * combine; "FusedDeepMoE Kernel 深度分析报告" sec. 9.3) one stage at a time,
 * with the per-stage arithmetic of sec. 6.1, 6.2, 7.2 and 4.2 of that page and
 * the W8A8 contract of "DeepSeek V4 Decode Optimization" sec. 0; the
 * group-wise activation scales follow sec. 3.1 of the latter.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

float moe_oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even (the CAST_RINT of the
 * FusedDeepMoE epilogues, sec. 6.2 and sec. 4.2). */
uint16_t moe_oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/*
 * Dispatch grouping (FusedDeepMoE sec. 4.1: per-expert token counts, their
 * prefix sum "groupList" and the expand index; the small-batch path builds a
 * token x expert table and takes a prefix sum over tokens, so rows of one
 * expert appear in token order). Pairs of masked-off tokens are skipped
 * (sec. 5.2.1 counts only active tokens). A pair whose global expert id lies
 * outside this rank's range is not local and is dropped; an id outside
 * [0, E_g) is dropped and counted in n_bad.
 */
int32_t moe_oracle_route(const moe_oracle_dims *d, const int32_t *expert_ids,
                         const uint8_t *mask, int32_t *counts, int32_t *offsets,
                         int32_t *sorted_pair, int32_t *row_of_pair, int32_t *n_bad) {
    const int32_t T = d->T, K = d->K, E = d->E_g / d->ep_size;
    const int32_t base = d->ep_rank * E;
    int32_t bad = 0;
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int32_t p = 0; p < T * K; ++p) row_of_pair[p] = -1;
    /* histogram */
    for (int32_t t = 0; t < T; ++t) {
        if (mask && !mask[t]) continue;
        for (int32_t k = 0; k < K; ++k) {
            int32_t g = expert_ids[t * K + k];
            if (g < 0 || g >= d->E_g) { ++bad; continue; }
            int32_t e = g - base;
            if (e < 0 || e >= E) continue;
            counts[e] += 1;
        }
    }
    /* exclusive prefix sum */
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    /* stable placement in (expert, token, k) order */
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int32_t t = 0; t < T; ++t) {
        if (mask && !mask[t]) continue;
        for (int32_t k = 0; k < K; ++k) {
            int32_t g = expert_ids[t * K + k];
            if (g < 0 || g >= d->E_g) continue;
            int32_t e = g - base;
            if (e < 0 || e >= E) continue;
            int32_t row = cursor[e]++;
            sorted_pair[row] = t * K + k;
            row_of_pair[t * K + k] = row;
        }
    }
    free(cursor);
    if (n_bad) *n_bad = bad;
    return offsets[E];
}

/*
 * Per-row dynamic int8 quantisation (FusedDeepMoE sec. 7.2 BlockQuant; the
 * eps floor of "DeepSeek V4 Decode Optimization" sec. 0):
 *   a   = max_i |v_i|, floored: a' = max(a, eps)
 *   scale (dequant, kept fp32) = a' * (1/127)
 *   q_i = rint_half_even((v_i * 127) * (1/a')), in [-127, 127]
 */
void moe_oracle_quant_row(const float *v, int32_t n, float eps, int8_t *q, float *scale) {
    float a = 0.0f;
    for (int32_t i = 0; i < n; ++i) {
        float m = fabsf(v[i]);
        if (m > a) a = m;
    }
    if (a < eps) a = eps;
    const float inv = 1.0f / a;
    const float inv127 = 1.0f / 127.0f;
    *scale = a * inv127;
    for (int32_t i = 0; i < n; ++i) {
        float t = v[i] * 127.0f;
        t = t * inv;
        float r = rintf(t);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i] = (int8_t)r;
    }
}

/* The narrowed amax of "DeepSeek V4 Decode Optimization" sec. 3.1: one amax,
 * and so one scale, per row and group instead of per row; each group is
 * quantised by the per-row rule above. */
void moe_oracle_quant_row_groups(const float *v, int32_t n, int32_t G, float eps, int8_t *q, float *scales) {
    for (int32_t g = 0; g < n / G; ++g) moe_oracle_quant_row(v + (size_t)g * G, G, eps, q + (size_t)g * G, &scales[g]);
}

/* Sec. 3.1 of the same page: each group's INT32 partial is dequantised by its
 * own group scale (the per-row dequant order, FusedDeepMoE sec. 6.1 / 6.2,
 * applied to the partial); the dequantised partials are added in fp32 from
 * zero, group by group. */
int32_t moe_oracle_gemm_i8_groups(const int8_t *a, const float *a_scales, const int8_t *B, const float *wscale,
                                  int32_t N, int32_t Kd, int32_t G, float *y) {
    int32_t rc = 0;
    for (int32_t n = 0; n < N; ++n) {
        const int8_t *b = B + (size_t)n * Kd;
        float sum = 0.0f;
        for (int32_t g = 0; g < Kd / G; ++g) {
            int64_t s = 0;
            for (int32_t k = g * G; k < (g + 1) * G; ++k) s += (int64_t)a[k] * (int64_t)b[k];
            if (s > INT32_MAX || s < INT32_MIN) rc = -1;
            float p = (float)(int32_t)s;
            p = p * wscale[n];
            p = p * a_scales[g];
            sum = sum + p;
        }
        y[n] = sum;
    }
    return rc;
}

/* Grouped-GEMM contraction of one group (FusedDeepMoE sec. 3.3: int8 A,
 * int8 B, int32 C). Weights are stored [N][K] (output channel major, the
 * contraction dimension contiguous). Exact in int64, checked against int32. */
int32_t moe_oracle_gemm_i8(const int8_t *A, const int8_t *B, int32_t M, int32_t N,
                           int32_t Kd, int32_t *C) {
    int32_t rc = 0;
    for (int32_t m = 0; m < M; ++m) {
        const int8_t *a = A + (size_t)m * Kd;
        for (int32_t n = 0; n < N; ++n) {
            const int8_t *b = B + (size_t)n * Kd;
            int64_t s = 0;
            for (int32_t k = 0; k < Kd; ++k) s += (int64_t)a[k] * (int64_t)b[k];
            if (s > INT32_MAX || s < INT32_MIN) rc = -1;
            C[(size_t)m * N + n] = (int32_t)s;
        }
    }
    return rc;
}

/* SwiGLU (FusedDeepMoE sec. 6.1 left half x / (1 + exp(-x)); sec. 7.2 then
 * multiplies by the right half): gate = y[0..n_half), up = y[n_half..2n_half). */
void moe_oracle_swiglu(const float *y, int32_t n_half, float *h) {
    for (int32_t j = 0; j < n_half; ++j) {
        float g = y[j];
        float ng = -g;
        float e = expf(ng);
        float den = 1.0f + e;
        float s = g / den;
        h[j] = s * y[n_half + j];
    }
}

/* FP8 E4M3 from fp32: round to nearest, ties to even, on the E4M3 grid
 * (subnormal step 2^-9, normal values (8 + m) * 2^(e - 10)); magnitudes that
 * round above 448 saturate to 448. */
uint8_t moe_oracle_f32_to_e4m3(float f) {
    if (isnan(f)) return 0x7F;
    const uint8_t sign = signbit(f) ? 0x80 : 0x00;
    const float a = fabsf(f);
    if (a >= 448.0f) return sign | 0x7E;
    if (a < 0.015625f) {                     /* below 2^-6: subnormal codes m * 2^-9 */
        const float m = rintf(a * 512.0f);   /* exact scaling; m == 8 is the smallest normal */
        return sign | (uint8_t)m;
    }
    int e2;
    (void)frexpf(a, &e2);                     /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;                           /* unbiased exponent, -6..8 */
    float m = rintf(ldexpf(a, 3 - E));        /* significand in eighths, 8..16 */
    if (m == 16.0f) { m = 8.0f; E += 1; }
    if (E > 8 || (E == 8 && m > 14.0f)) return sign | 0x7E;
    return sign | (uint8_t)(((E + 7) << 3) | ((int)m - 8));
}

float moe_oracle_e4m3_to_f32(uint8_t c) {
    const int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const float v = e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
    return (c & 0x80) ? -v : v;
}

float moe_oracle_e2m1_to_f32(uint8_t nib) {
    const int e = (nib >> 1) & 3, m = nib & 1;
    const float v = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return (nib & 8) ? -v : v;
}

/* Per-row dynamic FP8 quantisation: the int8 rule with 448 (the largest E4M3
 * value) in place of 127 and E4M3 rounding in place of rint. */
void moe_oracle_quant_row_fp8(const float *v, int32_t n, float eps, uint8_t *q, float *scale) {
    float a = 0.0f;
    for (int32_t i = 0; i < n; ++i) {
        float m = fabsf(v[i]);
        if (m > a) a = m;
    }
    if (a < eps) a = eps;
    const float inv = 1.0f / a;
    const float inv448 = 1.0f / 448.0f;
    *scale = a * inv448;
    for (int32_t i = 0; i < n; ++i) {
        float t = v[i] * 448.0f;
        t = t * inv;
        q[i] = moe_oracle_f32_to_e4m3(t);
    }
}

/* Integer forms: an E4M3 value is qa * 2^-9 and an E2M1 value qb * 2^-1 with
 * integers qa, qb, so a 32-element block sum is an exact int64 times
 * 2^(E - 127 - 10). */
static int32_t e4m3_units(uint8_t c) { return (int32_t)ldexpf(moe_oracle_e4m3_to_f32(c), 9); }
static int32_t e2m1_units(uint8_t nib) { return (int32_t)(2.0f * moe_oracle_e2m1_to_f32(nib)); }

void moe_oracle_gemm_mx(const uint8_t *A, const uint8_t *B, const uint8_t *S, int32_t M, int32_t N,
                        int32_t Kd, float *C) {
    const int32_t nb = Kd / 32;
    for (int32_t m = 0; m < M; ++m) {
        const uint8_t *a = A + (size_t)m * Kd;
        for (int32_t n = 0; n < N; ++n) {
            const uint8_t *b = B + (size_t)n * (Kd / 2);
            const uint8_t *sc = S + (size_t)n * nb;
            double acc = 0.0;
            for (int32_t blk = 0; blk < nb; ++blk) {
                int64_t s = 0;
                for (int32_t k = blk * 32; k < blk * 32 + 32; ++k) {
                    const uint8_t byte = b[k / 2];
                    const uint8_t nib = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
                    s += (int64_t)e4m3_units(a[k]) * (int64_t)e2m1_units(nib);
                }
                acc += ldexp((double)s, (int)sc[blk] - 127 - 10);
            }
            C[(size_t)m * N + n] = (float)acc;
        }
    }
}

/* Dequantise one int32 accumulator row: fl(fl(float(acc) * w_scale[n]) * row_scale)
 * (FusedDeepMoE sec. 6.1 steps 2-4 and sec. 6.2 steps 1-4; int32 -> fp32 with
 * round-to-nearest-even). */
static void dequant_row(const int32_t *acc, const float *wscale, float row_scale,
                        int32_t n, float *y) {
    for (int32_t i = 0; i < n; ++i) {
        float f = (float)acc[i];
        f = f * wscale[i];
        y[i] = f * row_scale;
    }
}

/* The same with an fp32 accumulator (FP4/FP8 GEMMs). */
static void dequant_row_f(const float *acc, const float *wscale, float row_scale, int32_t n, float *y) {
    for (int32_t i = 0; i < n; ++i) {
        float f = acc[i] * wscale[i];
        y[i] = f * row_scale;
    }
}

/* One expert's weights: int8 [N][K] (w1b == NULL), or FP4 nibble pairs
 * [N][K/2] with E8M0 block scales w1b / w2b [N][K/32]. */
typedef struct {
    const void *w1; const float *w1s; const void *w2; const float *w2s;
    const float *smooth; int32_t inter;
    const uint8_t *w1b, *w2b;
} expert_view;

/* One grouped row through quant -> GEMM1 -> dequant/SwiGLU -> requant ->
 * GEMM2 -> dequant -> bf16 (FusedDeepMoE sec. 7.1 data flow). With `fold`
 * the GEMM2 row scale is fl(hs * route_w), the routing weight folded in
 * ("DeepSeek V4 Decode Optimization" sec. 2.3: one fused row scale);
 * otherwise it is hs. */
static int32_t run_row(const moe_oracle_dims *d, const uint16_t *xrow, const expert_view *ev,
                       int fold, float route_w,
                       int32_t row, int32_t Imax, moe_oracle_trace *tr, uint16_t *zrow,
                       float *vbuf, int8_t *qx, int32_t *acc1, float *y, float *h,
                       int8_t *qh, int32_t *acc2, float *gsc) {
    const int32_t H = d->H, I = ev->inter;
    int32_t rc = 0;
    float xs, hs;
    const int32_t G = d->quant_group;
    if (G > 0) {
        /* group-wise activation scales (int8 weights only): x and h are
         * quantised per group, each GEMM partial is dequantised by its own
         * group scale; the fp32 GEMM outputs live in the int32 buffers */
        float *xsg = gsc, *hsg = gsc + H / G;
        float *y2 = (float *)(void *)acc2;
        for (int32_t i = 0; i < H; ++i) {
            float v = moe_oracle_bf16_to_f32(xrow[i]);
            if (ev->smooth) v = v * ev->smooth[i];
            vbuf[i] = v;
        }
        moe_oracle_quant_row_groups(vbuf, H, G, d->eps, qx, xsg);
        rc |= moe_oracle_gemm_i8_groups(qx, xsg, (const int8_t *)ev->w1, ev->w1s, 2 * I, H, G, y);
        moe_oracle_swiglu(y, I, h);
        moe_oracle_quant_row_groups(h, I, G, d->eps, qh, hsg);
        rc |= moe_oracle_gemm_i8_groups(qh, hsg, (const int8_t *)ev->w2, ev->w2s, H, I, G, y2);
        for (int32_t n = 0; n < H; ++n) zrow[n] = moe_oracle_f32_to_bf16(y2[n]);
        if (tr) {
            if (tr->q_x) memcpy(tr->q_x + (size_t)row * H, qx, (size_t)H);
            if (tr->xs) memcpy(tr->xs + (size_t)row * (H / G), xsg, sizeof(float) * (size_t)(H / G));
            if (tr->acc1) memcpy(tr->acc1 + (size_t)row * 2 * Imax, y, sizeof(float) * 2 * (size_t)I);
            if (tr->h) memcpy(tr->h + (size_t)row * Imax, h, sizeof(float) * (size_t)I);
            if (tr->q_h) memcpy(tr->q_h + (size_t)row * Imax, qh, (size_t)I);
            if (tr->hs) memcpy(tr->hs + (size_t)row * (Imax / G), hsg, sizeof(float) * (size_t)(I / G));
            if (tr->acc2) memcpy(tr->acc2 + (size_t)row * H, y2, sizeof(float) * (size_t)H);
            if (tr->z) memcpy(tr->z + (size_t)row * H, zrow, sizeof(uint16_t) * (size_t)H);
        }
        return rc;
    }
    for (int32_t i = 0; i < H; ++i) {
        float v = moe_oracle_bf16_to_f32(xrow[i]);
        if (ev->smooth) v = v * ev->smooth[i];
        vbuf[i] = v;
    }
    const int mx = ev->w1b != NULL;
    /* (fp32 accumulators of the FP4 path live in the int32 buffers, bit for bit) */
    float *acc1f = (float *)(void *)acc1, *acc2f = (float *)(void *)acc2;
    if (mx) {
        moe_oracle_quant_row_fp8(vbuf, H, d->eps, (uint8_t *)qx, &xs);
        moe_oracle_gemm_mx((const uint8_t *)qx, (const uint8_t *)ev->w1, ev->w1b, 1, 2 * I, H, acc1f);
        dequant_row_f(acc1f, ev->w1s, xs, 2 * I, y);
    } else {
        moe_oracle_quant_row(vbuf, H, d->eps, qx, &xs);
        rc |= moe_oracle_gemm_i8(qx, (const int8_t *)ev->w1, 1, 2 * I, H, acc1);
        dequant_row(acc1, ev->w1s, xs, 2 * I, y);
    }
    moe_oracle_swiglu(y, I, h);
    if (mx) {
        moe_oracle_quant_row_fp8(h, I, d->eps, (uint8_t *)qh, &hs);
        moe_oracle_gemm_mx((const uint8_t *)qh, (const uint8_t *)ev->w2, ev->w2b, 1, H, I, acc2f);
    } else {
        moe_oracle_quant_row(h, I, d->eps, qh, &hs);
        rc |= moe_oracle_gemm_i8(qh, (const int8_t *)ev->w2, 1, H, I, acc2);
    }
    const float rs2 = fold ? hs * route_w : hs;
    if (mx)
        dequant_row_f(acc2f, ev->w2s, rs2, H, vbuf);
    else
        dequant_row(acc2, ev->w2s, rs2, H, vbuf);
    for (int32_t n = 0; n < H; ++n) zrow[n] = moe_oracle_f32_to_bf16(vbuf[n]);
    if (tr) {
        if (tr->q_x) memcpy(tr->q_x + (size_t)row * H, qx, (size_t)H);
        if (tr->xs) tr->xs[row] = xs;
        if (tr->acc1) memcpy(tr->acc1 + (size_t)row * 2 * Imax, acc1, sizeof(int32_t) * 2 * (size_t)I);
        if (tr->h) memcpy(tr->h + (size_t)row * Imax, h, sizeof(float) * (size_t)I);
        if (tr->q_h) memcpy(tr->q_h + (size_t)row * Imax, qh, (size_t)I);
        if (tr->hs) tr->hs[row] = hs;
        if (tr->acc2) memcpy(tr->acc2 + (size_t)row * H, acc2, sizeof(int32_t) * (size_t)H);
        if (tr->z) memcpy(tr->z + (size_t)row * H, zrow, sizeof(uint16_t) * (size_t)H);
    }
    return rc;
}

/* Weights are int8 when w1b is NULL, FP4 with E8M0 block scales otherwise. */
static int32_t forward_impl(const moe_oracle_dims *d, const uint16_t *x,
                            const int32_t *expert_ids, const float *expert_scales,
                            const void *w1, const uint8_t *w1b, const float *w1s,
                            const void *w2, const uint8_t *w2b, const float *w2s,
                            const void *sw1, const uint8_t *sw1b, const float *sw1s,
                            const void *sw2, const uint8_t *sw2b, const float *sw2s,
                            const float *smooth, const float *share_smooth,
                            const uint8_t *mask,
                            const int32_t *token_subset, int32_t n_subset,
                            uint16_t *output, uint16_t *share_output,
                            int32_t *expert_token_nums, moe_oracle_trace *tr) {
    if (!d || d->T < 0 || d->H <= 0 || d->I <= 0 || d->K <= 0 || d->E_g <= 0 ||
        d->ep_size <= 0 || d->E_g % d->ep_size || d->ep_rank < 0 || d->ep_rank >= d->ep_size)
        return -1;
    const int32_t T = d->T, H = d->H, I = d->I, K = d->K, Is = d->I_s;
    const int32_t E = d->E_g / d->ep_size;
    const int32_t Imax = Is > I ? Is : I;
    const int has_shared = Is > 0;
    const int32_t G = d->quant_group;
    if (G < 0 || (G > 0 && (H % G || I % G || Is % G || w1b || d->fuse_route_scale))) return -1;
    if (has_shared && (!sw1 || !sw1s || !sw2 || !sw2s || !share_output)) return -2;

    /* 1. dispatch grouping */
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *sorted_pair = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * K + 1));
    int32_t *row_of_pair = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * K + 1));
    int32_t *shared_row = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T + 1));
    int32_t n_bad = 0;
    const int32_t P = moe_oracle_route(d, expert_ids, mask, counts, offsets, sorted_pair,
                                       row_of_pair, &n_bad);
    int32_t T_act = 0;
    for (int32_t t = 0; t < T; ++t) {
        shared_row[t] = -1;
        if (mask && !mask[t]) continue;
        if (tr && tr->shared_token) tr->shared_token[T_act] = t;
        shared_row[t] = P + T_act++;
    }
    if (expert_token_nums) memcpy(expert_token_nums, counts, sizeof(int32_t) * (size_t)E);
    if (tr) {
        if (tr->sorted_pair) memcpy(tr->sorted_pair, sorted_pair, sizeof(int32_t) * (size_t)P);
        if (tr->row_of_pair) memcpy(tr->row_of_pair, row_of_pair, sizeof(int32_t) * (size_t)(T * K));
        if (tr->offsets) memcpy(tr->offsets, offsets, sizeof(int32_t) * (size_t)(E + 1));
        if (tr->num_rows) { tr->num_rows[0] = P; tr->num_rows[1] = T_act; tr->num_rows[2] = n_bad; }
    }

    float *vbuf = (float *)malloc(sizeof(float) * (size_t)H);
    int8_t *qx = (int8_t *)malloc((size_t)H);
    int32_t *acc1 = (int32_t *)malloc(sizeof(int32_t) * 2 * (size_t)Imax);
    float *y = (float *)malloc(sizeof(float) * 2 * (size_t)Imax);
    float *h = (float *)malloc(sizeof(float) * (size_t)Imax);
    int8_t *qh = (int8_t *)malloc((size_t)Imax);
    int32_t *acc2 = (int32_t *)malloc(sizeof(int32_t) * (size_t)H);
    uint16_t *zk = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)H * (size_t)K);
    float *sum = (float *)malloc(sizeof(float) * (size_t)H);
    float *gsc = (float *)malloc(sizeof(float) * (size_t)(H + Imax));
    int32_t rc = 0;

    const int32_t nt = token_subset ? n_subset : T;
    for (int32_t it = 0; it < nt; ++it) {
        const int32_t t = token_subset ? token_subset[it] : it;
        if (t < 0 || t >= T) { rc = -3; continue; }
        const uint16_t *xrow = x + (size_t)t * H;
        /* 2-6. routed rows of this token, k ascending */
        for (int32_t k = 0; k < K; ++k) {
            const int32_t row = row_of_pair[t * K + k];
            if (row < 0) continue;
            const int32_t e = expert_ids[t * K + k] - d->ep_rank * E;
            const int mx = w1b != NULL;
            const size_t wb1 = (size_t)e * 2 * I * H / (mx ? 2 : 1), wb2 = (size_t)e * H * I / (mx ? 2 : 1);
            expert_view ev = {(const uint8_t *)w1 + wb1, w1s + (size_t)e * 2 * I,
                              (const uint8_t *)w2 + wb2, w2s + (size_t)e * H,
                              smooth ? smooth + (size_t)e * H : NULL, I,
                              mx ? w1b + (size_t)e * 2 * I * (H / 32) : NULL,
                              mx ? w2b + (size_t)e * H * (I / 32) : NULL};
            rc |= run_row(d, xrow, &ev, d->fuse_route_scale != 0, expert_scales[t * K + k], row, Imax,
                          tr, zk + (size_t)k * H, vbuf, qx, acc1, y, h, qh, acc2, gsc);
        }
        /* 7. combine: fp32 sum from zero over kept pairs, k ascending, then
         * one bf16 cast (FusedDeepMoE sec. 4.2 LocalWindowCopy). Tokens with
         * no kept pair (masked off, or all pairs non-local) give zero rows.
         * Each row is weighted here, unless its weight was folded into its
         * GEMM2 row scale. */
        for (int32_t n = 0; n < H; ++n) sum[n] = 0.0f;
        for (int32_t k = 0; k < K; ++k) {
            if (row_of_pair[t * K + k] < 0) continue;
            const float s = expert_scales[t * K + k];
            const uint16_t *zr = zk + (size_t)k * H;
            for (int32_t n = 0; n < H; ++n) {
                float m = moe_oracle_bf16_to_f32(zr[n]);
                if (!d->fuse_route_scale) m = m * s;
                sum[n] = sum[n] + m;
            }
        }
        if (output)
            for (int32_t n = 0; n < H; ++n) output[(size_t)t * H + n] = moe_oracle_f32_to_bf16(sum[n]);
        /* 8. shared expert on every active token, unweighted, separate output
         * (FusedDeepMoE sec. 1.2 share_output; sec. 5.2.1 shared quant first). */
        if (has_shared) {
            uint16_t *so = share_output + (size_t)t * H;
            if (shared_row[t] < 0) {
                for (int32_t n = 0; n < H; ++n) so[n] = 0;
            } else {
                expert_view ev = {sw1, sw1s, sw2, sw2s, share_smooth, Is, sw1b, sw2b};
                rc |= run_row(d, xrow, &ev, 0, 1.0f, shared_row[t], Imax, tr, so, vbuf, qx, acc1, y, h,
                              qh, acc2, gsc);
            }
        }
    }
    free(counts); free(offsets); free(sorted_pair); free(row_of_pair); free(shared_row);
    free(vbuf); free(qx); free(acc1); free(y); free(h); free(qh); free(acc2); free(zk); free(sum); free(gsc);
    return rc;
}

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
                           int32_t *expert_token_nums, moe_oracle_trace *tr) {
    return forward_impl(d, x, expert_ids, expert_scales, w1, NULL, w1s, w2, NULL, w2s, sw1, NULL, sw1s, sw2, NULL,
                        sw2s, smooth, share_smooth, mask, token_subset, n_subset, output, share_output,
                        expert_token_nums, tr);
}

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
                              int32_t *expert_token_nums, moe_oracle_trace *tr) {
    if (!w1b || !w2b || (d && d->I_s > 0 && (!sw1b || !sw2b))) return -2;
    if (d && (d->H % 32 || d->I % 32 || d->I_s % 32)) return -1;
    return forward_impl(d, x, expert_ids, expert_scales, w1, w1b, w1s, w2, w2b, w2s, sw1, sw1b, sw1s, sw2, sw2b,
                        sw2s, smooth, share_smooth, mask, token_subset, n_subset, output, share_output,
                        expert_token_nums, tr);
}
