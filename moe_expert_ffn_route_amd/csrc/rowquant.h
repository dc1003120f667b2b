// Per-row dynamic INT8 (or FP8 E4M3) quantisation, as block-cooperative
// device functions.
//
// The rule ("FusedDeepMoE Kernel 深度分析报告" sec. 7.2 BlockQuant, with the
// eps floor of "DeepSeek V4 Decode Optimization" sec. 0):
//   a' = max(max_i |v_i|, eps);  scale = a' * (1/127);
//   q_i = rint((v_i * 127) * (1/a'))  (round to nearest even)
// The FP8 form (FP4-weight variant) takes 448, the largest E4M3 value, for 127
// and rounds to the E4M3 grid instead of to integers.
// Every product is a separate IEEE fp32 operation (the library is built with
// -ffp-contract=off) and 1/a' is a correctly rounded division, so the codes
// are the exact function of the fp32 inputs that the rule defines.
//
// A row is handled by kTPR threads of one workgroup; each thread keeps its
// share of the row in registers, so the row is read from memory once: load,
// amax (wave shuffles, then LDS across the row's waves), quantise, store.
#pragma once
#include "internal.h"

namespace moe {

constexpr int kTPR = 256;                       // threads per row
constexpr int kMaxRowLen = 16384;               // hidden / intermediate bound
constexpr int kBf16Chunks = kMaxRowLen / (8 * kTPR);  // 16-byte chunks of bf16 per thread
constexpr int kF32Chunks = kMaxRowLen / (4 * kTPR);   // 16-byte chunks of fp32 per thread

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
    return v;
}

// Max over aligned segments of GL consecutive lanes (GL a power of two <= 64):
// the group amax when a group's values sit in GL neighbouring lanes.
template <int GL>
__device__ __forceinline__ float segment_max(float v) {
#pragma unroll
    for (int d = GL / 2; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
    return v;
}

// amax over the kTPR threads of row slot `slot` (tr = thread index in the row).
// s_part holds kTPR / kWave floats per slot. Contains one __syncthreads().
__device__ __forceinline__ float row_amax(float m, int slot, int tr, float *s_part) {
    m = wave_max(m);
    if ((tr & (kWave - 1)) == 0) s_part[slot * (kTPR / kWave) + tr / kWave] = m;
    __syncthreads();
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < kTPR / kWave; ++w) a = fmaxf(a, s_part[slot * (kTPR / kWave) + w]);
    return a;
}

// fp32 -> FP8 E4M3 code (OCP "e4m3fn": bias 7, 3 mantissa bits, largest
// finite 448): round to nearest, ties to even, on the E4M3 grid (subnormal
// step 2^-9); magnitudes that round above 448 saturate to 448; NaN -> 0x7F.
// Branch-free: normal values round the fp32 mantissa to 3 bits in integer
// arithmetic (a carry moves into the exponent), then rebias the exponent
// from 127 to 7; below 2^-6 the code is rint(|f| * 2^9).
__host__ __device__ __forceinline__ uint32_t e4m3_code(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t a = u & 0x7FFFFFFFu;
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);   // RNE at mantissa bit 20
    uint32_t nrm = (r >> 20) - (120u << 3);               // (e - 120) << 3 | m
    nrm = nrm < 0x7Eu ? nrm : 0x7Eu;                      // saturate at 448
    const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f));
    const uint32_t c = (a < 0x3C800000u ? sub : nrm) | ((u >> 24) & 0x80u);
    return a > 0x7F800000u ? 0x7Fu : c;
}

// Largest code value of the format: 127 (int8) or 448 (FP8 E4M3).
template <bool FP8>
constexpr float kQMax = FP8 ? 448.0f : 127.0f;

// Four values quantised with one row's inv = 1/a': int8 q = rint((v * 127) *
// inv) in [-127, 127], or FP8 q = e4m3((v * 448) * inv); packed little end
// first.
template <bool FP8 = false>
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float inv) {
    auto q = [inv](float v) -> uint32_t {
        float t = v * kQMax<FP8>;
        t = t * inv;
        if (FP8) return e4m3_code(t);
        float r = __builtin_rintf(t);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        return static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(static_cast<int>(r))));
    };
    return q(a) | (q(b) << 8) | (q(c) << 16) | (q(d) << 24);
}

// Quantise a bf16 row of length n (multiple of 8), optionally times smooth
// scales, into dst; lane tr of slot `slot`. `active` may be false for a
// whole slot (its threads still take part in the barrier). GL > 0: group-wise
// scales ("DeepSeek V4 Decode Optimization" sec. 3.1), one per group of 8 * GL
// elements (the chunks of GL neighbouring lanes), written to scale_out[group];
// no barrier then.
template <bool FP8 = false, int GL = 0>
__device__ __forceinline__ void quant_bf16_row(const uint16_t *src, const float *smooth, int n, float eps,
                                               int8_t *dst, float *scale_out, bool active, int slot, int tr,
                                               float *s_part) {
    float v[kBf16Chunks][8];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < kBf16Chunks; ++j) {
        const int i = (tr + j * kTPR) * 8;
        if (active && i < n) {
            const uint4 raw = *reinterpret_cast<const uint4 *>(src + i);
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[j][2 * e] = bf16_to_f32(static_cast<uint16_t>(w[e] & 0xFFFFu));
                v[j][2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(w[e] >> 16));
            }
            if (smooth) {
                const float4 s0 = *reinterpret_cast<const float4 *>(smooth + i);
                const float4 s1 = *reinterpret_cast<const float4 *>(smooth + i + 4);
                v[j][0] = v[j][0] * s0.x; v[j][1] = v[j][1] * s0.y;
                v[j][2] = v[j][2] * s0.z; v[j][3] = v[j][3] * s0.w;
                v[j][4] = v[j][4] * s1.x; v[j][5] = v[j][5] * s1.y;
                v[j][6] = v[j][6] * s1.z; v[j][7] = v[j][7] * s1.w;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[j][e]));
        }
    }
    if constexpr (GL > 0) {
        if (!active) return;  // whole slots, i.e. whole waves
#pragma unroll
        for (int j = 0; j < kBf16Chunks; ++j) {
            const int i = (tr + j * kTPR) * 8;
            if (j * kTPR * 8 >= n) break;  // uniform
            float mj = 0.0f;
            if (i < n) {
#pragma unroll
                for (int e = 0; e < 8; ++e) mj = fmaxf(mj, fabsf(v[j][e]));
            }
            const float ap = fmaxf(segment_max<GL>(mj), eps);  // a group never straddles n
            const float inv = 1.0f / ap;
            if (i < n) {
                const uint32_t lo = quant4<FP8>(v[j][0], v[j][1], v[j][2], v[j][3], inv);
                const uint32_t hi = quant4<FP8>(v[j][4], v[j][5], v[j][6], v[j][7], inv);
                *reinterpret_cast<uint2 *>(dst + i) = make_uint2(lo, hi);
                if ((tr & (GL - 1)) == 0) scale_out[i / (8 * GL)] = ap * (1.0f / kQMax<FP8>);
            }
        }
        return;
    }
    const float ap = fmaxf(row_amax(m, slot, tr, s_part), eps);
    if (!active) return;
    const float inv = 1.0f / ap;
#pragma unroll
    for (int j = 0; j < kBf16Chunks; ++j) {
        const int i = (tr + j * kTPR) * 8;
        if (i < n) {
            const uint32_t lo = quant4<FP8>(v[j][0], v[j][1], v[j][2], v[j][3], inv);
            const uint32_t hi = quant4<FP8>(v[j][4], v[j][5], v[j][6], v[j][7], inv);
            *reinterpret_cast<uint2 *>(dst + i) = make_uint2(lo, hi);
        }
    }
    if (tr == 0) *scale_out = ap * (1.0f / kQMax<FP8>);
}

// Quantise an fp32 row of length n (multiple of 4) into dst. GL > 0: one
// scale per group of 4 * GL elements, as in quant_bf16_row.
template <bool FP8 = false, int GL = 0>
__device__ __forceinline__ void quant_f32_row(const float *src, int n, float eps, int8_t *dst, float *scale_out,
                                              bool active, int slot, int tr, float *s_part) {
    float4 v[kF32Chunks];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < kF32Chunks; ++j) {
        const int i = (tr + j * kTPR) * 4;
        if (active && i < n) {
            v[j] = *reinterpret_cast<const float4 *>(src + i);
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
        }
    }
    if constexpr (GL > 0) {
        if (!active) return;
#pragma unroll
        for (int j = 0; j < kF32Chunks; ++j) {
            const int i = (tr + j * kTPR) * 4;
            if (j * kTPR * 4 >= n) break;  // uniform
            const float mj = i < n ? fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w)))
                                   : 0.0f;
            const float ap = fmaxf(segment_max<GL>(mj), eps);
            const float inv = 1.0f / ap;
            if (i < n) {
                *reinterpret_cast<uint32_t *>(dst + i) = quant4<FP8>(v[j].x, v[j].y, v[j].z, v[j].w, inv);
                if ((tr & (GL - 1)) == 0) scale_out[i / (4 * GL)] = ap * (1.0f / kQMax<FP8>);
            }
        }
        return;
    }
    const float ap = fmaxf(row_amax(m, slot, tr, s_part), eps);
    if (!active) return;
    const float inv = 1.0f / ap;
#pragma unroll
    for (int j = 0; j < kF32Chunks; ++j) {
        const int i = (tr + j * kTPR) * 4;
        if (i < n) *reinterpret_cast<uint32_t *>(dst + i) = quant4<FP8>(v[j].x, v[j].y, v[j].z, v[j].w, inv);
    }
    if (tr == 0) *scale_out = ap * (1.0f / kQMax<FP8>);
}

}  // namespace moe
