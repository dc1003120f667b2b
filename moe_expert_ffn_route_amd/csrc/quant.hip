// Per-row dynamic INT8 quantisation, one wavefront per grouped row.
//
// The rule ("FusedDeepMoE Kernel 深度分析报告" sec. 7.2 BlockQuant, with the
// eps floor of "DeepSeek V4 Decode Optimization" sec. 0):
//   a' = max(max_i |v_i|, eps);  scale = a' * (1/127);
//   q_i = rint((v_i * 127) * (1/a'))  (round to nearest even)
// Every product is a separate IEEE fp32 operation (the library is built with
// -ffp-contract=off) and 1/a' is a correctly rounded division, so the codes
// are the exact function of the fp32 inputs that the rule defines.
//
// quant_kernel gathers the GEMM1 input: grouped row r reads token row_token[r]
// of x (bf16), times the smooth scales of its expert when given (sec. 1.2
// expert_smooth_scales / share_smooth_scales), so the quantisation of the
// dispatch step (sec. 4.1) and the gather into expert order are one pass.
// requant_kernel quantises the SwiGLU output h of each row (sec. 7.2).
//
// Both kernels are HBM/L2-bound and tiny next to the weight stream: a row is
// read twice (amax pass, then quantise pass; the second read hits the cache)
// with 16-byte loads.
#include "internal.h"

namespace moe {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 waves, one row each

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
    return v;
}

__device__ __forceinline__ int8_t quant_one(float v, float inv) {
    float t = v * 127.0f;
    t = t * inv;
    float r = __builtin_rintf(t);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return static_cast<int8_t>(static_cast<int>(r));
}

// 8 consecutive x values of one token, times the smooth scales if present.
__device__ __forceinline__ void load8(const uint16_t *xr, const float *sm, int i, float v[8]) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(xr + i);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16_to_f32(static_cast<uint16_t>(w[j] & 0xFFFFu));
        v[2 * j + 1] = bf16_to_f32(static_cast<uint16_t>(w[j] >> 16));
    }
    if (sm) {
        const float4 s0 = *reinterpret_cast<const float4 *>(sm + i);
        const float4 s1 = *reinterpret_cast<const float4 *>(sm + i + 4);
        v[0] = v[0] * s0.x; v[1] = v[1] * s0.y; v[2] = v[2] * s0.z; v[3] = v[3] * s0.w;
        v[4] = v[4] * s1.x; v[5] = v[5] * s1.y; v[6] = v[6] * s1.z; v[7] = v[7] * s1.w;
    }
}

__global__ __launch_bounds__(kRowsPerBlock * kWave) void quant_kernel(QuantArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int r = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    const int nrows = a.meta[kMetaP] + (a.has_shared ? a.meta[kMetaTAct] : 0);
    if (r >= nrows) return;
    const int t = a.row_token[r];
    const int g = a.row_group[r];
    const float *sm = g < a.E_loc ? (a.smooth ? a.smooth + static_cast<size_t>(g) * a.H : nullptr)
                                  : a.share_smooth;
    const uint16_t *xr = a.x + static_cast<size_t>(t) * a.H;

    float amax = 0.0f;
    for (int i = lane * 8; i < a.H; i += kWave * 8) {
        float v[8];
        load8(xr, sm, i, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    }
    amax = wave_max(amax);
    const float ap = fmaxf(amax, a.eps);
    const float inv = 1.0f / ap;
    int8_t *qr = a.q + static_cast<size_t>(r) * a.H;
    for (int i = lane * 8; i < a.H; i += kWave * 8) {
        float v[8];
        load8(xr, sm, i, v);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo |= (static_cast<uint32_t>(static_cast<uint8_t>(quant_one(v[j], inv))) << (8 * j));
            hi |= (static_cast<uint32_t>(static_cast<uint8_t>(quant_one(v[4 + j], inv))) << (8 * j));
        }
        *reinterpret_cast<uint2 *>(qr + i) = make_uint2(lo, hi);
    }
    if (lane == 0) a.scale[r] = ap * (1.0f / 127.0f);
}

__global__ __launch_bounds__(kRowsPerBlock * kWave) void requant_kernel(RequantArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int r = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    const int nrows = a.meta[kMetaP] + (a.has_shared ? a.meta[kMetaTAct] : 0);
    if (r >= nrows) return;
    const int n = a.row_group[r] < a.E_loc ? a.I : a.I_s;
    const float *hr = a.h + static_cast<size_t>(r) * a.imax;

    float amax = 0.0f;
    for (int i = lane * 4; i < n; i += kWave * 4) {
        const float4 v = *reinterpret_cast<const float4 *>(hr + i);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    amax = wave_max(amax);
    const float ap = fmaxf(amax, a.eps);
    const float inv = 1.0f / ap;
    int8_t *qr = a.q + static_cast<size_t>(r) * a.imax;
    for (int i = lane * 4; i < n; i += kWave * 4) {
        const float4 v = *reinterpret_cast<const float4 *>(hr + i);
        const uint32_t packed = static_cast<uint32_t>(static_cast<uint8_t>(quant_one(v.x, inv))) |
                                (static_cast<uint32_t>(static_cast<uint8_t>(quant_one(v.y, inv))) << 8) |
                                (static_cast<uint32_t>(static_cast<uint8_t>(quant_one(v.z, inv))) << 16) |
                                (static_cast<uint32_t>(static_cast<uint8_t>(quant_one(v.w, inv))) << 24);
        *reinterpret_cast<uint32_t *>(qr + i) = packed;
    }
    if (lane == 0) a.scale[r] = ap * (1.0f / 127.0f);
}

}  // namespace

hipError_t launch_quant(const QuantArgs &a, hipStream_t s) {
    const int blocks = (a.rows_max + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(quant_kernel, dim3(blocks), dim3(kRowsPerBlock * kWave), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_requant(const RequantArgs &a, hipStream_t s) {
    const int blocks = (a.rows_max + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(requant_kernel, dim3(blocks), dim3(kRowsPerBlock * kWave), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
