// Grouped FP8 x FP4 GEMMs with fused epilogues: the FP4-weight variant of the
// expert block ("FIFO Pipeline Analysis ... Mega MoE": FP8 GEMMs with FP4
// weights, FP8 cast after SwiGLU), on the CDNA4 block-scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4.
//
//   GEMM1: acc = sum_k e4m3(q_x[r,k]) * e2m1(W1[g,n,k]) * 2^(S1[g,n,k/32]-127)
//     for the gate channel n = j and the up channel I + j; the epilogue is
//     the INT8 one with an fp32 accumulator: y = (acc * w1s[n]) * xs[r],
//     h = (y_g / (1 + exp(-y_g))) * y_u.
//   GEMM2: acc over q_h and W2 likewise; z = bf16((acc * w2s[n]) * hs[r]).
//
// The work decomposition is gemm.hip's decode one (chunks of 16 rows, or of 32
// rows above 16 tokens, a 16-channel tile pair per workgroup, K split over the
// waves, partial tiles summed in LDS, linear blockIdx so every XCD streams a
// share of every expert); only the operands change:
//   - a K step is 128 elements: the FP8 A operand of lane l (row l % 16,
//     g = l / 16) is 32 bytes, row bytes 16g .. +16 (register bytes 0..15)
//     and 64 + 16g .. +16 (bytes 16..31) of the step; the FP4 B operand is 16
//     bytes, elements 32g .. +32 of the step (low nibble first), which is one
//     16-byte slot of a 1 KB packed block exactly as for INT8 weights;
//   - lane l also supplies the E8M0 scale of B row l % 16 for the 32-element
//     block l / 16 of the step: one byte per lane per step, from the scale
//     region of the packed buffer; the A scale is the unit code 127 (the
//     per-row fp32 scale is applied in the epilogue);
//   - accumulation is fp32 inside the MFMA (rounded, unlike the exact int32
//     INT8 path), and the waves' partial tiles are summed in wave order.
// The weight stream is 0.5 B per element plus 1/32 B of scale, so a decode
// step moves about half the bytes of the INT8 path.
#include "internal.h"

#include <hip/hip_ext.h>

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kStepK = 128;        // K elements per MFMA
constexpr int kUnitScale = 127;    // E8M0 code of 1.0

__device__ __forceinline__ v4i ld16(const uint8_t *p) { return *reinterpret_cast<const v4i *>(p); }
__device__ __forceinline__ v4i ld16_stream(const uint8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
}

// KIND 1 = GEMM1 + SwiGLU, 2 = GEMM2 + bf16. KS = 128-element K steps a wave
// loads per batch; NPASS = batches per wave (0: n_pass_rt at run time); MT =
// 16-row tiles per chunk (each weight fragment feeds all of them, so a chunk
// reads its weights once).
// (Four-wave one-tile blocks ask for three resident blocks per CU: the
// register budget of three waves per SIMD, which the 8-step batch fits.)
template <int KIND, int WAVES, int KS, int NPASS, int MT>
__global__ __launch_bounds__(WAVES * kWave, WAVES == 4 && MT == 1 ? 3 : 1) void gemm_mx_kernel(GemmArgs a, int k_dim,
                                                                                                  int n_pass_rt) {
    constexpr int kThreads = WAVES * kWave;
    constexpr int kCols = KIND == 1 ? kTileN : 2 * kTileN;
    constexpr int kElems = kTileN * kCols;
    constexpr int kEpt = (kElems + kThreads - 1) / kThreads;
    const int n_pass = NPASS > 0 ? NPASS : n_pass_rt;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    int c = blockIdx.x / a.n_tiles;
    int nt = blockIdx.x % a.n_tiles;
    int4 ch = a.chunks[c];  // c < max_chunks: inside the chunk list even when unused
    if (c >= a.meta[a.count_word]) return;
    const int nch = ch.z >> kChunkCountShift;
    if (nch > 1 && (a.n_tiles & 7) == 0) {
        // the chunks of one N tile 8 blocks apart: same XCD, weights shared in L2
        const int c0 = c - ch.w;
        const int i = blockIdx.x - c0 * a.n_tiles;
        const int q = i / (8 * nch), rem = i - q * 8 * nch;
        c = c0 + rem / 8;
        nt = q * 8 + rem % 8;
        ch = a.chunks[c];
    }
    const int g = ch.x, row0 = ch.y, rows = ch.z & kChunkRowsMask;
    if (g < a.g_lo || g >= a.g_hi) return;
    const bool routed = g < a.E_loc;
    const int inter = routed ? a.I : a.I_s;
    const int Kd = k_dim;

    // Packed buffer of one weight tensor: the element blocks of every group,
    // then the scale blocks of every group.
    const int n_out = KIND == 1 ? 2 * inter : a.H;  // output channels per group
    const size_t g_data = static_cast<size_t>(n_out) * (Kd / 2);
    const size_t g_scale = static_cast<size_t>(n_out) * (Kd / 32);
    const size_t n_groups = routed ? a.E_loc : 1;
    const size_t gi = routed ? g : 0;
    const uint8_t *base = reinterpret_cast<const uint8_t *>(routed ? a.W : a.W_sh);
    const uint8_t *Wd = base + gi * g_data;
    const uint8_t *Wsc = base + n_groups * g_data + gi * g_scale;
    const float *Ws;
    size_t ta, tb;  // packed tile positions of the two weight tiles
    if (KIND == 1) {
        if (nt * kTileN >= inter) return;
        Ws = routed ? a.Ws + static_cast<size_t>(g) * 2 * inter : a.Ws_sh;
        ta = g1_tile_pos(nt, inter / kTileN);
        tb = g1_tile_pos(inter / kTileN + nt, inter / kTileN);
    } else {
        if (nt * 2 * kTileN >= a.H) return;
        Ws = routed ? a.Ws + static_cast<size_t>(g) * a.H : a.Ws_sh;
        ta = 2 * static_cast<size_t>(nt);
        tb = ta + 1;
    }
    const int r16 = lane & 15, kg = lane >> 4;
    const size_t steps_k = Kd / kStepK;
    const int step0 = wave * KS * n_pass;

    // (1) independent small loads (activation row index, epilogue rows,
    //     channel scales) ahead of the weight stream
    const int32_t *aidx = KIND == 1 ? (routed ? a.idx_r : a.row_token) : nullptr;
    // epilogue rows' index: GEMM1 the activation scale's row, GEMM2 the z row
    // (pair id) of a routed row or the share_output row of a shared one
    const int32_t *tidx = KIND == 1 ? aidx : (routed ? a.zrow : a.row_token);
    const uint8_t *Abase = reinterpret_cast<const uint8_t *>(KIND == 1 ? (routed ? a.A_r : a.A_s) : a.A);
    const float *Ascale = KIND == 1 ? (routed ? a.a_scale_r : a.a_scale_s) : a.a_scale;
    int arow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int lr = min(mt * kTileN + r16, rows - 1);
        arow[mt] = KIND == 1 ? aidx[row0 + lr] : row0 + lr;
    }
    const int jc = tid % kCols;
    const int col = (KIND == 1 ? nt * kTileN : nt * 2 * kTileN) + jc;
    const float wsc0 = Ws[col];
    const float wsc1 = KIND == 1 ? Ws[inter + col] : 0.0f;
    int rrow[kEpt], rtok[kEpt];
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
        rrow[e] = row0 + min(min(tid + e * kThreads, kElems - 1) / kCols, rows - 1);
        rtok[e] = tidx[rrow[e]];
    }
    __builtin_amdgcn_sched_barrier(0);

    // (2) first weight batch: 1 KB element blocks and 64-byte scale blocks
    const uint8_t *pw0 = Wd + (ta * steps_k + step0) * 1024 + lane * 16;
    const uint8_t *pw1 = Wd + (tb * steps_k + step0) * 1024 + lane * 16;
    const uint8_t *ps0 = Wsc + (ta * steps_k + step0) * 64 + lane;
    const uint8_t *ps1 = Wsc + (tb * steps_k + step0) * 64 + lane;
    v4i wbuf[2][2][KS];
    int sbuf[2][2][KS];
    auto ldw = [&](v4i (&w)[2][KS], int (&sc)[2][KS], int pass) {
        const size_t sp = static_cast<size_t>(pass) * KS;
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            w[0][i] = ld16_stream(pw0 + (sp + i) * 1024);
            w[1][i] = ld16_stream(pw1 + (sp + i) * 1024);
            sc[0][i] = ps0[(sp + i) * 64];
            sc[1][i] = ps1[(sp + i) * 64];
        }
    };
    ldw(wbuf[0], sbuf[0], 0);
    __builtin_amdgcn_sched_barrier(0);

    // (3) row scales of the epilogue rows
    float rsc[kEpt];
#pragma unroll
    for (int e = 0; e < kEpt; ++e) rsc[e] = Ascale[KIND == 1 ? rtok[e] : rrow[e]];
    __builtin_amdgcn_sched_barrier(0);

    const uint8_t *pa[MT];
    v4f acc0[MT], acc1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        pa[mt] = Abase + static_cast<size_t>(arow[mt]) * a.a_stride + static_cast<size_t>(step0) * kStepK + kg * 16;
        acc0[mt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        acc1[mt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // One K batch: this batch's A rows, then (if any) the next weight batch,
    // then the MFMAs. Row tiles past the chunk's rows are skipped (uniform).
    auto batch = [&](const v4i (&w)[2][KS], const int (&sc)[2][KS], v4i (&nw)[2][KS], int (&nsc)[2][KS], int pass,
                     bool has_next) {
        v4i x0[MT][KS], x1[MT][KS];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (MT == 1 || mt * kTileN < rows) {
                const uint8_t *pam = pa[mt] + static_cast<size_t>(pass) * KS * kStepK;
#pragma unroll
                for (int i = 0; i < KS; ++i) {
                    x0[mt][i] = ld16(pam + i * kStepK);
                    x1[mt][i] = ld16(pam + i * kStepK + 64);
                }
            }
        }
        if (has_next) ldw(nw, nsc, pass + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (MT == 1 || mt * kTileN < rows) {
                const bool av = mt * kTileN + r16 < rows;
#pragma unroll
                for (int i = 0; i < KS; ++i) {
                    const v4i lo = av ? x0[mt][i] : v4i{0, 0, 0, 0};
                    const v4i hi = av ? x1[mt][i] : v4i{0, 0, 0, 0};
                    const v8i xa = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    const v8i b0 = {w[0][i][0], w[0][i][1], w[0][i][2], w[0][i][3], 0, 0, 0, 0};
                    const v8i b1 = {w[1][i][0], w[1][i][1], w[1][i][2], w[1][i][3], 0, 0, 0, 0};
                    // cbsz 0: A is FP8 E4M3; blgp 4: B is FP4 E2M1 (4 registers)
                    acc0[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa, b0, acc0[mt], 0, 4, 0, kUnitScale,
                                                                                0, sc[0][i]);
                    acc1[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa, b1, acc1[mt], 0, 4, 0, kUnitScale,
                                                                                0, sc[1][i]);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (NPASS > 0) {
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass)
            batch(wbuf[pass & 1], sbuf[pass & 1], wbuf[(pass + 1) & 1], sbuf[(pass + 1) & 1], pass, pass + 1 < NPASS);
    } else {
        for (int pass = 0; pass < n_pass; pass += 2) {
            batch(wbuf[0], sbuf[0], wbuf[1], sbuf[1], pass, pass + 1 < n_pass);
            if (pass + 1 < n_pass) batch(wbuf[1], sbuf[1], wbuf[0], sbuf[0], pass + 1, pass + 2 < n_pass);
        }
    }

    __shared__ float red[WAVES][2][kTileN][kTileN];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
    if (mt * kTileN >= rows) break;  // uniform
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        red[wave][0][4 * kg + i][r16] = acc0[mt][i];
        red[wave][1][4 * kg + i][r16] = acc1[mt][i];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
        const int idx = tid + e * kThreads;
        const int m = idx / kCols;
        const int lr = mt * kTileN + m;
        if (idx < kElems && lr < rows) {
            const int r = row0 + lr;
            // the first tile's row scales and tokens were fetched up front
            const float rs = mt == 0 ? rsc[e] : Ascale[KIND == 1 ? aidx[r] : r];
            if (KIND == 1) {
                float ag = 0.0f, au = 0.0f;
#pragma unroll
                for (int w = 0; w < WAVES; ++w) {
                    ag += red[w][0][m][jc];
                    au += red[w][1][m][jc];
                }
                a.h[static_cast<size_t>(r) * a.imax + col] = swiglu(ag, au, wsc0, wsc1, rs);
                if (a.dbg_acc) {
                    a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + col] = __float_as_int(ag);
                    a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + inter + col] = __float_as_int(au);
                }
            } else {
                float acc = 0.0f;
#pragma unroll
                for (int w = 0; w < WAVES; ++w) acc += red[w][jc / kTileN][m][jc % kTileN];
                const uint16_t zb = f32_to_bf16(dequant(acc, wsc0, rs));
                const int t = mt == 0 ? rtok[e] : tidx[r];
                (routed ? a.z : a.share_out)[static_cast<size_t>(t) * a.H + col] = zb;
                if (a.dbg_acc) a.dbg_acc[static_cast<size_t>(r) * a.H + col] = __float_as_int(acc);
                if (a.dbg_z) a.dbg_z[static_cast<size_t>(r) * a.H + col] = zb;
            }
        }
    }
    __syncthreads();
    }
}

template <int KIND, int WAVES, int KS, int NPASS, int MT>
hipError_t launch_one(const GemmArgs &a, dim3 grid, int k_dim, int n_pass, hipStream_t s, hipEvent_t e0,
                      hipEvent_t e1) {
    const dim3 blk(WAVES * kWave);
    if (e0 || e1)
        hipExtLaunchKernelGGL((gemm_mx_kernel<KIND, WAVES, KS, NPASS, MT>), grid, blk, 0, s, e0, e1, 0, a, k_dim,
                              n_pass);
    else
        hipLaunchKernelGGL((gemm_mx_kernel<KIND, WAVES, KS, NPASS, MT>), grid, blk, 0, s, a, k_dim, n_pass);
    return hipGetLastError();
}

// K is split over MOE_MX_WAVES waves when its 128-element steps divide by
// that, else over 4 or 2 (k_dim % 256 == 0, so the step count is even). With
// at most 8 steps per wave a wave loads its whole slice in one batch; longer
// slices go in batches of 4, 2 or 1 steps, software pipelined. 4 waves (8
// steps, 256 bytes per lane in flight at hidden 4096) beat 8 waves (4 steps)
// on the decode workload: GEMM1 78 us against 83 us on MI355X.
#ifndef MOE_MX_WAVES
#define MOE_MX_WAVES 4
#endif
template <int KIND, int W, int MT>
hipError_t launch_split(const GemmArgs &a, dim3 grid, int k_dim, int spw, hipStream_t s, hipEvent_t e0,
                        hipEvent_t e1) {
    switch (spw) {
        case 1: return launch_one<KIND, W, 1, 1, MT>(a, grid, k_dim, 1, s, e0, e1);
        case 2: return launch_one<KIND, W, 2, 1, MT>(a, grid, k_dim, 1, s, e0, e1);
        case 3: return launch_one<KIND, W, 3, 1, MT>(a, grid, k_dim, 1, s, e0, e1);
        case 4: return launch_one<KIND, W, 4, 1, MT>(a, grid, k_dim, 1, s, e0, e1);
        case 5: return launch_one<KIND, W, 5, 1, MT>(a, grid, k_dim, 1, s, e0, e1);
        case 6: return launch_one<KIND, W, 6, 1, MT>(a, grid, k_dim, 1, s, e0, e1);
        case 7: return launch_one<KIND, W, 7, 1, MT>(a, grid, k_dim, 1, s, e0, e1);
        case 8: return launch_one<KIND, W, 8, 1, MT>(a, grid, k_dim, 1, s, e0, e1);
        default: break;
    }
    if (spw % 4 == 0) return launch_one<KIND, W, 4, 0, MT>(a, grid, k_dim, spw / 4, s, e0, e1);
    if (spw % 2 == 0) return launch_one<KIND, W, 2, 0, MT>(a, grid, k_dim, spw / 2, s, e0, e1);
    return launch_one<KIND, W, 1, 0, MT>(a, grid, k_dim, spw, s, e0, e1);
}

// One row tile per chunk (batches of at most 16 tokens) splits K over
// MOE_MX_WAVES waves; two row tiles (32-row chunks, larger batches) over 8,
// which keeps a wave's A and weight registers of a batch within budget.
#ifndef MOE_MX_WIDE_KS
#define MOE_MX_WIDE_KS 0  // two row tiles: steps per batch (0: the whole slice when it is at most 8 steps)
#endif
template <int KIND, int MT>
hipError_t launch_mt(const GemmArgs &a, dim3 grid, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    constexpr int W = MT == 1 ? MOE_MX_WAVES : 8;
    const int steps = k_dim / kStepK;
    if constexpr (MT == 2 && MOE_MX_WIDE_KS > 0) {
        if (steps % (W * MOE_MX_WIDE_KS) == 0)
            return launch_one<KIND, W, MOE_MX_WIDE_KS, 0, MT>(a, grid, k_dim, steps / (W * MOE_MX_WIDE_KS), s, e0,
                                                               e1);
    }
    if (steps % W == 0) return launch_split<KIND, W, MT>(a, grid, k_dim, steps / W, s, e0, e1);
    if (steps % 4 == 0) return launch_one<KIND, 4, 1, 0, MT>(a, grid, k_dim, steps / 4, s, e0, e1);
    return launch_one<KIND, 2, 1, 0, MT>(a, grid, k_dim, steps / 2, s, e0, e1);
}

template <int KIND>
hipError_t launch_kind(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    static_assert(MOE_MX_WAVES == 8 || MOE_MX_WAVES == 4, "MOE_MX_WAVES is 8 or 4");
    if ((a.mt != 1 && a.mt != 2) || k_dim % 256) return hipErrorInvalidValue;
    const long blocks = static_cast<long>(max_chunks) * a.n_tiles;
    if (blocks <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(blocks));
    return a.mt == 1 ? launch_mt<KIND, 1>(a, grid, k_dim, s, e0, e1) : launch_mt<KIND, 2>(a, grid, k_dim, s, e0, e1);
}

}  // namespace

hipError_t launch_gemm1_mx(const GemmArgs &a, int max_chunks, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
    return launch_kind<1>(a, max_chunks, a.H, s, ev_start, ev_stop);
}

hipError_t launch_gemm2_mx(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t ev_start,
                           hipEvent_t ev_stop) {
    return launch_kind<2>(a, max_chunks, k_dim, s, ev_start, ev_stop);
}

}  // namespace moe
