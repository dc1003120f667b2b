// Grouped INT8 GEMMs on CDNA4 MFMA (v_mfma_i32_16x16x64_i8) with fused
// epilogues.
//
//   GEMM1 ("FusedDeepMoE Kernel 深度分析报告" sec. 3.3 / 5.2.1 / 6.1):
//     acc = q_x[r,:] . W1[g, n, :] for the gate channel n = j and the up
//     channel n = I + j of the same work item, so the epilogue holds both
//     halves of SwiGLU: y = (float(acc) * w1s[n]) * xs[r];
//     h = (y_g / (1 + exp(-y_g))) * y_u, written as fp32.
//   GEMM2 (sec. 3.4 / 5.2.2 / 6.2):
//     acc = q_h[r,:] . W2[g, n, :];  z = bf16((float(acc) * w2s[n]) * hs[r]),
//     to the routed row buffer, or straight into share_output for the shared
//     expert (sec. 6.2: the shared expert's rows go to memory, routed rows on
//     to combine).
//
// Decode is bound by the weight stream (each touched expert's bytes are read
// once; per-expert rows M are 1..64), so the kernel is shaped around HBM, not
// around MFMA throughput:
//   - a work item is (chunk of <= 64 rows of one expert, 16-channel N tile
//     pair); its 2 x 16 weight rows are split over the waves along K, and each
//     wave pulls its whole K slice into registers with 16-byte loads up
//     front, so a workgroup keeps 64-128 KB of weights in flight;
//   - with packed weights (moe_w8a8_pack_weights) every wave load is one
//     contiguous 1 KB block, read non-temporally;
//   - the weights stay in registers while the chunk's 16-row MFMA tiles are
//     swept, so a chunk reads its weight slice exactly once;
//   - the partial int32 tiles of the waves are summed in LDS (exact);
//   - blockIdx maps linearly to (chunk, N tile), so the round-robin placement
//     of blocks on the 8 XCDs gives each XCD an equal share of every expert;
//   - the epilogue's scales are fetched before the weight stream starts.
// MFMA operand layout: lane l holds 16 bytes of row (l % 16) at byte offset
// 16 * (l / 16) of a 64-byte K step, for A (token rows) and B (weight rows)
// alike, so every product pairs equal K indices. Result lane l, register i
// holds D[4 * (l / 16) + i][l % 16].
#include "internal.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kMT = kChunkRows / kTileN;  // row tiles per chunk

__device__ __forceinline__ v4i ld16(const int8_t *p) { return *reinterpret_cast<const v4i *>(p); }
__device__ __forceinline__ v4i ld16_stream(const int8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
}

template <int KIND, int WAVES, int KSTEPS, bool PACKED>
__global__ __launch_bounds__(WAVES * kWave) void gemm_kernel(GemmArgs a, int k_dim, int n_pass) {
    constexpr int kThreads = WAVES * kWave;
    constexpr int kCols = KIND == 1 ? kTileN : 2 * kTileN;  // output columns of one work item
    constexpr int kElems = kTileN * kCols;                   // outputs of one 16-row tile
    constexpr int kEpt = (kElems + kThreads - 1) / kThreads; // outputs per thread per tile
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    // Work item = (chunk, N tile), linear in blockIdx: the hardware deals
    // consecutive blocks round-robin to the 8 XCDs, so every XCD streams an
    // equal share of every expert's weights (whole chunks per XCD left the
    // XCDs up to one expert apart).
    const int c = blockIdx.x / a.n_tiles;
    const int nt = blockIdx.x % a.n_tiles;
    const int4 ch = a.chunks[c];  // c < max_chunks: inside the chunk list even when unused
    if (c >= a.meta[kMetaChunks]) return;
    const int g = ch.x, row0 = ch.y, rows = ch.z;
    if (g < a.g_lo || g >= a.g_hi) return;
    const bool routed = g < a.E_loc;
    const int inter = routed ? a.I : a.I_s;

    const int8_t *W;
    const float *Ws;
    int rowA, rowB;
    if (KIND == 1) {
        if (nt * kTileN >= inter) return;
        W = routed ? a.W + static_cast<size_t>(g) * 2 * inter * a.H : a.W_sh;
        Ws = routed ? a.Ws + static_cast<size_t>(g) * 2 * inter : a.Ws_sh;
        rowA = nt * kTileN;           // gate channels
        rowB = inter + nt * kTileN;   // matching up channels
    } else {
        if (nt * 2 * kTileN >= a.H) return;
        W = routed ? a.W + static_cast<size_t>(g) * a.H * inter : a.W_sh;
        Ws = routed ? a.Ws + static_cast<size_t>(g) * a.H : a.Ws_sh;
        rowA = nt * 2 * kTileN;
        rowB = rowA + kTileN;
    }
    const int Kd = k_dim;
    const int r16 = lane & 15, kg = lane >> 4;
    const int step0 = wave * KSTEPS * n_pass;  // first 64-byte K step of this wave
    // Row-major weights: lane reads 16 bytes of row (tile row + l%16) at byte
    // 64*step + 16*(l/16). Packed weights (moe_w8a8_pack_weights) hold exactly
    // those bytes as one contiguous 1 KB block per (16-row tile, step), so a
    // wave's load is 1 KB contiguous and consecutive steps are adjacent.
    const int8_t *pw0, *pw1;
    size_t wstep;
    if (PACKED) {
        const size_t steps_k = Kd / 64;
        pw0 = W + ((rowA / kTileN) * steps_k + step0) * 1024 + lane * 16;
        pw1 = W + ((rowB / kTileN) * steps_k + step0) * 1024 + lane * 16;
        wstep = 1024;
    } else {
        pw0 = W + static_cast<size_t>(rowA + r16) * Kd + step0 * 64 + kg * 16;
        pw1 = W + static_cast<size_t>(rowB + r16) * Kd + step0 * 64 + kg * 16;
        wstep = 64;
    }
    // GEMM1 rows of groups without smooth scales read the per-token rows of
    // x (quantised once per token); every other A row is the grouped row.
    const bool by_tok = KIND == 1 && (routed ? a.routed_by_token : a.shared_by_token);
    const int8_t *Abase = by_tok ? a.A_tok : a.A;
    const float *Ascale = by_tok ? a.a_scale_tok : a.a_scale;
    int arow[kMT];  // source row of this lane's A operand in each row tile
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        const int lr = mt * kTileN + r16;
        arow[mt] = lr < rows ? (by_tok ? a.row_token[row0 + lr] : row0 + lr) : 0;
    }

    // Epilogue operands of the first row tile, fetched before the weight
    // stream so that their latency hides under it. A thread's output column
    // is the same in every row tile (kThreads is a multiple of kCols).
    const int jc = tid % kCols;
    const int col = (KIND == 1 ? nt * kTileN : nt * 2 * kTileN) + jc;
    float wsc0 = 0.0f, wsc1 = 0.0f;
    if (tid < kElems) {
        wsc0 = Ws[col];
        if (KIND == 1) wsc1 = Ws[inter + col];
    }
    float rsc[kEpt];
    int rtok[kEpt];
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
        const int m = (tid + e * kThreads) / kCols;
        rsc[e] = 0.0f;
        rtok[e] = 0;
        if (tid + e * kThreads < kElems && m < rows) {
            rsc[e] = Ascale[by_tok ? a.row_token[row0 + m] : row0 + m];
            if (KIND == 2 && !routed) rtok[e] = a.row_token[row0 + m];
        }
    }

    v4i acc0[kMT], acc1[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        acc0[mt] = v4i{0, 0, 0, 0};
        acc1[mt] = v4i{0, 0, 0, 0};
    }

    for (int pass = 0; pass < n_pass; ++pass) {
        v4i w0[KSTEPS], w1[KSTEPS];
        const int sp = pass * KSTEPS;
#pragma unroll
        for (int i = 0; i < KSTEPS; ++i) {
            // streamed weights: non-temporal when each wave load is a whole
            // contiguous 1 KB block, plain loads for 64-byte row segments
            if (PACKED) {
                w0[i] = ld16_stream(pw0 + (sp + i) * wstep);
                w1[i] = ld16_stream(pw1 + (sp + i) * wstep);
            } else {
                w0[i] = ld16(pw0 + (sp + i) * wstep);
                w1[i] = ld16(pw1 + (sp + i) * wstep);
            }
        }
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            if (mt * kTileN < rows) {
                const bool av = mt * kTileN + r16 < rows;
                const int8_t *pam = Abase + static_cast<size_t>(arow[mt]) * a.a_stride + (step0 + sp) * 64 + kg * 16;
#pragma unroll
                for (int i = 0; i < KSTEPS; ++i) {
                    const v4i x = av ? ld16(pam + i * 64) : v4i{0, 0, 0, 0};
                    acc0[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x, w0[i], acc0[mt], 0, 0, 0);
                    acc1[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x, w1[i], acc1[mt], 0, 0, 0);
                }
            }
        }
    }

    __shared__ int red[WAVES][2][kTileN][kTileN];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        if (mt * kTileN >= rows) break;
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
                const float rs = mt == 0 ? rsc[e] : Ascale[by_tok ? a.row_token[r] : r];
                if (KIND == 1) {
                    int ag = 0, au = 0;
#pragma unroll
                    for (int w = 0; w < WAVES; ++w) {
                        ag += red[w][0][m][jc];
                        au += red[w][1][m][jc];
                    }
                    float yg = static_cast<float>(ag) * wsc0;
                    yg = yg * rs;
                    float yu = static_cast<float>(au) * wsc1;
                    yu = yu * rs;
                    const float ex = expf(-yg);
                    const float den = 1.0f + ex;
                    const float sg = yg / den;
                    a.h[static_cast<size_t>(r) * a.imax + col] = sg * yu;
                    if (a.dbg_acc) {
                        a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + col] = ag;
                        a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + inter + col] = au;
                    }
                } else {
                    int acc = 0;
#pragma unroll
                    for (int w = 0; w < WAVES; ++w) acc += red[w][jc / kTileN][m][jc % kTileN];
                    float y = static_cast<float>(acc) * wsc0;
                    y = y * rs;
                    const uint16_t zb = f32_to_bf16(y);
                    if (routed) {
                        a.z[static_cast<size_t>(r) * a.H + col] = zb;
                    } else {
                        const int t = mt == 0 ? rtok[e] : a.row_token[r];
                        a.share_out[static_cast<size_t>(t) * a.H + col] = zb;
                    }
                    if (a.dbg_acc) a.dbg_acc[static_cast<size_t>(r) * a.H + col] = acc;
                    if (a.dbg_z) a.dbg_z[static_cast<size_t>(r) * a.H + col] = zb;
                }
            }
        }
        __syncthreads();
    }
}

// Tuning (measured on MI355X for the decode shapes): waves per workgroup and
// the number of 64-byte K steps a wave loads per batch (fewer steps per batch
// = fewer VGPRs = more resident waves streaming).
#ifndef MOE_GEMM1_WAVES
#define MOE_GEMM1_WAVES 4
#endif
#ifndef MOE_GEMM1_KSTEPS
#define MOE_GEMM1_KSTEPS 4
#endif
#ifndef MOE_GEMM2_WAVES
#define MOE_GEMM2_WAVES 8
#endif
#ifndef MOE_GEMM2_KSTEPS
#define MOE_GEMM2_KSTEPS 1
#endif

template <int KIND, int WAVES, bool PACKED>
hipError_t launch_impl(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s) {
    const int steps = k_dim / (64 * WAVES);
    int ks = KIND == 1 ? MOE_GEMM1_KSTEPS : MOE_GEMM2_KSTEPS;
    while (ks > 1 && steps % ks) ks >>= 1;
    const int n_pass = steps / ks;
    const long grid = static_cast<long>(max_chunks) * a.n_tiles;
    if (grid <= 0) return hipSuccess;
    const dim3 blk(WAVES * kWave);
    switch (ks) {
        case 16: hipLaunchKernelGGL((gemm_kernel<KIND, WAVES, 16, PACKED>), dim3(grid), blk, 0, s, a, k_dim, n_pass); break;
        case 8: hipLaunchKernelGGL((gemm_kernel<KIND, WAVES, 8, PACKED>), dim3(grid), blk, 0, s, a, k_dim, n_pass); break;
        case 4: hipLaunchKernelGGL((gemm_kernel<KIND, WAVES, 4, PACKED>), dim3(grid), blk, 0, s, a, k_dim, n_pass); break;
        case 2: hipLaunchKernelGGL((gemm_kernel<KIND, WAVES, 2, PACKED>), dim3(grid), blk, 0, s, a, k_dim, n_pass); break;
        default: hipLaunchKernelGGL((gemm_kernel<KIND, WAVES, 1, PACKED>), dim3(grid), blk, 0, s, a, k_dim, n_pass); break;
    }
    return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s) {
    // k_dim is a multiple of 256 (64-byte MFMA K step x 4 waves)
    if constexpr ((KIND == 1 ? MOE_GEMM1_WAVES : MOE_GEMM2_WAVES) == 8) {
        if (k_dim % 512 == 0)
            return a.packed ? launch_impl<KIND, 8, true>(a, max_chunks, k_dim, s)
                            : launch_impl<KIND, 8, false>(a, max_chunks, k_dim, s);
    }
    return a.packed ? launch_impl<KIND, 4, true>(a, max_chunks, k_dim, s)
                    : launch_impl<KIND, 4, false>(a, max_chunks, k_dim, s);
}

}  // namespace

hipError_t launch_gemm1(const GemmArgs &a, int max_chunks, hipStream_t s) {
    return launch_kind<1>(a, max_chunks, a.H, s);
}

hipError_t launch_gemm2(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s) {
    return launch_kind<2>(a, max_chunks, k_dim, s);
}

}  // namespace moe
