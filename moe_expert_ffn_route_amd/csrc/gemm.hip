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
//     wave pulls its whole K slice into registers with 16-byte non-temporal
//     loads up front, so a workgroup keeps 64-128 KB of weights in flight;
//   - the weights stay in registers while the chunk's 16-row MFMA tiles are
//     swept, so a chunk reads its weight slice exactly once;
//   - the partial int32 tiles of the waves are summed in LDS (exact);
//   - blockIdx is mapped so that all N tiles of one chunk run on one XCD
//     (hardware places block b on XCD b % 8), keeping the chunk's activation
//     rows in that XCD's L2.
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

template <int KIND, int WAVES, int KSTEPS>
__global__ __launch_bounds__(WAVES * kWave) void gemm_kernel(GemmArgs a, int k_dim, int n_pass) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int b = blockIdx.x;
    const int q = b >> 3;
    const int nt = q % a.n_tiles;
    const int c = (b & 7) + 8 * (q / a.n_tiles);
    if (c >= a.meta[kMetaChunks]) return;
    const int4 ch = a.chunks[c];
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
    const int kw0 = wave * (KSTEPS * n_pass) * 64 + kg * 16;
    const int8_t *pw0 = W + static_cast<size_t>(rowA + r16) * Kd + kw0;
    const int8_t *pw1 = W + static_cast<size_t>(rowB + r16) * Kd + kw0;
    const int8_t *pa = a.A + static_cast<size_t>(row0 + r16) * a.a_stride + kw0;

    v4i acc0[kMT], acc1[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        acc0[mt] = v4i{0, 0, 0, 0};
        acc1[mt] = v4i{0, 0, 0, 0};
    }

    for (int pass = 0; pass < n_pass; ++pass) {
        v4i w0[KSTEPS], w1[KSTEPS];
        const int kp = pass * KSTEPS * 64;
#pragma unroll
        for (int i = 0; i < KSTEPS; ++i) {
            w0[i] = ld16_stream(pw0 + kp + i * 64);
            w1[i] = ld16_stream(pw1 + kp + i * 64);
        }
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            if (mt * kTileN < rows) {
                const bool av = mt * kTileN + r16 < rows;
                const int8_t *pam = pa + static_cast<size_t>(mt * kTileN) * a.a_stride + kp;
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
        if (KIND == 1) {
            for (int idx = tid; idx < kTileN * kTileN; idx += WAVES * kWave) {
                const int m = idx / kTileN, j = idx % kTileN;
                const int lr = mt * kTileN + m;
                if (lr < rows) {
                    int ag = 0, au = 0;
#pragma unroll
                    for (int w = 0; w < WAVES; ++w) {
                        ag += red[w][0][m][j];
                        au += red[w][1][m][j];
                    }
                    const int r = row0 + lr;
                    const int col = nt * kTileN + j;
                    const float xs = a.a_scale[r];
                    float yg = static_cast<float>(ag) * Ws[col];
                    yg = yg * xs;
                    float yu = static_cast<float>(au) * Ws[inter + col];
                    yu = yu * xs;
                    const float e = expf(-yg);
                    const float den = 1.0f + e;
                    const float s = yg / den;
                    a.h[static_cast<size_t>(r) * a.imax + col] = s * yu;
                    if (a.dbg_acc) {
                        a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + col] = ag;
                        a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + inter + col] = au;
                    }
                }
            }
        } else {
            for (int idx = tid; idx < kTileN * 2 * kTileN; idx += WAVES * kWave) {
                const int m = idx / (2 * kTileN), jj = idx % (2 * kTileN);
                const int lr = mt * kTileN + m;
                if (lr < rows) {
                    int acc = 0;
#pragma unroll
                    for (int w = 0; w < WAVES; ++w) acc += red[w][jj / kTileN][m][jj % kTileN];
                    const int r = row0 + lr;
                    const int col = nt * 2 * kTileN + jj;
                    float y = static_cast<float>(acc) * Ws[col];
                    y = y * a.a_scale[r];
                    const uint16_t zb = f32_to_bf16(y);
                    if (routed)
                        a.z[static_cast<size_t>(r) * a.H + col] = zb;
                    else
                        a.share_out[static_cast<size_t>(a.row_token[r]) * a.H + col] = zb;
                    if (a.dbg_acc) a.dbg_acc[static_cast<size_t>(r) * a.H + col] = acc;
                    if (a.dbg_z) a.dbg_z[static_cast<size_t>(r) * a.H + col] = zb;
                }
            }
        }
        __syncthreads();
    }
}

template <int KIND, int WAVES>
hipError_t launch_impl(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s) {
    const int steps = k_dim / (64 * WAVES);
    int ks = 16;
    while (ks > 1 && steps % ks) ks >>= 1;
    const int n_pass = steps / ks;
    const int grid = ((max_chunks + 7) / 8) * 8 * a.n_tiles;
    if (grid <= 0) return hipSuccess;
    const dim3 blk(WAVES * kWave);
    switch (ks) {
        case 16: hipLaunchKernelGGL((gemm_kernel<KIND, WAVES, 16>), dim3(grid), blk, 0, s, a, k_dim, n_pass); break;
        case 8: hipLaunchKernelGGL((gemm_kernel<KIND, WAVES, 8>), dim3(grid), blk, 0, s, a, k_dim, n_pass); break;
        case 4: hipLaunchKernelGGL((gemm_kernel<KIND, WAVES, 4>), dim3(grid), blk, 0, s, a, k_dim, n_pass); break;
        case 2: hipLaunchKernelGGL((gemm_kernel<KIND, WAVES, 2>), dim3(grid), blk, 0, s, a, k_dim, n_pass); break;
        default: hipLaunchKernelGGL((gemm_kernel<KIND, WAVES, 1>), dim3(grid), blk, 0, s, a, k_dim, n_pass); break;
    }
    return hipGetLastError();
}

}  // namespace

// k_dim must be a multiple of 256 (64-byte MFMA K step x 4 waves).
hipError_t launch_gemm1(const GemmArgs &a, int max_chunks, hipStream_t s) {
    return launch_impl<1, 4>(a, max_chunks, a.H, s);
}

hipError_t launch_gemm2(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s) {
    return launch_impl<2, 4>(a, max_chunks, k_dim, s);
}

}  // namespace moe
