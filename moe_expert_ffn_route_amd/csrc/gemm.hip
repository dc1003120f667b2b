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
// Work items of 16 rows: decode batches (at most 16 tokens, so at most 16
// rows per expert; larger batches go to gemm_wide.hip), and with group-wise
// activation scales any batch whose local experts average fewer than 16
// rows. That work is bound by the weight stream: each touched expert's bytes
// are read once, so the kernel is shaped around HBM, not around MFMA
// throughput:
//   - a work item is (chunk of <= 16 rows of one expert, 16-channel N tile
//     pair); its 2 x 16 weight rows are split over the waves along K; each
//     wave streams its K slice in batches of KSTEPS 64-byte steps, software
//     pipelined (the next batch's loads are issued before this batch's
//     MFMAs), with the whole loop unrolled so that the compiler's wait
//     counters stay exact;
//   - with packed weights (moe_w8a8_pack_weights) every wave load is one
//     contiguous 1 KB block, read non-temporally;
//   - the kernel takes MT row tiles per chunk as a parameter (each weight
//     batch feeds all of them, so a chunk reads its weights once); the
//     library instantiates MT = 1;
//   - the partial int32 tiles of the waves are summed in LDS (exact);
//   - blockIdx maps linearly to (chunk, N tile), so the round-robin placement
//     of blocks on the 8 XCDs gives each XCD an equal share of every expert;
//   - the epilogue's scales are fetched before the weight stream starts;
//   - with group-wise activation scales (GS > 0, "DeepSeek V4 Decode
//     Optimization" sec. 3.1) each group's int32 partials are dequantised in
//     the K loop and the epilogue sums fp32 values instead.
// MFMA operand layout: lane l holds 16 bytes of row (l % 16) at byte offset
// 16 * (l / 16) of a 64-byte K step, for A (token rows) and B (weight rows)
// alike, so every product pairs equal K indices. Result lane l, register i
// holds D[4 * (l / 16) + i][l % 16].
#include "internal.h"
#include "rowquant.h"

#include <hip/hip_ext.h>

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i ld16(const int8_t *p) { return *reinterpret_cast<const v4i *>(p); }
__device__ __forceinline__ v4i ld16_stream(const int8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
}

// Agent-coherent fp32 store / load (global_store / global_load with the
// agent-scope coherence bit): a value stored this way by a block on one XCD is
// read by a block on another XCD through these loads once the store has
// completed, without writing back or invalidating any XCD's L2.
__device__ __forceinline__ void store_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 load4_coherent(const float *p) {
    return make_float4(load_coherent(p), load_coherent(p + 1), load_coherent(p + 2), load_coherent(p + 3));
}

// Requantisation of one chunk's h rows by the last of its N-tile blocks to
// arrive ("FusedDeepMoE Kernel 深度分析报告" sec. 7.2 BlockQuant, with the eps
// floor of "DeepSeek V4 Decode Optimization" sec. 0): per row, a' = max(max
// |h|, eps), hs = a' * (1/127), q = rint((h * 127) * (1/a')), the fp32
// operations of the requant kernel in the same order. One wave per row (wave
// max, no barrier); rows of up to kFinRegs * 256 values stay in registers,
// longer rows are read twice.
constexpr int kFinRegs = 8;
template <int WAVES>
__device__ __forceinline__ void finalize_requant(const GemmArgs &a, int row0, int rows, int n, int wave, int lane) {
    const int P = a.meta[kMetaP];
    for (int lr = wave; lr < rows; lr += WAVES) {  // uniform per wave
        const int r = row0 + lr;
        const float *src = a.h + static_cast<size_t>(r) * a.imax;
        int8_t *dst = a.fin_q + static_cast<size_t>(r) * a.imax;
        float m = 0.0f;
        float ap, inv;
        if (n <= kFinRegs * kWave * 4) {
            // every load is issued (lanes past the row re-read its start), so
            // the loads of the whole row are in flight together
            float4 v[kFinRegs];
#pragma unroll
            for (int j = 0; j < kFinRegs; ++j) {
                const int i = (lane + j * kWave) * 4;
                v[j] = load4_coherent(src + (i < n ? i : 0));
            }
#pragma unroll
            for (int j = 0; j < kFinRegs; ++j) {
                const int i = (lane + j * kWave) * 4;
                if (i < n) m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
            }
            ap = fmaxf(wave_max(m), a.fin_eps);
            inv = 1.0f / ap;
#pragma unroll
            for (int j = 0; j < kFinRegs; ++j) {
                const int i = (lane + j * kWave) * 4;
                if (i < n) *reinterpret_cast<uint32_t *>(dst + i) = quant4<false>(v[j].x, v[j].y, v[j].z, v[j].w, inv);
            }
        } else {
            for (int i = lane * 4; i < n; i += kWave * 4) {
                const float4 v = load4_coherent(src + i);
                m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            }
            ap = fmaxf(wave_max(m), a.fin_eps);
            inv = 1.0f / ap;
            for (int i = lane * 4; i < n; i += kWave * 4) {
                const float4 v = load4_coherent(src + i);
                *reinterpret_cast<uint32_t *>(dst + i) = quant4<false>(v.x, v.y, v.z, v.w, inv);
            }
        }
        if (lane == 0) {
            const float hs = ap * (1.0f / kQMax<false>);
            a.fin_scale[r] = hs;
            if (a.fin_scale2) a.fin_scale2[r] = r < P ? hs * a.fin_route_w[a.fin_sorted_pair[r]] : hs;
        }
    }
}

// KIND 1 = GEMM1 + SwiGLU, 2 = GEMM2 + bf16. MT = 16-row MFMA tiles per
// chunk. NPASS = K batches per wave (0: taken from n_pass_rt at run time).
// GS > 0: group-wise activation scales ("DeepSeek V4 Decode Optimization"
// sec. 3.1), one per GS 64-byte K steps of a row (a.a_ng per row): at the end
// of each group the lane's int32 partials are dequantised,
// p = (float(acc) * w_scale[n]) * group_scale[row], and added to its fp32
// sums, which the epilogue adds over the waves in wave order (a wave's K
// slice and each batch hold whole groups).
template <int KIND, int WAVES, int KSTEPS, bool PACKED, int MT, int NPASS, int GS = 0>
__global__ __launch_bounds__(WAVES * kWave) void gemm_kernel(GemmArgs a, int k_dim, int n_pass_rt) {
    static_assert(GS == 0 || KSTEPS % GS == 0, "group-wise scales: whole groups per batch");
    constexpr int kThreads = WAVES * kWave;
    constexpr int kCols = KIND == 1 ? kTileN : 2 * kTileN;  // output columns of one work item
    constexpr int kElems = kTileN * kCols;                   // outputs of one 16-row tile
    constexpr int kEpt = (kElems + kThreads - 1) / kThreads; // outputs per thread per tile
    const int n_pass = NPASS > 0 ? NPASS : n_pass_rt;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    // Work item = (chunk, N tile), linear in blockIdx: the hardware deals
    // consecutive blocks round-robin to the 8 XCDs, so every XCD streams an
    // equal share of every expert's weights.
    int c = blockIdx.x / a.n_tiles;
    int nt = blockIdx.x % a.n_tiles;
    int4 ch = a.chunks[c];  // c < max_chunks: inside the chunk list even when unused
    if (c >= a.meta[a.count_word]) return;
    const int nch = ch.z >> kChunkCountShift;
    if (nch > 1 && (a.n_tiles & 7) == 0) {
        // A group of several chunks owns blocks [c0 * n_tiles, (c0 + nch) *
        // n_tiles). Within that range the nch chunks of one N tile are put 8
        // blocks apart: on the same XCD and in flight together, so the tile's
        // weights come from HBM once and are shared through that XCD's L2.
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

    // Issue order matters: vmcnt retires loads in issue order, so a wait for
    // a small load issued after the weight stream would also wait for the
    // weights. Independent small loads go first, then the first weight
    // batch, then the loads that depend on the small ones, then the
    // software-pipelined K loop. Scheduling barriers keep the compiler from
    // reordering the phases.

    // (1) independent small loads: token of each A row, epilogue rows' tokens
    //     and the output channels' weight scales.
    // GEMM1 row r reads its activations through an index (routed rows: the
    // token's or the (token, expert) pair's quantised row; shared rows: the
    // token's); GEMM2 row r reads row r. Lanes past the chunk's last row read
    // that last row and are zeroed before the MFMA, so no load sits in a
    // divergent branch.
    const int32_t *aidx = KIND == 1 ? (routed ? a.idx_r : a.row_token) : nullptr;
    // epilogue rows' index: GEMM1 the activation scale's row, GEMM2 the z row
    // (the pair id) of a routed row or the share_output row of a shared one
    const int32_t *tidx = KIND == 1 ? aidx : (routed ? a.zrow : a.row_token);
    const int8_t *Abase = KIND == 1 ? (routed ? a.A_r : a.A_s) : a.A;
    const float *Ascale = KIND == 1 ? (routed ? a.a_scale_r : a.a_scale_s) : a.a_scale;
    int arow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int lr = min(mt * kTileN + r16, rows - 1);
        arow[mt] = KIND == 1 ? aidx[row0 + lr] : row0 + lr;
    }
    // A thread's output column is the same in every row tile (kThreads is a
    // multiple of kCols).
    const int jc = tid % kCols;
    const int col = (KIND == 1 ? nt * kTileN : nt * 2 * kTileN) + jc;
    const float wsc0 = Ws[col];
    const float wsc1 = KIND == 1 ? Ws[inter + col] : 0.0f;
    // group-wise scales: the lane's two output channels (one per weight tile)
    // and the activation rows of its four accumulator rows 4 * (l / 16) + i
    float wl0 = 0.0f, wl1 = 0.0f;
    int srow[MT][4];
    if constexpr (GS > 0) {
        wl0 = Ws[rowA + r16];
        wl1 = Ws[rowB + r16];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int lr = min(mt * kTileN + 4 * kg + i, rows - 1);
                srow[mt][i] = KIND == 1 ? aidx[row0 + lr] : row0 + lr;
            }
    }
    int rrow[kEpt], rtok[kEpt];  // epilogue rows of the first row tile
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
        rrow[e] = row0 + min(min(tid + e * kThreads, kElems - 1) / kCols, rows - 1);
        rtok[e] = tidx[rrow[e]];
    }
    __builtin_amdgcn_sched_barrier(0);

    // (2) first weight batch.
    // Row-major weights: lane reads 16 bytes of row (tile row + l%16) at byte
    // 64*step + 16*(l/16). Packed weights (moe_w8a8_pack_weights) hold exactly
    // those bytes as one contiguous 1 KB block per (16-row tile, step), so a
    // wave's load is 1 KB contiguous and consecutive steps are adjacent;
    // those are read non-temporally, 64-byte row segments with plain loads.
    const int8_t *pw0, *pw1;
    size_t wstep;
    if (PACKED) {
        const size_t steps_k = Kd / 64;
        const size_t ta = KIND == 1 ? g1_tile_pos(rowA / kTileN, inter / kTileN) : rowA / kTileN;
        const size_t tb = KIND == 1 ? g1_tile_pos(rowB / kTileN, inter / kTileN) : rowB / kTileN;
        pw0 = W + (ta * steps_k + step0) * 1024 + lane * 16;
        pw1 = W + (tb * steps_k + step0) * 1024 + lane * 16;
        wstep = 1024;
    } else {
        pw0 = W + static_cast<size_t>(rowA + r16) * Kd + step0 * 64 + kg * 16;
        pw1 = W + static_cast<size_t>(rowB + r16) * Kd + step0 * 64 + kg * 16;
        wstep = 64;
    }
    v4i wbuf[2][2][KSTEPS];
    auto ldw = [&](v4i (&w)[2][KSTEPS], int pass) {
        const size_t sp = static_cast<size_t>(pass) * KSTEPS;
#pragma unroll
        for (int i = 0; i < KSTEPS; ++i) {
            if (PACKED) {
                w[0][i] = ld16_stream(pw0 + (sp + i) * wstep);
                w[1][i] = ld16_stream(pw1 + (sp + i) * wstep);
            } else {
                w[0][i] = ld16(pw0 + (sp + i) * wstep);
                w[1][i] = ld16(pw1 + (sp + i) * wstep);
            }
        }
    };
    ldw(wbuf[0], 0);
    __builtin_amdgcn_sched_barrier(0);

    // (3) loads that depend on (1): the first row tile's row scales (none
    //     with group-wise scales, which the K loop applies)
    float rsc[kEpt];
#pragma unroll
    for (int e = 0; e < kEpt; ++e) rsc[e] = GS > 0 ? 0.0f : Ascale[KIND == 1 ? rtok[e] : rrow[e]];
    __builtin_amdgcn_sched_barrier(0);

    v4i acc0[MT], acc1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        acc0[mt] = v4i{0, 0, 0, 0};
        acc1[mt] = v4i{0, 0, 0, 0};
    }
    float f0[MT][4], f1[MT][4];  // group-wise sums
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f0[mt][e] = 0.0f;
            f1[mt][e] = 0.0f;
        }
    // One K batch: this batch's A rows, then (if any) the next weight batch,
    // then the MFMAs, which wait only for this batch's loads.
    auto batch = [&](const v4i (&w)[2][KSTEPS], v4i (&nxt)[2][KSTEPS], int pass, bool has_next) {
        v4i x[MT][KSTEPS];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (MT == 1 || mt * kTileN < rows) {  // uniform
                const int8_t *pam =
                    Abase + static_cast<size_t>(arow[mt]) * a.a_stride + (step0 + pass * KSTEPS) * 64 + kg * 16;
#pragma unroll
                for (int i = 0; i < KSTEPS; ++i) x[mt][i] = ld16(pam + i * 64);
            }
        }
        // group-wise scales of this batch's groups, for the lane's four rows
        // of each row tile
        constexpr int kGroups = GS > 0 ? KSTEPS / GS : 1;
        float gsc[MT][kGroups][4];
        if constexpr (GS > 0) {
            const int g0 = (step0 + pass * KSTEPS) / GS;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (!(MT == 1 || mt * kTileN < rows)) continue;  // uniform
                if (kGroups % 4 == 0 && (a.a_ng & 3) == 0) {     // uniform
                    // a row's scales of consecutive groups are contiguous and,
                    // with g0 a multiple of kGroups and a_ng of 4, 16-byte aligned
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int q = 0; q + 3 < kGroups; q += 4) {
                            const float4 v4 = *reinterpret_cast<const float4 *>(
                                Ascale + static_cast<size_t>(srow[mt][i]) * a.a_ng + g0 + q);
                            gsc[mt][q][i] = v4.x;
                            gsc[mt][q + 1][i] = v4.y;
                            gsc[mt][q + 2][i] = v4.z;
                            gsc[mt][q + 3][i] = v4.w;
                        }
                } else {
#pragma unroll
                    for (int q = 0; q < kGroups; ++q)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            gsc[mt][q][i] = Ascale[static_cast<size_t>(srow[mt][i]) * a.a_ng + g0 + q];
                }
            }
        }
        if (has_next) ldw(nxt, pass + 1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (GS > 0) {
            // Each group's first MFMA starts from zero; a finished group's
            // partials are dequantised only after the next group's first
            // MFMAs are issued, so the VALU work never waits right behind the
            // MFMA that produced its operands (the batch's last group waits
            // once, at the end).
            const v4i zero = {0, 0, 0, 0};
            v4i pend0[MT], pend1[MT];
            auto flush = [&](int mt, int q) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float p0 = static_cast<float>(pend0[mt][e]) * wl0;
                    p0 = p0 * gsc[mt][q][e];
                    f0[mt][e] = f0[mt][e] + p0;
                    float p1 = static_cast<float>(pend1[mt][e]) * wl1;
                    p1 = p1 * gsc[mt][q][e];
                    f1[mt][e] = f1[mt][e] + p1;
                }
            };
#pragma unroll
            for (int i = 0; i < KSTEPS; ++i) {
                const bool first = i % GS == 0;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (MT == 1 || mt * kTileN < rows) {  // uniform
                        const v4i xi = mt * kTileN + r16 < rows ? x[mt][i] : zero;
                        acc0[mt] =
                            __builtin_amdgcn_mfma_i32_16x16x64_i8(xi, w[0][i], first ? zero : acc0[mt], 0, 0, 0);
                        acc1[mt] =
                            __builtin_amdgcn_mfma_i32_16x16x64_i8(xi, w[1][i], first ? zero : acc1[mt], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (MT == 1 || mt * kTileN < rows) {
                        if (first && i > 0) flush(mt, i / GS - 1);
                        if ((i + 1) % GS == 0) {
                            pend0[mt] = acc0[mt];
                            pend1[mt] = acc1[mt];
                        }
                    }
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                if (MT == 1 || mt * kTileN < rows) flush(mt, kGroups - 1);
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (MT == 1 || mt * kTileN < rows) {
                    const bool av = mt * kTileN + r16 < rows;
#pragma unroll
                    for (int i = 0; i < KSTEPS; ++i) {
                        const v4i xi = av ? x[mt][i] : v4i{0, 0, 0, 0};
                        acc0[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xi, w[0][i], acc0[mt], 0, 0, 0);
                        acc1[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xi, w[1][i], acc1[mt], 0, 0, 0);
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (NPASS > 0) {
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) batch(wbuf[pass & 1], wbuf[(pass + 1) & 1], pass, pass + 1 < NPASS);
    } else {
        for (int pass = 0; pass < n_pass; pass += 2) {
            batch(wbuf[0], wbuf[1], pass, pass + 1 < n_pass);
            if (pass + 1 < n_pass) batch(wbuf[1], wbuf[0], pass + 1, pass + 2 < n_pass);
        }
    }

    if constexpr (GS > 0) {
        // the waves' fp32 sums, added in wave order, one row tile at a time
        __shared__ float redf[WAVES][2][kTileN][kTileN];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
        if (mt * kTileN >= rows) break;  // uniform
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            redf[wave][0][4 * kg + i][r16] = f0[mt][i];
            redf[wave][1][4 * kg + i][r16] = f1[mt][i];
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kEpt; ++e) {
            const int idx = tid + e * kThreads;
            const int m = idx / kCols;
            const int lr = mt * kTileN + m;
            if (idx < kElems && lr < rows) {
                const int r = row0 + lr;
                if (KIND == 1) {
                    float yg = 0.0f, yu = 0.0f;
#pragma unroll
                    for (int w = 0; w < WAVES; ++w) {
                        yg = yg + redf[w][0][m][jc];
                        yu = yu + redf[w][1][m][jc];
                    }
                    a.h[static_cast<size_t>(r) * a.imax + col] = swiglu_y(yg, yu);
                    if (a.dbg_acc) {
                        a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + col] = __float_as_int(yg);
                        a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + inter + col] = __float_as_int(yu);
                    }
                } else {
                    float y = 0.0f;
#pragma unroll
                    for (int w = 0; w < WAVES; ++w) y = y + redf[w][jc / kTileN][m][jc % kTileN];
                    const uint16_t zb = f32_to_bf16(y);
                    const int t = mt == 0 ? rtok[e] : tidx[r];
                    (routed ? a.z : a.share_out)[static_cast<size_t>(t) * a.H + col] = zb;
                    if (a.dbg_acc) a.dbg_acc[static_cast<size_t>(r) * a.H + col] = __float_as_int(y);
                    if (a.dbg_z) a.dbg_z[static_cast<size_t>(r) * a.H + col] = zb;
                }
            }
        }
        __syncthreads();
        }
        return;
    }
    __shared__ int red[WAVES][2][kTileN][kTileN];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
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
                const float rs = mt == 0 ? rsc[e] : Ascale[KIND == 1 ? aidx[r] : r];
                if (KIND == 1) {
                    int ag = 0, au = 0;
#pragma unroll
                    for (int w = 0; w < WAVES; ++w) {
                        ag += red[w][0][m][jc];
                        au += red[w][1][m][jc];
                    }
                    const float hv = swiglu(ag, au, wsc0, wsc1, rs);
                    if (a.fin_count) store_coherent(a.h + static_cast<size_t>(r) * a.imax + col, hv);
                    else a.h[static_cast<size_t>(r) * a.imax + col] = hv;
                    if (a.dbg_acc) {
                        a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + col] = ag;
                        a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + inter + col] = au;
                    }
                } else {
                    int acc = 0;
#pragma unroll
                    for (int w = 0; w < WAVES; ++w) acc += red[w][jc / kTileN][m][jc % kTileN];
                    const uint16_t zb = f32_to_bf16(dequant(acc, wsc0, rs));
                    const int t = mt == 0 ? rtok[e] : tidx[r];
                    (routed ? a.z : a.share_out)[static_cast<size_t>(t) * a.H + col] = zb;
                    if (a.dbg_acc) a.dbg_acc[static_cast<size_t>(r) * a.H + col] = acc;
                    if (a.dbg_z) a.dbg_z[static_cast<size_t>(r) * a.H + col] = zb;
                }
            }
        }
        __syncthreads();
    }
    if (KIND == 1 && a.fin_count) {
        // Arrival count of this chunk: every thread waits until its h stores
        // (agent-coherent) have completed, the barrier gathers the block, and
        // one thread counts the block in. The block that brings the count to
        // the chunk's number of N tiles is the last: every other block's h
        // values are then visible to its coherent loads, and it quantises the
        // chunk's rows. Nothing waits on another block.
        __shared__ int s_last;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(a.fin_count + c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     inter / kTileN - 1;
        __syncthreads();
        if (s_last) finalize_requant<WAVES>(a, row0, rows, inter, wave, lane);
    }
}

// Tuning (measured on MI355X for the decode shapes): waves per workgroup and
// the number of 64-byte K steps a wave loads per batch (fewer steps per batch
// = fewer VGPRs = more resident waves streaming).
#ifndef MOE_GEMM1_WAVES
#define MOE_GEMM1_WAVES 8
#endif
#ifndef MOE_GEMM1_KSTEPS
#define MOE_GEMM1_KSTEPS 8
#endif
#ifndef MOE_GEMM2_WAVES
#define MOE_GEMM2_WAVES 8
#endif
#ifndef MOE_GEMM2_KSTEPS
#define MOE_GEMM2_KSTEPS 4
#endif
template <int KIND, int WAVES, int KSTEPS, bool PACKED, int MT, int NPASS, int GS = 0>
void launch_one(const GemmArgs &a, dim3 grid, int k_dim, int n_pass, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const dim3 blk(WAVES * kWave);
    if (e0 || e1)
        hipExtLaunchKernelGGL((gemm_kernel<KIND, WAVES, KSTEPS, PACKED, MT, NPASS, GS>), grid, blk, 0, s, e0, e1, 0,
                              a, k_dim, n_pass);
    else
        hipLaunchKernelGGL((gemm_kernel<KIND, WAVES, KSTEPS, PACKED, MT, NPASS, GS>), grid, blk, 0, s, a, k_dim,
                           n_pass);
}

template <int KIND, int WAVES, int KSTEPS, bool PACKED, int MT>
hipError_t launch_np(const GemmArgs &a, dim3 grid, int k_dim, int n_pass, hipStream_t s, hipEvent_t e0,
                     hipEvent_t e1) {
    switch (n_pass) {
        case 1: launch_one<KIND, WAVES, KSTEPS, PACKED, MT, 1>(a, grid, k_dim, 1, s, e0, e1); break;
        case 2: launch_one<KIND, WAVES, KSTEPS, PACKED, MT, 2>(a, grid, k_dim, 2, s, e0, e1); break;
        case 4: launch_one<KIND, WAVES, KSTEPS, PACKED, MT, 4>(a, grid, k_dim, 4, s, e0, e1); break;
        case 8: launch_one<KIND, WAVES, KSTEPS, PACKED, MT, 8>(a, grid, k_dim, 8, s, e0, e1); break;
        default: launch_one<KIND, WAVES, KSTEPS, PACKED, MT, 0>(a, grid, k_dim, n_pass, s, e0, e1); break;
    }
    return hipGetLastError();
}

// k_dim is a multiple of 256 (64-byte MFMA K step x 4 waves). A wave walks
// k_dim / (64 * waves) steps in batches of KS steps, or of 1 step when KS does
// not divide them. Work items here are single 16-row tiles (decode batches);
// chunks of several tiles go to gemm_wide.hip.
template <int KIND, int WAVES, int KS>
hipError_t launch_w(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (a.mt != 1) return hipErrorInvalidValue;
    const long blocks = static_cast<long>(max_chunks) * a.n_tiles;
    if (blocks <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(blocks));
    const int steps = k_dim / (64 * WAVES);
    if (steps % KS == 0)
        return a.packed ? launch_np<KIND, WAVES, KS, true, 1>(a, grid, k_dim, steps / KS, s, e0, e1)
                        : launch_np<KIND, WAVES, KS, false, 1>(a, grid, k_dim, steps / KS, s, e0, e1);
    return a.packed ? launch_np<KIND, WAVES, 1, true, 1>(a, grid, k_dim, steps, s, e0, e1)
                    : launch_np<KIND, WAVES, 1, false, 1>(a, grid, k_dim, steps, s, e0, e1);
}

// Group-wise scales (a.gsteps = GS steps of 64 per group): every wave's K
// slice must hold whole groups, so K is split over W = min(8, groups) waves
// (groups = k_dim / (64 * GS), a power-of-two count is not required: W is the
// largest of 8, 4, 2, 1 dividing it). A slice of up to 8 steps is one batch,
// longer slices go in batches of one group. (Chunks of two row tiles take
// the wide kernel of gemm_wide.hip instead.)
template <int KIND, bool PACKED, int GS, int W>
hipError_t launch_grp_w(const GemmArgs &a, dim3 grid, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const int spw = k_dim / (64 * W);
    switch (spw) {
        case GS: launch_one<KIND, W, GS, PACKED, 1, 1, GS>(a, grid, k_dim, 1, s, e0, e1); break;
        case 2 * GS: launch_one<KIND, W, 2 * GS, PACKED, 1, 1, GS>(a, grid, k_dim, 1, s, e0, e1); break;
        case 4 * GS:
            if constexpr (GS <= 2) launch_one<KIND, W, 4 * GS, PACKED, 1, 1, GS>(a, grid, k_dim, 1, s, e0, e1);
            else launch_one<KIND, W, GS, PACKED, 1, 0, GS>(a, grid, k_dim, 4, s, e0, e1);
            break;
        case 8 * GS:  // 64-element groups: two batches of 4, which keeps 4 waves per SIMD
            if constexpr (GS == 1) launch_one<KIND, W, 4, PACKED, 1, 2, GS>(a, grid, k_dim, 2, s, e0, e1);
            else launch_one<KIND, W, GS, PACKED, 1, 0, GS>(a, grid, k_dim, 8, s, e0, e1);
            break;
        default: launch_one<KIND, W, GS, PACKED, 1, 0, GS>(a, grid, k_dim, spw / GS, s, e0, e1); break;
    }
    return hipGetLastError();
}

template <int KIND, bool PACKED, int GS>
hipError_t launch_grp(const GemmArgs &a, dim3 grid, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const int groups = k_dim / (64 * GS);
    if (groups % 8 == 0) return launch_grp_w<KIND, PACKED, GS, 8>(a, grid, k_dim, s, e0, e1);
    if (groups % 4 == 0) return launch_grp_w<KIND, PACKED, GS, 4>(a, grid, k_dim, s, e0, e1);
    if (groups % 2 == 0) return launch_grp_w<KIND, PACKED, GS, 2>(a, grid, k_dim, s, e0, e1);
    return launch_grp_w<KIND, PACKED, GS, 1>(a, grid, k_dim, s, e0, e1);
}

template <int KIND, bool PACKED>
hipError_t launch_grp_p(const GemmArgs &a, dim3 grid, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    switch (a.gsteps) {
        case 1: return launch_grp<KIND, PACKED, 1>(a, grid, k_dim, s, e0, e1);
        case 2: return launch_grp<KIND, PACKED, 2>(a, grid, k_dim, s, e0, e1);
        case 4: return launch_grp<KIND, PACKED, 4>(a, grid, k_dim, s, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

template <int KIND>
hipError_t launch_kind(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (a.gsteps > 0) {
        if (a.mt != 1 || k_dim % (64 * a.gsteps)) return hipErrorInvalidValue;
        const long blocks = static_cast<long>(max_chunks) * a.n_tiles;
        if (blocks <= 0) return hipSuccess;
        const dim3 grid(static_cast<unsigned>(blocks));
        return a.packed ? launch_grp_p<KIND, true>(a, grid, k_dim, s, e0, e1)
                        : launch_grp_p<KIND, false>(a, grid, k_dim, s, e0, e1);
    }
    constexpr int W = KIND == 1 ? MOE_GEMM1_WAVES : MOE_GEMM2_WAVES;
    constexpr int KS = KIND == 1 ? MOE_GEMM1_KSTEPS : MOE_GEMM2_KSTEPS;
    if constexpr (W == 8) {
        if (k_dim % 512 == 0) return launch_w<KIND, 8, KS>(a, max_chunks, k_dim, s, e0, e1);
    }
    return launch_w<KIND, 4, KS>(a, max_chunks, k_dim, s, e0, e1);
}

}  // namespace
hipError_t launch_gemm1(const GemmArgs &a, int max_chunks, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
    return launch_kind<1>(a, max_chunks, a.H, s, ev_start, ev_stop);
}

hipError_t launch_gemm2(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t ev_start,
                        hipEvent_t ev_stop) {
    return launch_kind<2>(a, max_chunks, k_dim, s, ev_start, ev_stop);
}

}  // namespace moe
