// Grouped INT8 GEMMs for experts of hundreds of rows (tall work items), with
// the fused epilogues of the other GEMM kernels:
//   GEMM1 ("FusedDeepMoE Kernel 深度分析报告" sec. 3.3 / 6.1): gate and up
//     accumulators of one row and channel meet in one lane, which applies
//     y = (float(acc) * w1s[n]) * xs[r] to both and writes
//     h = (y_g / (1 + exp(-y_g))) * y_u as fp32;
//   GEMM2 (sec. 3.4 / 6.2): z = bf16((float(acc) * w2s[n]) * hs[r]), to the
//     routed row buffer or, for the shared expert, straight to share_output.
//
// When an expert holds hundreds of rows its weights are re-read by every
// chunk of rows, and the GEMM can be fed from on-chip memory at the MFMA
// rate. A work item is a 256-row chunk times 8 pairs of 16-row weight tiles
// (GEMM1: 128 gate tiles' channels with their up tiles; GEMM2: 256 output
// channels). Its 16 waves form a 4 x 4 grid: wave (wm, wn) multiplies rows
// [64 wm, 64 wm + 64) by the 2 tile pairs [2 wn, 2 wn + 2), so it holds
// 4 x 4 MFMA tiles of int32 sums and four waves share a SIMD. Both operands
// go through LDS one 64-byte K step (a stage, 32 KB) at a time, in four
// buffers filled by direct global-to-LDS copies three stages ahead (no
// staging registers), with one workgroup barrier per stage. Every activation
// fragment read from LDS feeds 4 MFMAs and every weight fragment 4.
//
// LDS stage layout, all in MFMA lane order (1 KB blocks, lane l at byte
// 16 l: row l % 16, bytes 16 (l / 16) .. +16 of the K step): the chunk's 16
// activation row tiles, then the block's 16 weight tiles as (pair, half)
// blocks. Lane-ordered reads and writes are free of bank conflicts.
#include "internal.h"

#include <hip/hip_ext.h>

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// Tuning: waves per workgroup, waves along N, tile pairs per wave (the rest
// follows; the chunk is always 256 rows by 8 tile pairs).
#ifndef MOE_TBIG_WAVES
#define MOE_TBIG_WAVES 16
#endif
#ifndef MOE_TBIG_WN
#define MOE_TBIG_WN 4
#endif
#ifndef MOE_TBIG_Q
#define MOE_TBIG_Q 2
#endif
#ifndef MOE_TALL_XCD
#define MOE_TALL_XCD 1
#endif
constexpr int kTWaves = MOE_TBIG_WAVES;             // a grid of kTWM (rows) x kTWN (weight tiles)
constexpr int kTThreads = kTWaves * kWave;
constexpr int kTWN = MOE_TBIG_WN;
constexpr int kTWM = kTWaves / kTWN;
constexpr int kTMT = kChunkRowsTall / kTileN / kTWM;  // 16-row tiles per wave
constexpr int kTQ = MOE_TBIG_Q;                     // tile pairs per wave
constexpr int kTPairs = kTWN * kTQ;                 // tile pairs per block
constexpr int kTSteps = 1;                          // 64-byte K steps per stage
constexpr int kTRowTiles = kChunkRowsTall / kTileN;
constexpr int kTAStage = kTRowTiles * kTSteps * 1024;
constexpr int kTWStage = 2 * kTPairs * kTSteps * 1024;
constexpr int kTStage = kTAStage + kTWStage;
constexpr int kTLoadsA = kTAStage / 1024 / kTWaves;  // 1 KB activation blocks per wave and stage
constexpr int kTLoadsW = kTWStage / 1024 / kTWaves;  // 1 KB weight blocks per wave and stage
static_assert(kTRowTiles == kTWM * kTMT, "a chunk is kTWM waves' rows");
static_assert(kTPairs == kTallPairs, "the host sizes the grid with kTallPairs");
static_assert(kTAStage == kTLoadsA * kTWaves * 1024 && kTWStage == kTLoadsW * kTWaves * 1024,
              "a stage is whole 1 KB blocks per wave");

template <int KIND, bool PACKED>
__global__ __launch_bounds__(kTThreads, 1) void gemm_tall_kernel(GemmArgs a, int k_dim) {
    __shared__ __attribute__((aligned(16))) int8_t s_d0[kTStage];
    __shared__ __attribute__((aligned(16))) int8_t s_d1[kTStage];
    __shared__ __attribute__((aligned(16))) int8_t s_d2[kTStage];
    __shared__ __attribute__((aligned(16))) int8_t s_d3[kTStage];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave % kTWM, wn = wave / kTWM;
    const int r16 = lane & 15, kg = lane >> 4;

    // Work item = (chunk, group of 8 tile pairs), chunk-major; within a group
    // of several chunks the items are ordered by 8 N groups, then chunk, so
    // the chunks of one N group are 8 items apart and in flight together.
    const int n_chunks = a.meta[a.count_word];
    int b = blockIdx.x;
#if MOE_TALL_XCD
    // XCD-aware order: the dispatcher hands block b to XCD b % 8, so the first
    // n8 = (items & ~7) blocks are renumbered to give XCD x the consecutive
    // items [x n8 / 8, (x + 1) n8 / 8): an expert's chunks and all their N
    // groups run on one XCD, whose L2 then serves both the weight tiles (read
    // by every chunk) and the activation chunks (read by every N group).
    const int n8 = (n_chunks * a.n_tiles) & ~7;
    if (b < n8) b = (b & 7) * (n8 >> 3) + (b >> 3);
#endif
    int c = b / a.n_tiles;
    int nt = b % a.n_tiles;
    if (c >= n_chunks) return;
    int4 ch = a.chunks[c];
    const int nch = ch.z >> kChunkCountShift;
    if (nch > 1 && (a.n_tiles & 7) == 0) {
        const int c0 = c - ch.w;
        const int i = b - c0 * a.n_tiles;
        const int q = i / (8 * nch), rem = i - q * 8 * nch;
        c = c0 + rem / 8;
        nt = q * 8 + rem % 8;
        ch = a.chunks[c];
    }
    const int g = ch.x, row0 = ch.y, rows = ch.z & kChunkRowsMask;
    if (g < a.g_lo || g >= a.g_hi) return;
    const bool routed = g < a.E_loc;
    const int inter = routed ? a.I : a.I_s;
    if (KIND == 1 && nt * kTPairs * kTileN >= inter) return;  // inter is a multiple of 256: all or nothing

    const size_t tile_bytes = static_cast<size_t>(kTileN) * k_dim;
    const int8_t *W;
    const float *Ws;
    if (KIND == 1) {
        W = routed ? a.W + static_cast<size_t>(g) * 2 * inter * a.H : a.W_sh;
        Ws = routed ? a.Ws + static_cast<size_t>(g) * 2 * inter : a.Ws_sh;
    } else {
        W = routed ? a.W + static_cast<size_t>(g) * a.H * inter : a.W_sh;
        Ws = routed ? a.Ws + static_cast<size_t>(g) * a.H : a.Ws_sh;
    }
    // first weight row (= output channel) of each tile of the block's pair q
    auto row_a = [&](int q) { return KIND == 1 ? (nt * kTPairs + q) * kTileN : nt * 2 * kTPairs * kTileN + q * 32; };
    auto row_b = [&](int q) { return KIND == 1 ? inter + row_a(q) : row_a(q) + kTileN; };

    // Global -> LDS copy of a stage: thread t copies the 16 bytes of lane
    // t % 64 of 1 KB block j = kTWaves i + wave (i < kTLoadsA, kTLoadsW) of
    // each operand (a copy instruction puts lane l's 16 bytes at byte 16 l of
    // the wave's block).
    // Activation block j is row tile j / kTSteps, K step j % kTSteps: lane l
    // reads row 16 (j / kTSteps) + l % 16 (rows past the chunk repeat its last
    // row; their outputs are never stored). Weight block j is tile pair
    // j / (2 kTSteps), half (j / kTSteps) % 2, K step j % kTSteps: 1 KB
    // contiguous in the packed layout.
    const int wstep = PACKED ? 1024 : 64;  // bytes between K steps of a tile
    const int wlane = PACKED ? lane * 16 : r16 * k_dim + kg * 16;
    const int8_t *wsrc[kTLoadsW];
    const int8_t *asrc[kTLoadsA];
    const int32_t *aidx = KIND == 1 ? (routed ? a.idx_r : a.row_token) : nullptr;
    const int8_t *Abase = KIND == 1 ? (routed ? a.A_r : a.A_s) : a.A;
    const float *Ascale = KIND == 1 ? (routed ? a.a_scale_r : a.a_scale_s) : a.a_scale;
#pragma unroll
    for (int i = 0; i < kTLoadsW; ++i) {
        const int j = i * kTWaves + wave;
        const int wrow = ((j / kTSteps) & 1) ? row_b(j / (2 * kTSteps)) : row_a(j / (2 * kTSteps));
        const size_t wt = KIND == 1 && PACKED ? g1_tile_pos(wrow / kTileN, inter / kTileN) : wrow / kTileN;
        wsrc[i] = W + wt * tile_bytes + (j % kTSteps) * wstep + wlane;
    }
#pragma unroll
    for (int i = 0; i < kTLoadsA; ++i) {
        const int j = i * kTWaves + wave;
        const int lr = min((j / kTSteps) * kTileN + r16, rows - 1);
        const int ar = KIND == 1 ? aidx[row0 + lr] : row0 + lr;
        asrc[i] = Abase + static_cast<size_t>(ar) * a.a_stride + (j % kTSteps) * 64 + kg * 16;
    }
    v4i acc0[kTMT][kTQ], acc1[kTMT][kTQ];
#pragma unroll
    for (int mt = 0; mt < kTMT; ++mt)
#pragma unroll
        for (int q = 0; q < kTQ; ++q) {
            acc0[mt][q] = v4i{0, 0, 0, 0};
            acc1[mt][q] = v4i{0, 0, 0, 0};
        }
    // the MFMAs of one stage, from the LDS buffer that holds it
    auto compute = [&](const int8_t *cur) {
#pragma unroll
        for (int st = 0; st < kTSteps; ++st) {
            v4i b0[kTQ], b1[kTQ], x[kTMT];
#pragma unroll
            for (int q = 0; q < kTQ; ++q) {
                const int pq = wn * kTQ + q;
                b0[q] = *reinterpret_cast<const v4i *>(cur + kTAStage + ((pq * 2 + 0) * kTSteps + st) * 1024 + lane * 16);
                b1[q] = *reinterpret_cast<const v4i *>(cur + kTAStage + ((pq * 2 + 1) * kTSteps + st) * 1024 + lane * 16);
            }
#pragma unroll
            for (int mt = 0; mt < kTMT; ++mt)
                x[mt] = *reinterpret_cast<const v4i *>(cur + ((wm * kTMT + mt) * kTSteps + st) * 1024 + lane * 16);
#pragma unroll
            for (int mt = 0; mt < kTMT; ++mt)
#pragma unroll
                for (int q = 0; q < kTQ; ++q) {
                    acc0[mt][q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x[mt], b0[q], acc0[mt][q], 0, 0, 0);
                    acc1[mt][q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x[mt], b1[q], acc1[mt][q], 0, 0, 0);
                }
        }
    };
    const int n_stages = k_dim / (kTSteps * 64);  // a multiple of 4: k_dim is a multiple of 256
    // Four LDS buffers, stage t in buffer t % 4, filled by direct
    // global-to-LDS copies (lane l's 16 bytes land at byte 16 l of the 1 KB
    // block, the MFMA lane order) three stages ahead: at stage s a thread
    // issues its copies of stage s + 3 into the buffer stage s - 1 used
    // (every wave finished reading it before the last barrier), runs stage
    // s's MFMAs, waits until its copies of stage s + 1 have landed (the
    // copies of stages s + 2 and s + 3 may still be in flight) and passes a
    // barrier. Copies past the last stage reload it into a free buffer; all
    // copies have landed before the waves leave.
    typedef __attribute__((address_space(3))) void lds_void;
    typedef __attribute__((address_space(1))) void glb_void;
    static_assert(kTSteps == 1, "one K step per stage");
    // s_waitcnt immediate: vmcnt(n) (bits 3:0 and 15:14), expcnt 7 (no wait,
    // bits 6:4), lgkmcnt(0) (bits 11:8)
    constexpr int kCopies = kTLoadsA + kTLoadsW;  // per thread and stage
    static_assert(2 * kCopies <= 63, "vmcnt range");
    constexpr int kWaitNext = (2 * kCopies & 15) | ((2 * kCopies >> 4) << 14) | (7 << 4);
    auto dma = [&](int s, int8_t *buf) {
#pragma unroll
        for (int i = 0; i < kTLoadsA; ++i)
            __builtin_amdgcn_global_load_lds((glb_void *)(asrc[i] + s * 64),
                                             (lds_void *)(buf + (i * kTWaves + wave) * 1024), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < kTLoadsW; ++i)
            __builtin_amdgcn_global_load_lds((glb_void *)(wsrc[i] + static_cast<size_t>(s) * wstep),
                                             (lds_void *)(buf + kTAStage + (i * kTWaves + wave) * 1024), 16, 0,
                                             PACKED ? 2 : 0);  // 2: nt
    };
    auto step = [&](int s, const int8_t *cur, int8_t *freebuf) {
        dma(min(s + 3, n_stages - 1), freebuf);
        __builtin_amdgcn_sched_barrier(0);  // issue the copies before the stage's LDS reads
        compute(cur);
        __builtin_amdgcn_s_waitcnt(kWaitNext);  // stage s + 1's copies have landed, and this wave's LDS reads
        __builtin_amdgcn_s_barrier();
    };
    dma(0, s_d0);
    dma(1, s_d1);
    dma(2, s_d2);
    __builtin_amdgcn_s_waitcnt(kWaitNext);
    __builtin_amdgcn_s_barrier();
    for (int s = 0; s < n_stages; s += 4) {  // n_stages is a multiple of 4
        step(s, s_d0, s_d3);
        step(s + 1, s_d1, s_d0);
        step(s + 2, s_d2, s_d1);
        step(s + 3, s_d3, s_d2);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): the reloads past the last stage have landed

    // Epilogue: lane l holds rows 4 (l / 16) + i of each of the wave's row
    // tiles, at channel l % 16 of each weight tile.
    const int32_t *tidx = KIND == 1 ? aidx : (routed ? a.zrow : a.row_token);
#pragma unroll
    for (int mt = 0; mt < kTMT; ++mt) {
        int otok[4];
        float rsc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lr = min(wm * kTMT * kTileN + mt * kTileN + 4 * kg + i, rows - 1);
            otok[i] = tidx[row0 + lr];
            rsc[i] = Ascale[KIND == 1 ? otok[i] : row0 + lr];
        }
#pragma unroll
        for (int q = 0; q < kTQ; ++q) {
            const int pq = wn * kTQ + q;
            const int rowA = row_a(pq), rowB = row_b(pq);
            const float ws0 = Ws[rowA + r16], ws1 = Ws[rowB + r16];
            if (KIND == 1) {
                const int col = rowA + r16;  // gate channel index = h column
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int lr = wm * kTMT * kTileN + mt * kTileN + 4 * kg + i;
                    if (lr < rows) {
                        const int r = row0 + lr;
                        a.h[static_cast<size_t>(r) * a.imax + col] =
                            swiglu(acc0[mt][q][i], acc1[mt][q][i], ws0, ws1, rsc[i]);
                        if (a.dbg_acc) {
                            a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + col] = acc0[mt][q][i];
                            a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + inter + col] = acc1[mt][q][i];
                        }
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int lr = wm * kTMT * kTileN + mt * kTileN + 4 * kg + i;
                    const uint32_t h0 = f32_to_bf16(dequant(acc0[mt][q][i], ws0, rsc[i]));
                    const uint32_t h1 = f32_to_bf16(dequant(acc1[mt][q][i], ws1, rsc[i]));
                    // neighbouring channels share a 4-byte store: even lanes
                    // take channels (c, c + 1) of tile A, odd lanes (c - 1, c)
                    // of tile B, so 16 lanes store 64 contiguous bytes
                    const uint32_t p0 = __shfl_xor(static_cast<int>(h0), 1, kWave);
                    const uint32_t p1 = __shfl_xor(static_cast<int>(h1), 1, kWave);
                    const bool even = (r16 & 1) == 0;
                    const uint32_t word = even ? (h0 | (p0 << 16)) : (p1 | (h1 << 16));
                    const int wcol = even ? rowA + r16 : rowB + r16 - 1;
                    if (lr < rows) {
                        const int r = row0 + lr;
                        uint16_t *dst = (routed ? a.z : a.share_out) + static_cast<size_t>(otok[i]) * a.H;
                        *reinterpret_cast<uint32_t *>(dst + wcol) = word;
                        if (a.dbg_acc) {
                            a.dbg_acc[static_cast<size_t>(r) * a.H + rowA + r16] = acc0[mt][q][i];
                            a.dbg_acc[static_cast<size_t>(r) * a.H + rowB + r16] = acc1[mt][q][i];
                        }
                        if (a.dbg_z)
                            *reinterpret_cast<uint32_t *>(a.dbg_z + static_cast<size_t>(r) * a.H + wcol) = word;
                    }
                }
            }
        }
    }
}

template <int KIND>
hipError_t launch_tall(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (k_dim % (4 * kTSteps * 64) != 0) return hipErrorInvalidValue;  // the loop runs 4 stages per turn
    const long blocks = static_cast<long>(max_chunks) * a.n_tiles;
    if (blocks <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(blocks)), blk(kTThreads);
    if (a.packed) {
        if (e0 || e1)
            hipExtLaunchKernelGGL((gemm_tall_kernel<KIND, true>), grid, blk, 0, s, e0, e1, 0, a, k_dim);
        else
            hipLaunchKernelGGL((gemm_tall_kernel<KIND, true>), grid, blk, 0, s, a, k_dim);
    } else {
        if (e0 || e1)
            hipExtLaunchKernelGGL((gemm_tall_kernel<KIND, false>), grid, blk, 0, s, e0, e1, 0, a, k_dim);
        else
            hipLaunchKernelGGL((gemm_tall_kernel<KIND, false>), grid, blk, 0, s, a, k_dim);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm1_tall(const GemmArgs &a, int max_chunks, hipStream_t s, hipEvent_t ev_start,
                             hipEvent_t ev_stop) {
    return launch_tall<1>(a, max_chunks, a.H, s, ev_start, ev_stop);
}

hipError_t launch_gemm2_tall(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t ev_start,
                             hipEvent_t ev_stop) {
    return launch_tall<2>(a, max_chunks, k_dim, s, ev_start, ev_stop);
}

}  // namespace moe
