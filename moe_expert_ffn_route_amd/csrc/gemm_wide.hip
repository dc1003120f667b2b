// Grouped INT8 GEMMs for work items of several 16-row MFMA tiles (more than
// 16 tokens in the batch), with the same fused epilogues as gemm.hip:
//   GEMM1 ("FusedDeepMoE Kernel 深度分析报告" sec. 3.3 / 6.1): gate and up
//     accumulators of one row and channel meet in one lane, which applies
//     y = (float(acc) * w1s[n]) * xs[r] to both and writes
//     h = (y_g / (1 + exp(-y_g))) * y_u as fp32;
//   GEMM2 (sec. 3.4 / 6.2): z = bf16((float(acc) * w2s[n]) * hs[r]), to the
//     routed row buffer or, for the shared expert, straight to share_output.
//
// Here the rows of a chunk (up to 16 * MT) are reused across many weight
// rows, so the chunk's activations are shared by the waves of a workgroup
// instead of being fetched by each wave:
//   - the workgroup covers NW pairs of 16-row weight tiles; wave w owns pair
//     w and walks the whole K range, streaming its weights straight from
//     memory into registers (a ring of SLAB 64-byte K steps: the load of
//     step s + SLAB is issued right after the MFMAs of step s consumed its
//     slot), so every weight byte is read once and only by one wave;
//   - the activation rows go through LDS in slabs of SLAB K steps, double
//     buffered: the waves load slab s + 1 into registers while they multiply
//     slab s, write it to LDS at the end of the slab and meet at one
//     workgroup barrier per slab;
//   - with no K split there is no cross-wave reduction: each lane holds the
//     finished int32 sums of its (row, channel) outputs;
//   - with group-wise activation scales each group's int32 sums are
//     dequantised by the group's scale at the group's end and added to fp32
//     sums in group order, which is the order the oracle adds them in.
// LDS layout: the slab's rows, each padded by 16 bytes (see wide_body).
#include "internal.h"

#include <hip/hip_ext.h>

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i ld16(const int8_t *p) { return *reinterpret_cast<const v4i *>(p); }
__device__ __forceinline__ v4i ld16_stream(const int8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
}

// What a wave knows about its work item once the block has decoded it.
struct WideItem {
    const int8_t *wb0, *wb1;  // wave-uniform bases of the first pair of weight tiles
    size_t jstride;           // bytes from one of the wave's tile pairs to the next
    const float *Ws;
    const int8_t *Abase;
    const float *Ascale;
    uint32_t wlane;           // lane offset of a weight load
    int wstep;                // bytes between consecutive K steps of a tile
    int rowA, rowB;           // first weight row (= output channel) of the first pair
    int jcol;                 // channels from one tile pair to the next
    int row0, rows, S, inter;
    const int32_t *aidx;        // GEMM1: where row r's activations are (null: row r)
    const int32_t *tidx;        // epilogue rows' scale index (GEMM1) / z or share_output row (GEMM2)
    bool routed;
};

// The K loop and epilogue for MTA active row tiles (the chunk's rows, rounded
// up to whole tiles) and NT pairs of weight tiles per wave. Runs the same
// sequence in every wave of the block.
// GS > 0: group-wise activation scales ("DeepSeek V4 Decode Optimization"
// sec. 3.1), one per GS 64-byte K steps of a row (a.a_ng per row). At the end
// of each group the lane's int32 sums are dequantised, p = (float(acc) *
// w_scale[n]) * group_scale[row], and added to fp32 sums in group order (a
// wave walks the whole K, so the order is the groups' own); each group's
// first MFMA starts from zero. The groups' scales of a slab travel with its
// activation rows through LDS (s_g).
template <int KIND, int NW, int NT, int MTA, int SLAB, int RING, bool PACKED, int GS = 0>
__device__ __forceinline__ void wide_body(const GemmArgs &a, const WideItem &it, v4i *s_a, float *s_g) {
    // Activation slab layout in LDS: the chunk's 16 * MTA rows, each holding
    // the slab's SLAB * 64 bytes plus 16 bytes of padding. A load instruction
    // reads kRpi whole row segments (contiguous, so every 128-byte line it
    // touches is used in full), a store writes them unchanged, and the
    // padding spreads the 16 rows an MFMA operand read gathers over distinct
    // LDS banks.
    constexpr int kLpr = 4 * SLAB;                 // lanes per row segment (16 bytes each)
    constexpr int kRpi = kWave / kLpr;             // row segments per load instruction
    constexpr int kStr = kLpr + 1;                 // LDS row stride, in 16-byte units
    constexpr int kBuf = kTileN * MTA * kStr;      // one slab buffer
    constexpr int kUnits = kTileN * MTA / kRpi;    // load instructions per slab (= SLAB * MTA)
    constexpr int kUpw = (kUnits + NW - 1) / NW;   // of them, per wave
    constexpr int kSlabsPerRing = RING / SLAB;
    static_assert(kWave % kLpr == 0, "a load instruction covers whole row segments");
    static_assert(GS == 0 || SLAB % GS == 0, "group-wise scales: whole groups per slab");
    constexpr int kGps = GS > 0 ? SLAB / GS : 1;    // groups per slab
    constexpr int kGvals = kTileN * MTA * kGps;    // group scales of a slab
    static_assert(kGvals <= NW * kWave, "one thread stages each group scale of a slab");
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int r16 = lane & 15, kg = lane >> 4;
    const int rows = it.rows, row0 = it.row0;

    // (1) independent small loads: the token of each activation row this
    //     wave stages and of each output row it finishes (4 * (lane / 16) + i
    //     of every row tile), and the channel scales
    const int8_t *asrc[kUpw];
    const int seg = lane % kLpr;  // this lane's 16 bytes within a row segment
#pragma unroll
    for (int j = 0; j < kUpw; ++j) {
        const int u = wave + j * NW;
        const int lr = min(u * kRpi + lane / kLpr, rows - 1);  // rows past the chunk repeat its last row
        const int ar = it.aidx ? it.aidx[row0 + lr] : row0 + lr;
        asrc[j] = it.Abase + static_cast<size_t>(ar) * a.a_stride + seg * 16;
    }
    // group-wise scales: thread t < kGvals stages the scale of row t / kGps,
    // group t % kGps of each slab
    const float *gsrc = nullptr;
    if constexpr (GS > 0) {
        const int t = threadIdx.x;
        const int lr = min(min(t, kGvals - 1) / kGps, rows - 1);
        const int srow = it.aidx ? it.aidx[row0 + lr] : row0 + lr;
        gsrc = it.Ascale + static_cast<size_t>(srow) * a.a_ng + min(t, kGvals - 1) % kGps;
    }
    // a token indexes the row scale of per-token rows and the share_output
    // row of the shared expert's GEMM2
    int otok[MTA][4];
    float rsc[MTA][4];
    auto load_tokens = [&] {
#pragma unroll
        for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int lr = min(mt * kTileN + 4 * kg + i, rows - 1);
                otok[mt][i] = it.tidx ? it.tidx[row0 + lr] : 0;
            }
    };
    auto load_scales = [&] {
#pragma unroll
        for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                rsc[mt][i] = GS > 0 ? 0.0f
                                    : it.Ascale[it.aidx ? otok[mt][i] : row0 + min(mt * kTileN + 4 * kg + i, rows - 1)];
    };
    load_tokens();
    float ws0[NT], ws1[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        ws0[j] = it.Ws[it.rowA + j * it.jcol + r16];
        ws1[j] = it.Ws[it.rowB + j * it.jcol + r16];
    }
    __builtin_amdgcn_sched_barrier(0);

    // (2) the first activation slab, then the first ring of weight steps
    auto ldw = [&](const int8_t *base, int j, int step) {
        const int8_t *p = base + j * it.jstride + static_cast<size_t>(step) * it.wstep + it.wlane;
        return PACKED ? ld16_stream(p) : ld16(p);
    };
    v4i stage[kUpw];
    float gstage = 0.0f;
    auto load_slab = [&](int s) {
#pragma unroll
        for (int j = 0; j < kUpw; ++j)
            if (kUnits % NW == 0 || wave + j * NW < kUnits) stage[j] = ld16(asrc[j] + s * SLAB * 64);
        if constexpr (GS > 0) {
            if (static_cast<int>(threadIdx.x) < kGvals) gstage = gsrc[s * kGps];
        }
    };
    auto store_slab = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kUpw; ++j)
            if (kUnits % NW == 0 || wave + j * NW < kUnits)
                s_a[buf * kBuf + ((wave + j * NW) * kRpi + lane / kLpr) * kStr + seg] = stage[j];
        if constexpr (GS > 0) {
            if (static_cast<int>(threadIdx.x) < kGvals) s_g[buf * kGvals + threadIdx.x] = gstage;
        }
    };
    load_slab(0);
    __builtin_amdgcn_sched_barrier(0);
    v4i w0[RING][NT], w1[RING][NT];
#pragma unroll
    for (int i = 0; i < RING; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            w0[i][j] = ldw(it.wb0, j, i);
            w1[i][j] = ldw(it.wb1, j, i);
        }
    __builtin_amdgcn_sched_barrier(0);

    // (3) loads that depend on (1): the row scales of this lane's output rows
    load_scales();
    __builtin_amdgcn_sched_barrier(0);

    store_slab(0);
    __syncthreads();

    v4i acc0[MTA][NT], acc1[MTA][NT];
    float f0[MTA][NT][4], f1[MTA][NT][4];  // group-wise: dequantised sums
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            acc0[mt][j] = v4i{0, 0, 0, 0};
            acc1[mt][j] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f0[mt][j][i] = 0.0f;
                f1[mt][j][i] = 0.0f;
            }
        }
    // group-wise: dequantise the finished group q of slab buffer `cur` into
    // the fp32 sums, in group order
    auto flush = [&](int cur, int q) {
#pragma unroll
        for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gsc = s_g[cur * kGvals + (mt * kTileN + 4 * kg + i) * kGps + q];
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    float p0 = static_cast<float>(acc0[mt][j][i]) * ws0[j];
                    p0 = p0 * gsc;
                    f0[mt][j][i] = f0[mt][j][i] + p0;
                    float p1 = static_cast<float>(acc1[mt][j][i]) * ws1[j];
                    p1 = p1 * gsc;
                    f1[mt][j][i] = f1[mt][j][i] + p1;
                }
            }
    };
    // One slab of SLAB K steps at ring position h: the next slab's activation
    // loads, then for each step the MFMAs of all row tiles followed by the
    // weight loads that refill the step's ring slot (RING steps ahead); at the
    // end the next slab goes to the other LDS buffer. Scheduling barriers keep
    // each refill right after its step's MFMAs (left alone, the compiler sinks
    // the refills to the end of the slab).
    auto slab = [&](int s, int h, bool more_a, bool more_w) {
        const int cur = s & 1;
        if (more_a) load_slab(s + 1);
        const int wnext = s * SLAB + RING;
#pragma unroll
        for (int i = 0; i < SLAB; ++i) {
            const int slot = h * SLAB + i;
            const bool first = GS > 0 && i % (GS > 0 ? GS : 1) == 0;  // a group's first step
            const v4i zero = {0, 0, 0, 0};
#pragma unroll
            for (int mt = 0; mt < MTA; ++mt) {
                const v4i x = s_a[cur * kBuf + (mt * kTileN + r16) * kStr + i * 4 + kg];
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    acc0[mt][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x, w0[slot][j], first ? zero : acc0[mt][j],
                                                                        0, 0, 0);
                    acc1[mt][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x, w1[slot][j], first ? zero : acc1[mt][j],
                                                                        0, 0, 0);
                }
            }
            if (GS > 0 && (i + 1) % (GS > 0 ? GS : 1) == 0) flush(cur, i / (GS > 0 ? GS : 1));
            if (more_w) {
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    w0[slot][j] = ldw(it.wb0, j, wnext + i);
                    w1[slot][j] = ldw(it.wb1, j, wnext + i);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (more_a) store_slab(cur ^ 1);
        __syncthreads();
    };
    // Every row tile is multiplied, also past the chunk's last row: those A
    // rows repeat the last row, and since an MFMA output row depends only on
    // its own A row, they only produce outputs that are never stored.
    const int ncyc = it.S / RING;
    for (int cyc = 0; cyc + 1 < ncyc; ++cyc) {
#pragma unroll
        for (int h = 0; h < kSlabsPerRing; ++h) slab(cyc * kSlabsPerRing + h, h, true, true);
    }
#pragma unroll
    for (int h = 0; h < kSlabsPerRing; ++h)
        slab((ncyc - 1) * kSlabsPerRing + h, h, h + 1 < kSlabsPerRing, false);

    // Epilogue: lane l holds rows 4 * (l / 16) + i of every row tile, at
    // channel l % 16 of every weight tile.
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int rowA = it.rowA + j * it.jcol, rowB = it.rowB + j * it.jcol;
            if (KIND == 1) {
                const int col = rowA + r16;  // gate channel index = h column
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int lr = mt * kTileN + 4 * kg + i;
                    if (lr < rows) {
                        const int r = row0 + lr;
                        a.h[static_cast<size_t>(r) * a.imax + col] =
                            GS > 0 ? swiglu_y(f0[mt][j][i], f1[mt][j][i])
                                   : swiglu(acc0[mt][j][i], acc1[mt][j][i], ws0[j], ws1[j], rsc[mt][i]);
                        if (a.dbg_acc) {
                            a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + col] =
                                GS > 0 ? __float_as_int(f0[mt][j][i]) : acc0[mt][j][i];
                            a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + it.inter + col] =
                                GS > 0 ? __float_as_int(f1[mt][j][i]) : acc1[mt][j][i];
                        }
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int lr = mt * kTileN + 4 * kg + i;
                    const uint32_t b0 =
                        f32_to_bf16(GS > 0 ? f0[mt][j][i] : dequant(acc0[mt][j][i], ws0[j], rsc[mt][i]));
                    const uint32_t b1 =
                        f32_to_bf16(GS > 0 ? f1[mt][j][i] : dequant(acc1[mt][j][i], ws1[j], rsc[mt][i]));
                    // pair up neighbouring channels for 4-byte stores: even
                    // lanes take channels (c, c + 1) of tile A, odd lanes
                    // (c - 1, c) of tile B, so 16 lanes store 64 contiguous
                    // bytes of the row
                    const uint32_t p0 = __shfl_xor(static_cast<int>(b0), 1, kWave);
                    const uint32_t p1 = __shfl_xor(static_cast<int>(b1), 1, kWave);
                    const bool even = (r16 & 1) == 0;
                    const uint32_t word = even ? (b0 | (p0 << 16)) : (p1 | (b1 << 16));
                    const int wcol = even ? rowA + r16 : rowB + r16 - 1;
                    if (lr < rows) {
                        const int r = row0 + lr;
                        uint16_t *dst = (it.routed ? a.z : a.share_out) + static_cast<size_t>(otok[mt][i]) * a.H;
                        *reinterpret_cast<uint32_t *>(dst + wcol) = word;
                        if (a.dbg_acc) {
                            a.dbg_acc[static_cast<size_t>(r) * a.H + rowA + r16] =
                                GS > 0 ? __float_as_int(f0[mt][j][i]) : acc0[mt][j][i];
                            a.dbg_acc[static_cast<size_t>(r) * a.H + rowB + r16] =
                                GS > 0 ? __float_as_int(f1[mt][j][i]) : acc1[mt][j][i];
                        }
                        if (a.dbg_z)
                            *reinterpret_cast<uint32_t *>(a.dbg_z + static_cast<size_t>(r) * a.H + wcol) = word;
                    }
                }
            }
        }
    }
}

// Decodes the work item of block index b of one item class (chunk list,
// chunk count word, N groups per chunk) into `it`, for a block of NW waves
// holding NT tile pairs each. Returns false when the block has no work.
template <int KIND, int NW, int NT, bool PACKED>
__device__ __forceinline__ bool decode_item(const GemmArgs &a, const int4 *chunks, int count_word, int n_tiles,
                                            int b, int k_dim, WideItem &it) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    int c = b / n_tiles;
    int nt = b % n_tiles;
    int4 ch = chunks[c];  // c < the class's capacity: inside the list even when unused
    if (c >= a.meta[count_word]) return false;
    const int nch = ch.z >> kChunkCountShift;
    if (nch > 1 && (n_tiles & 7) == 0) {
        // the chunks of one N tile run 8 blocks apart, on one XCD (gemm.hip)
        const int c0 = c - ch.w;
        const int i = b - c0 * n_tiles;
        const int q = i / (8 * nch), rem = i - q * 8 * nch;
        c = c0 + rem / 8;
        nt = q * 8 + rem % 8;
        ch = chunks[c];
    }
    const int g = ch.x;
    it.row0 = ch.y;
    it.rows = ch.z & kChunkRowsMask;
    if (g < a.g_lo || g >= a.g_hi) return false;
    it.routed = g < a.E_loc;
    it.inter = it.routed ? a.I : a.I_s;
    // inter and H are multiples of 256 and a block covers at most 256
    // channels, so a block either has work for all of its waves or for none
    if (KIND == 1 && nt * NW * NT * kTileN >= it.inter) return false;

    const int8_t *W;
    const int tp = (nt * NW + wave) * NT;  // this wave's first pair of 16-row weight tiles
    it.S = k_dim / 64;                     // 64-byte K steps; a multiple of the ring (host-checked)
    const size_t tile_bytes = static_cast<size_t>(kTileN) * k_dim;
    if (KIND == 1) {
        W = it.routed ? a.W + static_cast<size_t>(g) * 2 * it.inter * a.H : a.W_sh;
        it.Ws = it.routed ? a.Ws + static_cast<size_t>(g) * 2 * it.inter : a.Ws_sh;
        it.rowA = tp * kTileN;             // gate channels
        it.rowB = it.inter + tp * kTileN;  // matching up channels
        it.jcol = kTileN;
    } else {
        W = it.routed ? a.W + static_cast<size_t>(g) * a.H * it.inter : a.W_sh;
        it.Ws = it.routed ? a.Ws + static_cast<size_t>(g) * a.H : a.Ws_sh;
        it.rowA = tp * 2 * kTileN;
        it.rowB = it.rowA + kTileN;
        it.jcol = 2 * kTileN;
    }
    it.jstride = (it.jcol / kTileN) * tile_bytes;  // a tile is 16 rows x k_dim bytes in both layouts
    // weight addresses: a wave-uniform base plus a 32-bit lane offset
    if (PACKED) {
        if (KIND == 1) {
            it.wb0 = W + g1_tile_pos(it.rowA / kTileN, it.inter / kTileN) * tile_bytes;
            it.wb1 = W + g1_tile_pos(it.rowB / kTileN, it.inter / kTileN) * tile_bytes;
            it.jstride = 2 * tile_bytes;  // the next gate tile
        } else {
            it.wb0 = W + static_cast<size_t>(it.rowA / kTileN) * tile_bytes;
            it.wb1 = W + static_cast<size_t>(it.rowB / kTileN) * tile_bytes;
        }
        it.wlane = lane * 16;
        it.wstep = 1024;
    } else {
        it.wb0 = W + static_cast<size_t>(it.rowA) * k_dim;
        it.wb1 = W + static_cast<size_t>(it.rowB) * k_dim;
        it.wlane = (lane & 15) * k_dim + (lane >> 4) * 16;
        it.wstep = 64;
    }
    // GEMM1 row r reads its activations through an index (routed rows: the
    // token's or the (token, expert) pair's quantised row; shared rows: the
    // token's); GEMM2 row r reads row r
    it.aidx = KIND == 1 ? (it.routed ? a.idx_r : a.row_token) : nullptr;
    it.tidx = KIND == 1 ? it.aidx : (it.routed ? a.zrow : a.row_token);
    it.Abase = KIND == 1 ? (it.routed ? a.A_r : a.A_s) : a.A;
    it.Ascale = KIND == 1 ? (it.routed ? a.a_scale_r : a.a_scale_s) : a.a_scale;
    return true;
}

// Tile parameters: 2 waves of one tile pair each, activation slabs of 4 K
// steps, a weight ring of 8 steps (4 where 8 does not divide K).
#ifndef MOE_WIDE_WAVES
#define MOE_WIDE_WAVES 2
#endif
#ifndef MOE_WIDE_SLAB
#define MOE_WIDE_SLAB 4
#endif
constexpr int kWideWaves = MOE_WIDE_WAVES, kWideSlab = MOE_WIDE_SLAB;

template <int KIND, int NW, int NT, int MT, int SLAB, int RING, bool PACKED, int GS>
__global__ __launch_bounds__(NW * kWave, 2) void gemm_wide_kernel(GemmArgs a, int k_dim) {
    __shared__ v4i s_a[2 * kTileN * MT * (4 * SLAB + 1)];
    __shared__ float s_g[GS > 0 ? 2 * kTileN * MT * (SLAB / (GS > 0 ? GS : 1)) : 1];
    WideItem it;
    if (!decode_item<KIND, NW, NT, PACKED>(a, a.chunks, a.count_word, a.n_tiles, blockIdx.x, k_dim, it)) return;
    // run the body for the row tiles the chunk actually fills
    static_assert(MT <= 2, "items of one or two row tiles");
    const int tiles = (it.rows + kTileN - 1) / kTileN;
    if constexpr (MT > 1) {
        if (tiles > 1) return wide_body<KIND, NW, NT, 2, SLAB, RING, PACKED, GS>(a, it, s_a, s_g);
    }
    wide_body<KIND, NW, NT, 1, SLAB, RING, PACKED, GS>(a, it, s_a, s_g);
}

template <int KIND, int NW, int NT, int MT, int SLAB, int RING, int GS>
hipError_t launch_t(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const long blocks = static_cast<long>(max_chunks) * a.n_tiles;
    if (blocks <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(blocks)), blk(NW * kWave);
    if (a.packed) {
        if (e0 || e1)
            hipExtLaunchKernelGGL((gemm_wide_kernel<KIND, NW, NT, MT, SLAB, RING, true, GS>), grid, blk, 0, s, e0, e1,
                                  0, a, k_dim);
        else
            hipLaunchKernelGGL((gemm_wide_kernel<KIND, NW, NT, MT, SLAB, RING, true, GS>), grid, blk, 0, s, a, k_dim);
    } else {
        if (e0 || e1)
            hipExtLaunchKernelGGL((gemm_wide_kernel<KIND, NW, NT, MT, SLAB, RING, false, GS>), grid, blk, 0, s, e0,
                                  e1, 0, a, k_dim);
        else
            hipLaunchKernelGGL((gemm_wide_kernel<KIND, NW, NT, MT, SLAB, RING, false, GS>), grid, blk, 0, s, a, k_dim);
    }
    return hipGetLastError();
}

// Longest weight ring with group-wise scales of 128 elements (the per-group
// dequantisation holds extra registers: with 64-element groups an 8-step
// ring spills, so those take 4). Measured at T = 512, 128-element groups:
// 8-step ring 1073 us per layer (234 VGPRs), 4-step 1088 us (153 VGPRs).
#ifndef MOE_WIDE_GRP_RING
#define MOE_WIDE_GRP_RING 8
#endif
template <int KIND, int GS>
hipError_t launch_rings(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    constexpr int kMaxRing = GS == 1 ? 4 : GS == 2 ? MOE_WIDE_GRP_RING : 8;
    if (kMaxRing == 8 && (k_dim / 64) % 8 == 0)
        return launch_t<KIND, kWideWaves, 1, kWideTiles, kWideSlab, 8, GS>(a, max_chunks, k_dim, s, e0, e1);
    return launch_t<KIND, kWideWaves, 1, kWideTiles, kWideSlab, 4, GS>(a, max_chunks, k_dim, s, e0, e1);
}

// k_dim is a multiple of 256, so rings of 4 steps always divide it; a group
// (gsteps = 1, 2 or 4 steps) never straddles a slab of 4 steps
template <int KIND>
hipError_t launch_items(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (a.mt != kWideTiles) return hipErrorInvalidValue;
    static_assert(kWideSlab % 4 == 0, "slabs hold whole groups of up to 4 steps");
    switch (a.gsteps) {
        case 0: return launch_rings<KIND, 0>(a, max_chunks, k_dim, s, e0, e1);
        case 1: return launch_rings<KIND, 1>(a, max_chunks, k_dim, s, e0, e1);
        case 2: return launch_rings<KIND, 2>(a, max_chunks, k_dim, s, e0, e1);
        case 4: return launch_rings<KIND, 4>(a, max_chunks, k_dim, s, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemm1_wide(const GemmArgs &a, int max_chunks, hipStream_t s, hipEvent_t ev_start,
                             hipEvent_t ev_stop) {
    return launch_items<1>(a, max_chunks, a.H, s, ev_start, ev_stop);
}

hipError_t launch_gemm2_wide(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t ev_start,
                             hipEvent_t ev_stop) {
    return launch_items<2>(a, max_chunks, k_dim, s, ev_start, ev_stop);
}

int wide_tile_pairs() { return kWideWaves; }

}  // namespace moe
