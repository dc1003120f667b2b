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
// Chunks of 16 rows take gemm.hip's decode decomposition (a 16-channel tile
// pair per workgroup, K split over the waves, partial tiles summed in LDS,
// linear blockIdx so every XCD streams a share of every expert); chunks of 32
// rows (batches whose local experts average 16 rows or more) take the
// two-tile kernel at the end of this file, which walks the whole K per wave.
// Against the INT8 kernels only the operands change:
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
// reads its weights once; the library instantiates MT = 1).
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

// Chunks of one row tile (batches of at most 16 tokens, or larger batches
// whose local experts average fewer than 16 rows) split K over MOE_MX_WAVES
// waves; chunks of two row tiles take the two-tile kernel below.
template <int KIND>
hipError_t launch_kind(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    static_assert(MOE_MX_WAVES == 8 || MOE_MX_WAVES == 4, "MOE_MX_WAVES is 8 or 4");
    constexpr int W = MOE_MX_WAVES;
    if (a.mt != 1 || k_dim % 256) return hipErrorInvalidValue;
    const long blocks = static_cast<long>(max_chunks) * a.n_tiles;
    if (blocks <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(blocks));
    const int steps = k_dim / kStepK;
    if (steps % W == 0) return launch_split<KIND, W, 1>(a, grid, k_dim, steps / W, s, e0, e1);
    if (steps % 4 == 0) return launch_one<KIND, 4, 1, 0, 1>(a, grid, k_dim, steps / 4, s, e0, e1);
    return launch_one<KIND, 2, 1, 0, 1>(a, grid, k_dim, steps / 2, s, e0, e1);
}

// ---------------------------------------------------------------------------
// Work items of two 16-row tiles (32-row chunks: batches where the local
// experts average 16 rows or more). The K-split kernel above would re-read a
// chunk's FP8 rows (4 KB per 128-element step) for every 16-channel tile
// pair, twice the FP4 weight bytes of the pair; here a workgroup of NW waves
// covers NW * NT tile pairs, each wave walks the whole K range with its own
// pairs' weights streaming from memory into a register ring (RING steps ahead,
// every weight byte read once by one wave), and the chunk's activation rows go
// through LDS in double-buffered slabs of SLAB steps shared by all waves (one
// workgroup barrier per slab). No K split, so each lane ends with finished
// fp32 sums of its (row, channel) outputs, added in K order by the MFMA.
// LDS slab layout: the chunk's 32 rows, each SLAB * 128 bytes plus 16 bytes of
// padding (a load instruction reads whole row segments; the padding spreads
// the 16 rows of an operand read over the banks).
struct MxItem {
    const uint8_t *wd0, *wd1;  // element blocks of the wave's first pair of weight tiles, step 0
    const uint8_t *ws0, *ws1;  // their scale blocks
    size_t jd, js;             // bytes from one of the wave's pairs to the next: elements, scales
    const float *Ws;
    const uint8_t *Abase;
    const float *Ascale;
    int rowA, rowB, jcol;      // first output channel of each tile of the first pair; channels per pair
    int row0, rows, S, inter;  // S = 128-element K steps
    const int32_t *aidx;       // GEMM1: where row r's codes are (null: row r)
    const int32_t *tidx;       // epilogue rows' scale index (GEMM1) / z or share_output row (GEMM2)
    bool routed;
};

template <int KIND, int NW, int NT, int MTA, int SLAB, int RING>
__device__ __forceinline__ void mx_wide_body(const GemmArgs &a, const MxItem &it, v4i *s_a) {
    constexpr int kLpr = 8 * SLAB;                 // 16-byte units per row segment
    constexpr int kRpi = kWave / kLpr;             // row segments per load instruction
    constexpr int kStr = kLpr + 1;                 // LDS row stride in 16-byte units
    constexpr int kBuf = kTileN * MTA * kStr;      // one slab buffer
    constexpr int kUnits = kTileN * MTA / kRpi;    // load instructions per slab
    constexpr int kUpw = (kUnits + NW - 1) / NW;   // of them, per wave
    constexpr int kSlabsPerRing = RING / SLAB;
    static_assert(kWave % kLpr == 0 && RING % SLAB == 0, "whole row segments; whole slabs per ring");
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int r16 = lane & 15, kg = lane >> 4;
    const int rows = it.rows, row0 = it.row0;

    // (1) independent small loads: activation rows this wave stages, the
    //     rows of its outputs, the channel scales
    const uint8_t *asrc[kUpw];
    const int seg = lane % kLpr;
#pragma unroll
    for (int j = 0; j < kUpw; ++j) {
        const int u = wave + j * NW;
        const int lr = min(u * kRpi + lane / kLpr, rows - 1);  // rows past the chunk repeat its last row
        const int ar = it.aidx ? it.aidx[row0 + lr] : row0 + lr;
        asrc[j] = it.Abase + static_cast<size_t>(ar) * a.a_stride + seg * 16;
    }
    int otok[MTA][4];
    float rsc[MTA][4];
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lr = min(mt * kTileN + 4 * kg + i, rows - 1);
            otok[mt][i] = it.tidx ? it.tidx[row0 + lr] : 0;
        }
    float wsc0[NT], wsc1[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        wsc0[j] = it.Ws[it.rowA + j * it.jcol + r16];
        wsc1[j] = it.Ws[it.rowB + j * it.jcol + r16];
    }
    __builtin_amdgcn_sched_barrier(0);

    // (2) the first activation slab, then the first ring of weight steps
    v4i stage[kUpw];
    auto load_slab = [&](int s) {
#pragma unroll
        for (int j = 0; j < kUpw; ++j)
            if (kUnits % NW == 0 || wave + j * NW < kUnits) stage[j] = ld16(asrc[j] + s * SLAB * kStepK);
    };
    auto store_slab = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kUpw; ++j)
            if (kUnits % NW == 0 || wave + j * NW < kUnits)
                s_a[buf * kBuf + ((wave + j * NW) * kRpi + lane / kLpr) * kStr + seg] = stage[j];
    };
    auto ldw = [&](const uint8_t *base, int j, int step) {
        return ld16_stream(base + j * it.jd + static_cast<size_t>(step) * 1024 + lane * 16);
    };
    auto lds = [&](const uint8_t *base, int j, int step) {
        return static_cast<int>(base[j * it.js + static_cast<size_t>(step) * 64 + lane]);
    };
    load_slab(0);
    __builtin_amdgcn_sched_barrier(0);
    v4i w0[RING][NT], w1[RING][NT];
    int s0[RING][NT], s1[RING][NT];
#pragma unroll
    for (int i = 0; i < RING; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            w0[i][j] = ldw(it.wd0, j, i);
            w1[i][j] = ldw(it.wd1, j, i);
            s0[i][j] = lds(it.ws0, j, i);
            s1[i][j] = lds(it.ws1, j, i);
        }
    __builtin_amdgcn_sched_barrier(0);

    // (3) loads that depend on (1): the row scales of this lane's output rows
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            rsc[mt][i] = it.Ascale[it.aidx ? otok[mt][i] : row0 + min(mt * kTileN + 4 * kg + i, rows - 1)];
    __builtin_amdgcn_sched_barrier(0);

    store_slab(0);
    __syncthreads();

    v4f acc0[MTA][NT], acc1[MTA][NT];
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            acc0[mt][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            acc1[mt][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        }
    // One slab at ring position h: the next slab's activation loads, then per
    // step the MFMAs of all row tiles followed by the refill of the step's
    // ring slot (RING steps ahead); at the end the next slab goes to the other
    // LDS buffer.
    auto slab = [&](int s, int h, bool more_a, bool more_w) {
        const int cur = s & 1;
        if (more_a) load_slab(s + 1);
        const int wnext = s * SLAB + RING;
#pragma unroll
        for (int i = 0; i < SLAB; ++i) {
            const int slot = h * SLAB + i;
#pragma unroll
            for (int mt = 0; mt < MTA; ++mt) {
                // A operand of lane l: row l % 16, bytes 16 g .. +16 and
                // 64 + 16 g .. +16 of the 128-byte step (g = l / 16)
                const int base = cur * kBuf + (mt * kTileN + r16) * kStr + i * 8 + kg;
                const v4i lo = s_a[base], hi = s_a[base + 4];
                const v8i xa = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const v8i b0 = {w0[slot][j][0], w0[slot][j][1], w0[slot][j][2], w0[slot][j][3], 0, 0, 0, 0};
                    const v8i b1 = {w1[slot][j][0], w1[slot][j][1], w1[slot][j][2], w1[slot][j][3], 0, 0, 0, 0};
                    // cbsz 0: A is FP8 E4M3; blgp 4: B is FP4 E2M1
                    acc0[mt][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa, b0, acc0[mt][j], 0, 4, 0,
                                                                                   kUnitScale, 0, s0[slot][j]);
                    acc1[mt][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa, b1, acc1[mt][j], 0, 4, 0,
                                                                                   kUnitScale, 0, s1[slot][j]);
                }
            }
            if (more_w) {
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    w0[slot][j] = ldw(it.wd0, j, wnext + i);
                    w1[slot][j] = ldw(it.wd1, j, wnext + i);
                    s0[slot][j] = lds(it.ws0, j, wnext + i);
                    s1[slot][j] = lds(it.ws1, j, wnext + i);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (more_a) store_slab(cur ^ 1);
        __syncthreads();
    };
    const int ncyc = it.S / RING;
    for (int cyc = 0; cyc + 1 < ncyc; ++cyc) {
#pragma unroll
        for (int h = 0; h < kSlabsPerRing; ++h) slab(cyc * kSlabsPerRing + h, h, true, true);
    }
#pragma unroll
    for (int h = 0; h < kSlabsPerRing; ++h)
        slab((ncyc - 1) * kSlabsPerRing + h, h, h + 1 < kSlabsPerRing, false);

    // Epilogue: lane l holds rows 4 (l / 16) + i of every row tile at channel
    // l % 16 of every weight tile.
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int rowA = it.rowA + j * it.jcol, rowB = it.rowB + j * it.jcol;
            if (KIND == 1) {
                const int col = rowA + r16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int lr = mt * kTileN + 4 * kg + i;
                    if (lr < rows) {
                        const int r = row0 + lr;
                        a.h[static_cast<size_t>(r) * a.imax + col] =
                            swiglu(acc0[mt][j][i], acc1[mt][j][i], wsc0[j], wsc1[j], rsc[mt][i]);
                        if (a.dbg_acc) {
                            a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + col] = __float_as_int(acc0[mt][j][i]);
                            a.dbg_acc[static_cast<size_t>(r) * 2 * a.imax + it.inter + col] =
                                __float_as_int(acc1[mt][j][i]);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int lr = mt * kTileN + 4 * kg + i;
                    const uint32_t b0 = f32_to_bf16(dequant(acc0[mt][j][i], wsc0[j], rsc[mt][i]));
                    const uint32_t b1 = f32_to_bf16(dequant(acc1[mt][j][i], wsc1[j], rsc[mt][i]));
                    // neighbouring channels paired for 4-byte stores (even
                    // lanes: channels c, c + 1 of tile A; odd: c - 1, c of B)
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
                            a.dbg_acc[static_cast<size_t>(r) * a.H + rowA + r16] = __float_as_int(acc0[mt][j][i]);
                            a.dbg_acc[static_cast<size_t>(r) * a.H + rowB + r16] = __float_as_int(acc1[mt][j][i]);
                        }
                        if (a.dbg_z)
                            *reinterpret_cast<uint32_t *>(a.dbg_z + static_cast<size_t>(r) * a.H + wcol) = word;
                    }
                }
            }
        }
    }
}

template <int KIND, int NW, int NT, int SLAB, int RING>
__global__ __launch_bounds__(NW * kWave, 2) void gemm_mx_wide_kernel(GemmArgs a, int k_dim) {
    __shared__ v4i s_a[2 * kTileN * 2 * (8 * SLAB + 1)];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    int c = blockIdx.x / a.n_tiles;
    int nt = blockIdx.x % a.n_tiles;
    int4 ch = a.chunks[c];  // c < max_chunks: inside the chunk list even when unused
    if (c >= a.meta[a.count_word]) return;
    const int nch = ch.z >> kChunkCountShift;
    if (nch > 1 && (a.n_tiles & 7) == 0) {
        // the chunks of one N group 8 blocks apart: same XCD, weights shared in L2
        const int c0 = c - ch.w;
        const int i = blockIdx.x - c0 * a.n_tiles;
        const int q = i / (8 * nch), rem = i - q * 8 * nch;
        c = c0 + rem / 8;
        nt = q * 8 + rem % 8;
        ch = a.chunks[c];
    }
    const int g = ch.x;
    if (g < a.g_lo || g >= a.g_hi) return;
    MxItem it;
    it.row0 = ch.y;
    it.rows = ch.z & kChunkRowsMask;
    it.routed = g < a.E_loc;
    it.inter = it.routed ? a.I : a.I_s;
    // inter and H are multiples of 256, a block covers at most 256 channels:
    // a block has work for all of its waves or for none
    if (KIND == 1 && nt * NW * NT * kTileN >= it.inter) return;
    const int tp = (nt * NW + wave) * NT;  // this wave's first 16-row tile pair
    it.S = k_dim / kStepK;
    const int n_out = KIND == 1 ? 2 * it.inter : a.H;
    const size_t g_data = static_cast<size_t>(n_out) * (k_dim / 2);
    const size_t g_scale = static_cast<size_t>(n_out) * (k_dim / 32);
    const size_t n_groups = it.routed ? a.E_loc : 1;
    const size_t gi = it.routed ? g : 0;
    const uint8_t *base = reinterpret_cast<const uint8_t *>(it.routed ? a.W : a.W_sh);
    const uint8_t *Wd = base + gi * g_data;
    const uint8_t *Wsc = base + n_groups * g_data + gi * g_scale;
    // packed tile positions: GEMM1 gate tile t at 2t, its up tile at 2t + 1;
    // GEMM2 pair t's tiles at 2t, 2t + 1; the next pair two positions on
    const size_t ta = 2 * static_cast<size_t>(tp), tb = ta + 1;
    it.wd0 = Wd + ta * it.S * 1024;
    it.wd1 = Wd + tb * it.S * 1024;
    it.ws0 = Wsc + ta * it.S * 64;
    it.ws1 = Wsc + tb * it.S * 64;
    it.jd = 2 * static_cast<size_t>(it.S) * 1024;
    it.js = 2 * static_cast<size_t>(it.S) * 64;
    if (KIND == 1) {
        it.Ws = it.routed ? a.Ws + static_cast<size_t>(g) * 2 * it.inter : a.Ws_sh;
        it.rowA = tp * kTileN;
        it.rowB = it.inter + tp * kTileN;
        it.jcol = kTileN;
    } else {
        it.Ws = it.routed ? a.Ws + static_cast<size_t>(g) * a.H : a.Ws_sh;
        it.rowA = tp * 2 * kTileN;
        it.rowB = it.rowA + kTileN;
        it.jcol = 2 * kTileN;
    }
    it.aidx = KIND == 1 ? (it.routed ? a.idx_r : a.row_token) : nullptr;
    it.tidx = KIND == 1 ? it.aidx : (it.routed ? a.zrow : a.row_token);
    it.Abase = reinterpret_cast<const uint8_t *>(KIND == 1 ? (it.routed ? a.A_r : a.A_s) : a.A);
    it.Ascale = KIND == 1 ? (it.routed ? a.a_scale_r : a.a_scale_s) : a.a_scale;
    (void)lane;
    // run the body for the row tiles the chunk fills
    if (it.rows > kTileN) return mx_wide_body<KIND, NW, NT, 2, SLAB, RING>(a, it, s_a);
    mx_wide_body<KIND, NW, NT, 1, SLAB, RING>(a, it, s_a);
}

// Workgroup shape of the two-tile MX kernel per GEMM: waves, tile pairs per
// wave, longest weight ring (steps; 8 or 4). Measured at T = 512 (µs, GEMM1 /
// GEMM2): 4 waves of one pair 391-395 / 207; 2 waves 378 / 234; 8 waves 476 /
// 222; 4 waves with a 4-step ring 397 / 205.
#ifndef MOE_MX_WIDE_WAVES1
#define MOE_MX_WIDE_WAVES1 2
#endif
#ifndef MOE_MX_WIDE_WAVES2
#define MOE_MX_WIDE_WAVES2 4
#endif
#ifndef MOE_MX_WIDE_NT1
#define MOE_MX_WIDE_NT1 1
#endif
#ifndef MOE_MX_WIDE_NT2
#define MOE_MX_WIDE_NT2 1
#endif
#ifndef MOE_MX_WIDE_RING
#define MOE_MX_WIDE_RING 8
#endif
template <int KIND>
struct MxWideShape {
    static constexpr int kWaves = KIND == 1 ? MOE_MX_WIDE_WAVES1 : MOE_MX_WIDE_WAVES2;
    static constexpr int kNt = KIND == 1 ? MOE_MX_WIDE_NT1 : MOE_MX_WIDE_NT2;
};

template <int KIND, int SLAB, int RING>
hipError_t launch_mx_wide_t(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t e0,
                            hipEvent_t e1) {
    constexpr int NW = MxWideShape<KIND>::kWaves, NT = MxWideShape<KIND>::kNt;
    const long blocks = static_cast<long>(max_chunks) * a.n_tiles;
    if (blocks <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(blocks)), blk(NW * kWave);
    if (e0 || e1)
        hipExtLaunchKernelGGL((gemm_mx_wide_kernel<KIND, NW, NT, SLAB, RING>), grid, blk, 0, s, e0, e1, 0, a, k_dim);
    else
        hipLaunchKernelGGL((gemm_mx_wide_kernel<KIND, NW, NT, SLAB, RING>), grid, blk, 0, s, a, k_dim);
    return hipGetLastError();
}

// k_dim is a multiple of 256, so the 128-element step count is even: rings
// of 8, 4 or 2 steps divide it.
template <int KIND>
hipError_t launch_mx_wide(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (a.mt != 2 || k_dim % 256) return hipErrorInvalidValue;
    const int steps = k_dim / kStepK;
    if (MOE_MX_WIDE_RING == 8 && steps % 8 == 0) return launch_mx_wide_t<KIND, 4, 8>(a, max_chunks, k_dim, s, e0, e1);
    if (steps % 4 == 0) return launch_mx_wide_t<KIND, 4, 4>(a, max_chunks, k_dim, s, e0, e1);
    return launch_mx_wide_t<KIND, 2, 2>(a, max_chunks, k_dim, s, e0, e1);
}

}  // namespace

hipError_t launch_gemm1_mx(const GemmArgs &a, int max_chunks, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
    if (a.mt == 2) return launch_mx_wide<1>(a, max_chunks, a.H, s, ev_start, ev_stop);
    return launch_kind<1>(a, max_chunks, a.H, s, ev_start, ev_stop);
}

hipError_t launch_gemm2_mx(const GemmArgs &a, int max_chunks, int k_dim, hipStream_t s, hipEvent_t ev_start,
                           hipEvent_t ev_stop) {
    if (a.mt == 2) return launch_mx_wide<2>(a, max_chunks, k_dim, s, ev_start, ev_stop);
    return launch_kind<2>(a, max_chunks, k_dim, s, ev_start, ev_stop);
}

int mx_wide_tile_pairs(int kind) {
    return kind == 1 ? MxWideShape<1>::kWaves * MxWideShape<1>::kNt : MxWideShape<2>::kWaves * MxWideShape<2>::kNt;
}

}  // namespace moe
