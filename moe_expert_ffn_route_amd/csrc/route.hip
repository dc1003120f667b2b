// Dispatch grouping ("FusedDeepMoE Kernel 深度分析报告" sec. 4.1: per-expert
// token counts, their prefix sum and the expand index; sec. 5.2.1: only active
// tokens are counted; "DeepSeek V4 Decode Optimization" sec. 3.5: counters
// reused across calls must be reset per call, which this kernel does by
// rebuilding every index it owns from scratch).
//
// Block 0 of the launch routes (the other blocks quantise x); the order of
// rows is a stable counting sort keyed by (local expert, token, k), and no
// step depends on the order of atomics, so the result is deterministic. Three
// paths by the number of (token, k) pairs, all with the same outputs:
//   - at most 64 pairs (decode): one wave, no workgroup barrier (route_wave);
//   - up to 4096 pairs and 1024 tokens: the 16 waves take consecutive runs
//     of pairs, keep per-wave running counts in LDS, and meet at four
//     barriers (route_block_fast);
//   - beyond that, rounds of 1024 pairs: within a round a wave finds the
//     lanes that share its expert with ballots on the expert id's bits, ranks
//     itself with a popcount of the lower lanes, and adds the counts of the
//     lower waves and of earlier rounds (route_block).
#include "internal.h"
#include "rowquant.h"

namespace moe {
namespace {

__device__ __forceinline__ unsigned long long lanes_below(int lane) {
    return (1ull << lane) - 1ull;
}

// Exclusive scan of v over the 1024 threads of the block; returns the prefix,
// and the block total through *total. s_tmp holds kRouteWaves ints.
__device__ int block_exclusive_scan(int v, int *s_tmp, int *total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    int inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int o = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += o;
    }
    if (lane == kWave - 1) s_tmp[wave] = inc;
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < kRouteWaves; ++w) {
        int c = s_tmp[w];
        if (w < wave) before += c;
        all += c;
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

// Pairs held in registers by the routing block (rounds of kRouteThreads);
// enough for every pair at T = 512, top-8.
constexpr int kRouteRegRounds = 4;
// Routed rows whose (expert, pair) entries are collected in LDS and written
// out in row order, as coalesced stores, when P fits (a store per row at its
// scattered position would cost the one routing workgroup a cache-line write
// per row and array). Entry = expert << kStagePairBits | pair.
constexpr int kRouteStage = 4096;
constexpr int kStagePairBits = 20;
static_assert(static_cast<long>(kMaxTokens) * kMaxTopK <= (1l << kStagePairBits), "pair ids fit the entry");
static_assert(kMaxLocalExperts <= (1 << (31 - kStagePairBits)), "expert ids fit the entry");
constexpr int kPairDropped = -1;  // inactive token or expert of another rank
constexpr int kPairBad = -2;      // expert id outside [0, E_g)

// Local expert of a pair with global id `g`, or kPairDropped / kPairBad.
__device__ __forceinline__ int classify_id(const RouteArgs &a, int g, bool active) {
    if (!active) return kPairDropped;
    if (g < 0 || g >= a.E_g) return kPairBad;
    const int e = g - a.base;
    return e >= 0 && e < a.E_loc ? e : kPairDropped;
}

__device__ __forceinline__ int classify_pair(const RouteArgs &a, int p) {
    return classify_id(a, a.ids[p], !a.mask || a.mask[p / a.K]);
}

__device__ void route_block(const RouteArgs &a) {
    __shared__ int s_count[kMaxLocalExperts + 1];
    __shared__ int s_off[kMaxLocalExperts + 2];
    __shared__ int s_run[kMaxLocalExperts];
    __shared__ int s_tbl[kRouteWaves][kMaxLocalExperts];
    __shared__ int s_tmp[kRouteWaves];
    __shared__ int s_bad;
    __shared__ int s_nch;  // chunks emitted so far
    __shared__ uint32_t s_stage[kRouteStage];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int E = a.E_loc, TK = a.T * a.K;

    // 0. Every global input the routing needs, fetched at once: the first
    //    kRouteRegRounds rounds of pairs are classified into registers, and the
    //    first round of tokens' mask bits is read alongside (rounds beyond
    //    those are read again where they are used).
    int e_reg[kRouteRegRounds];
    {
        int id_v[kRouteRegRounds];
        bool act_v[kRouteRegRounds];
#pragma unroll
        for (int j = 0; j < kRouteRegRounds; ++j) {
            const int p = j * kRouteThreads + tid;
            id_v[j] = p < TK ? a.ids[p] : 0;
            act_v[j] = p < TK && (!a.mask || a.mask[p / a.K]);
        }
#pragma unroll
        for (int j = 0; j < kRouteRegRounds; ++j) e_reg[j] = classify_id(a, id_v[j], act_v[j]);
    }
    const bool tok_act0 = tid < a.T && (!a.mask || a.mask[tid]);

    // per-call reset of the arrival counters a later launch of this call
    // counts in (the workspace is never assumed to be zero)
    for (int i = tid; i < a.n_zero; i += kRouteThreads) a.zero_words[i] = 0;
    for (int i = tid; i < E; i += kRouteThreads) {
        s_count[i] = 0;
        s_run[i] = 0;
        for (int w = 0; w < kRouteWaves; ++w) s_tbl[w][i] = 0;
    }
    if (tid == 0) {
        s_bad = 0;
        s_nch = 0;
    }
    __syncthreads();

    // 1. histogram of kept pairs per local expert
    auto count = [&](int e) {
        if (e == kPairBad) atomicAdd(&s_bad, 1);
        else if (e >= 0) atomicAdd(&s_count[e], 1);
    };
#pragma unroll
    for (int j = 0; j < kRouteRegRounds; ++j) count(e_reg[j]);
    for (int p = kRouteRegRounds * kRouteThreads + tid; p < TK; p += kRouteThreads) count(classify_pair(a, p));
    __syncthreads();

    // 2. exclusive prefix sum of the counts
    {
        int total;
        const int v = tid < E ? s_count[tid] : 0;
        const int ex = block_exclusive_scan(v, s_tmp, &total);
        if (tid < E) s_off[tid] = ex;
        if (tid == 0) s_off[E] = total;
    }
    __syncthreads();
    const int P = s_off[E];
    const bool staged = P <= kRouteStage;

    // 3. stable placement, one round of 1024 pairs at a time
    auto place = [&](int base, int e) {
        const int p = base + tid;
        const bool valid = e >= 0;
        unsigned long long peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 10; ++b) {  // expert ids < 1024
            const bool bit = valid && ((e >> b) & 1);
            const unsigned long long m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const unsigned long long lower = peers & lanes_below(lane);
        const int rank = __popcll(lower);
        const int cnt = __popcll(peers);
        const bool leader = valid && lower == 0ull;
        if (leader) s_tbl[wave][e] = cnt;
        __syncthreads();
        if (p < TK) {
            if (valid) {
                int pre = 0;
                for (int w = 0; w < wave; ++w) pre += s_tbl[w][e];
                const int pos = s_off[e] + s_run[e] + pre + rank;
                a.row_of_pair[p] = pos;
                if (staged) {
                    s_stage[pos] = (static_cast<uint32_t>(e) << kStagePairBits) | static_cast<uint32_t>(p);
                } else {
                    a.sorted_pair[pos] = p;
                    a.row_token[pos] = p / a.K;
                    a.row_group[pos] = e;
                }
            } else {
                a.row_of_pair[p] = -1;
            }
        }
        __syncthreads();
        if (leader) {
            atomicAdd(&s_run[e], cnt);
            s_tbl[wave][e] = 0;
        }
        __syncthreads();
    };
#pragma unroll
    for (int j = 0; j < kRouteRegRounds; ++j)
        if (j * kRouteThreads < TK) place(j * kRouteThreads, e_reg[j]);  // uniform
    for (int base = kRouteRegRounds * kRouteThreads; base < TK; base += kRouteThreads)
        place(base, base + tid < TK ? classify_pair(a, base + tid) : kPairDropped);
    if (staged) {  // place() ends with a barrier, so every entry is in LDS
        for (int r = tid; r < P; r += kRouteThreads) {
            const uint32_t v = s_stage[r];
            const int p = static_cast<int>(v & ((1u << kStagePairBits) - 1u));
            a.sorted_pair[r] = p;
            a.row_token[r] = p / a.K;
            a.row_group[r] = static_cast<int>(v >> kStagePairBits);
        }
    }

    // 4. shared-expert rows: active tokens in token order, after the routed rows
    int t_act = 0;
    for (int base = 0; base < a.T; base += kRouteThreads) {
        const int t = base + tid;
        const bool act = base == 0 ? tok_act0 : t < a.T && (!a.mask || a.mask[t]);
        int total;
        const int ex = block_exclusive_scan(act ? 1 : 0, s_tmp, &total);
        if (act) {
            const int i = t_act + ex;
            if (a.has_shared) {
                a.row_token[P + i] = t;
                a.row_group[P + i] = E;
            }
            if (a.dbg_shared_token) a.dbg_shared_token[i] = t;
        }
        t_act += total;
    }

    // 5. GEMM work items: each group's rows cut into chunks of chunk_rows;
    //    an entry also carries the group's chunk count and its own index in it
    const int G = E + (a.has_shared ? 1 : 0);
    for (int g0 = 0; g0 < G; g0 += kRouteThreads) {
        const int g = g0 + tid;
        int M = 0, row0 = 0;
        if (g < G) {
            M = g < E ? s_count[g] : t_act;
            row0 = g < E ? s_off[g] : P;
        }
        const int nch = (M + a.chunk_rows - 1) / a.chunk_rows;
        int total;
        const int c = s_nch + block_exclusive_scan(nch, s_tmp, &total);
        for (int i = 0; i < nch; ++i) {
            const int r = i * a.chunk_rows;
            a.chunks[c + i] = make_int4(g, row0 + r, min(a.chunk_rows, M - r) | (nch << kChunkCountShift), i);
        }
        __syncthreads();
        if (tid == 0) s_nch += total;
        __syncthreads();
    }

    for (int e = tid; e < E; e += kRouteThreads) a.counts_out[e] = s_count[e];
    for (int e = tid; e <= E; e += kRouteThreads) a.offsets[e] = s_off[e];
    if (tid == 0) {
        a.offsets[E + 1] = P + t_act;
        a.meta[kMetaP] = P;
        a.meta[kMetaTAct] = t_act;
        a.meta[kMetaBad] = s_bad;
        a.meta[kMetaChunks] = s_nch;
    }
}

// Exclusive prefix sum over the 64 lanes of a wave; *total gets the sum.
__device__ __forceinline__ int wave_exclusive_scan(int v, int *total) {
    const int lane = threadIdx.x & (kWave - 1);
    int inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += o;
    }
    *total = __shfl(inc, kWave - 1, kWave);
    return inc - v;
}

// Orders one wave's LDS accesses for the compiler; the hardware performs a
// wave's LDS operations in issue order, so no barrier is needed between
// lanes of one wave.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

constexpr int kWaveExperts = (kMaxLocalExperts + kWave - 1) / kWave;  // local experts per lane

// The same routing for batches of at most 64 pairs (decode), by one wave with
// no workgroup barrier: lane p holds pair p; its rank among the pairs of its
// expert comes from ballots on the expert id's bits, the per-expert counts go
// to LDS through the first lane of each expert, and the exclusive prefixes
// over experts (row offsets, chunk indices) are wave scans over blocks of
// consecutive experts per lane. Same outputs as route_block.
__device__ void route_wave(const RouteArgs &a) {
    __shared__ int w_count[kMaxLocalExperts];
    __shared__ int w_off[kMaxLocalExperts];
    const int lane = threadIdx.x & (kWave - 1);
    const int E = a.E_loc, TK = a.T * a.K;
    const int p = lane;
    const int e = p < TK ? classify_pair(a, p) : kPairDropped;
    const bool act_tok = lane < a.T && (!a.mask || a.mask[lane]);
    for (int i = lane; i < a.n_zero; i += kWave) a.zero_words[i] = 0;
    const bool valid = e >= 0;
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 10; ++b) {  // expert ids < 1024
        const bool bit = valid && ((e >> b) & 1);
        const unsigned long long m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    const unsigned long long lower = peers & lanes_below(lane);
    const int rank = __popcll(lower);
    const int n_bad = __popcll(__ballot(e == kPairBad));
    for (int x = lane; x < E; x += kWave) w_count[x] = 0;
    wave_lds_fence();
    if (valid && lower == 0ull) w_count[e] = __popcll(peers);
    wave_lds_fence();

    // exclusive prefix of the counts (row offsets) and of the chunks per
    // expert: lane l covers experts [l * per, (l + 1) * per)
    const int per = (E + kWave - 1) / kWave;
    int cnt[kWaveExperts];
    int rsum = 0, csum = 0;
#pragma unroll
    for (int j = 0; j < kWaveExperts; ++j) {
        const int x = lane * per + j;
        cnt[j] = j < per && x < E ? w_count[x] : 0;
        rsum += cnt[j];
        csum += (cnt[j] + a.chunk_rows - 1) / a.chunk_rows;
    }
    int P, n_routed_chunks;
    int roff = wave_exclusive_scan(rsum, &P);
    int coff = wave_exclusive_scan(csum, &n_routed_chunks);
#pragma unroll
    for (int j = 0; j < kWaveExperts; ++j) {
        const int x = lane * per + j;
        if (j < per && x < E) {
            w_off[x] = roff;
            a.counts_out[x] = cnt[j];
            a.offsets[x] = roff;
            const int nch = (cnt[j] + a.chunk_rows - 1) / a.chunk_rows;
            for (int i = 0; i < nch; ++i) {
                const int r = i * a.chunk_rows;
                a.chunks[coff + i] =
                    make_int4(x, roff + r, min(a.chunk_rows, cnt[j] - r) | (nch << kChunkCountShift), i);
            }
            roff += cnt[j];
            coff += nch;
        }
    }
    wave_lds_fence();

    // rows of the kept pairs
    if (p < TK) {
        if (valid) {
            const int pos = w_off[e] + rank;
            a.row_of_pair[p] = pos;
            a.sorted_pair[pos] = p;
            a.row_token[pos] = p / a.K;
            a.row_group[pos] = e;
        } else {
            a.row_of_pair[p] = -1;
        }
    }
    // shared-expert rows: active tokens in token order, after the routed rows
    int t_act;
    const int ti = wave_exclusive_scan(act_tok ? 1 : 0, &t_act);
    if (act_tok) {
        if (a.has_shared) {
            a.row_token[P + ti] = lane;
            a.row_group[P + ti] = E;
        }
        if (a.dbg_shared_token) a.dbg_shared_token[ti] = lane;
    }
    int n_chunks = n_routed_chunks;
    if (a.has_shared) {
        const int nch = (t_act + a.chunk_rows - 1) / a.chunk_rows;
        for (int i = lane; i < nch; i += kWave) {
            const int r = i * a.chunk_rows;
            a.chunks[n_routed_chunks + i] =
                make_int4(E, P + r, min(a.chunk_rows, t_act - r) | (nch << kChunkCountShift), i);
        }
        n_chunks += nch;
    }
    if (lane == 0) {
        a.offsets[E] = P;
        a.offsets[E + 1] = P + t_act;
        a.meta[kMetaP] = P;
        a.meta[kMetaTAct] = t_act;
        a.meta[kMetaBad] = n_bad;
        a.meta[kMetaChunks] = n_chunks;
    }
}

// Exclusive scan of four values at once over the 1024 threads of the block
// (one barrier); *total gets the block sums. s_tmp holds kRouteWaves int4.
__device__ int4 block_exclusive_scan4(int4 v, int4 *s_tmp, int4 *total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    int4 inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int ox = __shfl_up(inc.x, d, kWave), oy = __shfl_up(inc.y, d, kWave);
        const int oz = __shfl_up(inc.z, d, kWave), ow = __shfl_up(inc.w, d, kWave);
        if (lane >= d) {
            inc.x += ox;
            inc.y += oy;
            inc.z += oz;
            inc.w += ow;
        }
    }
    if (lane == kWave - 1) s_tmp[wave] = inc;
    __syncthreads();
    int4 before = make_int4(0, 0, 0, 0), all = make_int4(0, 0, 0, 0);
    for (int w = 0; w < kRouteWaves; ++w) {
        const int4 c = s_tmp[w];
        if (w < wave) {
            before.x += c.x;
            before.y += c.y;
            before.z += c.z;
            before.w += c.w;
        }
        all.x += c.x;
        all.y += c.y;
        all.z += c.z;
        all.w += c.w;
    }
    *total = all;
    return make_int4(before.x + inc.x - v.x, before.y + inc.y - v.y, before.z + inc.z - v.z, before.w + inc.w - v.w);
}

constexpr int kFastRounds = 4;  // 64-pair rounds per wave: up to 4096 pairs

// The routing for 64 < T*K <= 4096 pairs and T <= 1024 tokens with four
// workgroup barriers. Wave w takes the consecutive pairs [w L, (w + 1) L)
// (L a multiple of 64), so the stable (expert, pair) order is: the pairs of
// lower waves, then this wave's earlier rounds, then the lower lanes of this
// round. Each wave keeps its running per-expert counts in a row of LDS of its
// own (a wave's LDS operations complete in issue order, so no barrier is
// needed within a wave); one pass per expert then turns the rows into
// per-wave prefixes, and one block scan of four values gives the experts' row
// offsets and chunk indices, the shared rows' positions and the count of ids
// out of range. Same outputs as route_block.
__device__ void route_block_fast(const RouteArgs &a) {
    __shared__ int f_tbl[kRouteWaves][kMaxLocalExperts];
    __shared__ int f_off[kMaxLocalExperts];
    __shared__ int4 f_tmp[kRouteWaves];
    __shared__ uint32_t f_stage[kRouteStage];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int E = a.E_loc, TK = a.T * a.K;
    const int L = (TK + kRouteThreads - 1) / kRouteThreads * kWave;  // pairs per wave
    const int rounds = L / kWave;

    int e_r[kFastRounds];
#pragma unroll
    for (int j = 0; j < kFastRounds; ++j) {
        const int p = wave * L + j * kWave + lane;
        e_r[j] = j < rounds && p < TK ? classify_pair(a, p) : kPairDropped;
    }
    const bool tok_act = tid < a.T && (!a.mask || a.mask[tid]);
    for (int i = tid; i < a.n_zero; i += kRouteThreads) a.zero_words[i] = 0;

    // 1. this wave's pairs: position among its own pairs of the same expert
    for (int x = lane; x < E; x += kWave) f_tbl[wave][x] = 0;
    wave_lds_fence();
    int pos_w[kFastRounds];
    int n_bad = 0;
#pragma unroll
    for (int j = 0; j < kFastRounds; ++j) {
        pos_w[j] = 0;
        if (j >= rounds) continue;  // uniform
        const int e = e_r[j];
        const bool valid = e >= 0;
        n_bad += e == kPairBad;
        unsigned long long peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 10; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const unsigned long long m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const unsigned long long lower = peers & lanes_below(lane);
        const int base = valid ? f_tbl[wave][e] : 0;
        wave_lds_fence();
        pos_w[j] = base + __popcll(lower);
        if (valid && lower == 0ull) f_tbl[wave][e] = base + __popcll(peers);
        wave_lds_fence();
    }
    __syncthreads();

    // 2. per expert (thread x): prefix over the waves in place, and the total
    int cnt = 0;
    if (tid < E) {
        for (int w = 0; w < kRouteWaves; ++w) {
            const int v = f_tbl[w][tid];
            f_tbl[w][tid] = cnt;
            cnt += v;
        }
    }
    const int nch = (cnt + a.chunk_rows - 1) / a.chunk_rows;
    // 3. row offsets and chunk indices of the experts, shared rows, bad ids
    int4 tot;
    const int4 ex = block_exclusive_scan4(make_int4(cnt, nch, tok_act ? 1 : 0, n_bad), f_tmp, &tot);
    const int P = tot.x, t_act = tot.z;
    if (tid < E) f_off[tid] = ex.x;
    __syncthreads();

    // 4. rows of the kept pairs, collected in LDS in row order
#pragma unroll
    for (int j = 0; j < kFastRounds; ++j) {
        const int p = wave * L + j * kWave + lane;
        if (j < rounds && p < TK) {
            const int e = e_r[j];
            if (e >= 0) {
                const int pos = f_off[e] + f_tbl[wave][e] + pos_w[j];
                a.row_of_pair[p] = pos;
                f_stage[pos] = (static_cast<uint32_t>(e) << kStagePairBits) | static_cast<uint32_t>(p);
            } else {
                a.row_of_pair[p] = -1;
            }
        }
    }
    if (tid < E) {
        a.counts_out[tid] = cnt;
        a.offsets[tid] = ex.x;
        for (int i = 0; i < nch; ++i) {
            const int r = i * a.chunk_rows;
            a.chunks[ex.y + i] = make_int4(tid, ex.x + r, min(a.chunk_rows, cnt - r) | (nch << kChunkCountShift), i);
        }
    }
    if (tok_act) {
        if (a.has_shared) {
            a.row_token[P + ex.z] = tid;
            a.row_group[P + ex.z] = E;
        }
        if (a.dbg_shared_token) a.dbg_shared_token[ex.z] = tid;
    }
    int n_chunks = tot.y;
    if (a.has_shared) {
        const int sch = (t_act + a.chunk_rows - 1) / a.chunk_rows;
        for (int i = tid; i < sch; i += kRouteThreads) {
            const int r = i * a.chunk_rows;
            a.chunks[tot.y + i] = make_int4(E, P + r, min(a.chunk_rows, t_act - r) | (sch << kChunkCountShift), i);
        }
        n_chunks += sch;
    }
    if (tid == 0) {
        a.offsets[E] = P;
        a.offsets[E + 1] = P + t_act;
        a.meta[kMetaP] = P;
        a.meta[kMetaTAct] = t_act;
        a.meta[kMetaBad] = tot.w;
        a.meta[kMetaChunks] = n_chunks;
    }
    __syncthreads();
    for (int r = tid; r < P; r += kRouteThreads) {
        const uint32_t v = f_stage[r];
        const int p = static_cast<int>(v & ((1u << kStagePairBits) - 1u));
        a.sorted_pair[r] = p;
        a.row_token[r] = p / a.K;
        a.row_group[r] = static_cast<int>(v >> kStagePairBits);
    }
}

constexpr int kTokQuantSlots = kRouteThreads / kTPR;  // rows quantised per block

// Rows the quantisation blocks of the routing launch work on: the tokens (when
// some group reads plain per-token rows), then the (token, expert) pairs (when
// expert smooth scales are given), then the tokens again (when the shared
// expert has smooth scales).
template <bool FP8, int GL>
__device__ __forceinline__ void quant_unit(const TokQuantArgs &q, int u, int slot, int tr, float *s_part) {
    const int n_tok = q.q_tok ? q.T : 0;
    const int n_pair = q.smooth ? q.T * q.K : 0;
    const uint16_t *src = q.x;
    const float *sm = nullptr;
    int8_t *dst = nullptr;
    float *scale = nullptr;
    bool active = false;
    if (u < n_tok) {
        active = !q.mask || q.mask[u];
        src += static_cast<size_t>(u) * q.H;
        dst = q.q_tok + static_cast<size_t>(u) * q.H;
        scale = q.s_tok + static_cast<size_t>(u) * q.ng;
    } else if (u < n_tok + n_pair) {
        const int p = u - n_tok, t = p / q.K;
        const int g = q.ids[p];
        const int e = g - q.base;
        // only kept pairs are read later: active token, id in range, local expert
        active = (!q.mask || q.mask[t]) && g >= 0 && g < q.E_g && e >= 0 && e < q.E_loc;
        src += static_cast<size_t>(t) * q.H;
        sm = q.smooth + static_cast<size_t>(active ? e : 0) * q.H;
        dst = q.q_sm + static_cast<size_t>(p) * q.H;
        scale = q.s_sm + static_cast<size_t>(p) * q.ng;
    } else {
        const int t = u - n_tok - n_pair;
        active = t < q.T && (!q.mask || q.mask[t]);
        src += static_cast<size_t>(active ? t : 0) * q.H;
        sm = q.share_smooth;
        const size_t row = static_cast<size_t>(q.T) * q.K + (active ? t : 0);
        dst = q.q_sm + row * q.H;
        scale = q.s_sm + row * q.ng;
    }
    quant_bf16_row<FP8, GL>(src, sm, q.H, q.eps, dst, scale, active, slot, tr, s_part);
}

__device__ __forceinline__ int quant_units(const TokQuantArgs &q) {
    return (q.q_tok ? q.T : 0) + (q.smooth ? q.T * q.K : 0) + (q.share_smooth ? q.T : 0);
}

// Block 0 routes; blocks 1.. quantise rows of x (FusedDeepMoE sec. 4.1
// quantises in dispatch). Neither job needs the other's result, so one launch
// runs both side by side. FP8: rows are quantised to E4M3 (FP4-weight
// variant) instead of INT8. GL > 0: group-wise scales, 8 * GL elements each.
template <bool FP8, int GL>
__global__ __launch_bounds__(kRouteThreads) void route_quant_kernel(RouteArgs a, TokQuantArgs q) {
    if (blockIdx.x == 0) {
        // up to 64 pairs: one wave routes, the block's other waves leave
        if (a.T * a.K <= kWave) {
            if (threadIdx.x < kWave) route_wave(a);
        } else if (a.T * a.K <= kFastRounds * kRouteThreads && a.T <= kRouteThreads) {
            route_block_fast(a);
        } else {
            route_block(a);
        }
        return;
    }
    __shared__ float s_part[kTokQuantSlots * (kTPR / kWave)];
    const int slot = threadIdx.x / kTPR, tr = threadIdx.x % kTPR;
    const int u = (blockIdx.x - 1) * kTokQuantSlots + slot;
    // units past the end take part in the block's barrier only
    if (u < quant_units(q)) {
        quant_unit<FP8, GL>(q, u, slot, tr, s_part);
    } else {
        quant_bf16_row<FP8, GL>(q.x, nullptr, q.H, q.eps, nullptr, nullptr, false, slot, tr, s_part);
    }
}

}  // namespace

hipError_t launch_route_quant(const RouteArgs &a, const TokQuantArgs &q, hipStream_t s) {
    const int units = (q.q_tok ? q.T : 0) + (q.smooth ? q.T * q.K : 0) + (q.share_smooth ? q.T : 0);
    const int qblocks = (units + kTokQuantSlots - 1) / kTokQuantSlots;
    const dim3 grid(1 + qblocks), blk(kRouteThreads);
    if (q.fp8)
        hipLaunchKernelGGL((route_quant_kernel<true, 0>), grid, blk, 0, s, a, q);
    else if (q.gl == 8)
        hipLaunchKernelGGL((route_quant_kernel<false, 8>), grid, blk, 0, s, a, q);
    else if (q.gl == 16)
        hipLaunchKernelGGL((route_quant_kernel<false, 16>), grid, blk, 0, s, a, q);
    else if (q.gl == 32)
        hipLaunchKernelGGL((route_quant_kernel<false, 32>), grid, blk, 0, s, a, q);
    else
        hipLaunchKernelGGL((route_quant_kernel<false, 0>), grid, blk, 0, s, a, q);
    return hipGetLastError();
}

}  // namespace moe
