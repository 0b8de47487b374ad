// Dynamic draft-tree kernels for gfx950: Expand (vocabulary chunks, then one
// merge per sequence that also selects the next frontier), Rerank, and flatten +
// ancestor mask + positions.
//
// Operations follow the EAGLE-2 page (news write-up of "EAGLE-2: Faster
// Inference of Language Models with Dynamic Draft Trees"): its two-stage passage
// (value = product of draft confidences on the root path, kept as an fp32 sum of
// log-confidences; Expand feeds the m best nodes of the last layer to the draft
// model and attaches its outputs as children; Rerank keeps the n best nodes of
// the whole tree, the shallower first on equal values) and the passage after it
// (flatten, ancestor-only mask, positions continuing the context).
#include "device_common.hpp"
#include "launchers.hpp"

namespace eagle {


// ---------------------------------------------------------------------------
// K1a: one workgroup per (vocabulary chunk of kChunk tokens, draft row,
// sequence); each wave owns 256 consecutive tokens of the chunk.  A wave takes its
// top-k keys (logit desc, token asc) by k rounds of a wave maximum, the round's
// owner dropping its key (no barriers), and the fp64 sum of exp(z - its max).
// Wave 0 then merges the four sorted wave lists by rank into the chunk's top-k,
// and rescales the wave sums to the chunk max.
// ---------------------------------------------------------------------------
constexpr int kChunkThreads = 256;
constexpr int kChunkWaves = kChunkThreads / kWave;
constexpr int kChunkPerLane = 4;
constexpr int kChunk = kChunkThreads * kChunkPerLane;  // 1024 tokens

__global__ __launch_bounds__(kChunkThreads) void expand_chunk_kernel(
    const float* __restrict__ logits, int V, int rows, int k, int C, uint64_t* __restrict__ ckeys,
    float* __restrict__ cmax, double* __restrict__ csum, int layer, int cap, int m,
    const int32_t* __restrict__ frontier, const float* __restrict__ value, float* __restrict__ fval_out) {
    __shared__ uint64_t s_wl[kChunkWaves][EAGLE_MAX_TOPK];  // each wave's top-k, best first
    __shared__ double s_ws[kChunkWaves];                     // each wave's sum of exp(z - wave max)
    const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
    const size_t row = (size_t)b * rows + j;
    const float* z = logits + row * (size_t)V;
    const int t0 = c * kChunk + wid * (kWave * kChunkPerLane);
    // chunk 0's workgroup also gathers the value of draft row j's frontier node for
    // the merge kernel (a dependent pair of loads, off that kernel's critical path)
    if (c == 0 && tid == 0 && layer > 1) {
        const int f = frontier[(size_t)b * m + j];
        fval_out[(size_t)b * rows + j] = value[(size_t)b * cap + f];
    }
    float zv[kChunkPerLane];
    uint64_t key[kChunkPerLane];
#pragma unroll
    for (int i = 0; i < kChunkPerLane; ++i) {
        const int t = t0 + i * kWave + lane;
        zv[i] = t < V ? z[t] : 0.0f;
        key[i] = t < V ? logit_key(zv[i], (uint32_t)t) : 0;
    }
    // this wave's top-k: lane r ends holding the r-th key (0: fewer than k tokens)
    uint64_t mine = 0;
    for (int r = 0; r < k; ++r) {
        uint64_t loc = key[0];
#pragma unroll
        for (int i = 1; i < kChunkPerLane; ++i) loc = key[i] > loc ? key[i] : loc;
        const uint64_t best = wave_max_key_u64(loc);
        if (best != 0) {
#pragma unroll
            for (int i = 0; i < kChunkPerLane; ++i)
                if (key[i] == best) key[i] = 0;  // keys are unique: one owner
        }
        if (lane == r) mine = best;
    }
    const uint64_t wtop = __shfl(mine, 0, kWave);
    double s = 0.0;
    if (wtop != 0) {
        const double wm = (double)logit_key_value(wtop);
#pragma unroll
        for (int i = 0; i < kChunkPerLane; ++i)
            if (t0 + i * kWave + lane < V) s += exp((double)zv[i] - wm);
    }
    s = wave_sum_f64(s);
    if (lane < k) s_wl[wid][lane] = mine;
    if (lane == 0) s_ws[wid] = s;
    __syncthreads();
    if (wid != 0) return;
    // merge the four sorted wave lists by rank: a key's place in the chunk's list
    // is the number of larger keys in the pool (keys are unique), the sum over the
    // four lists (each sorted, best first, zero-padded) of how many of its entries
    // are larger, found by a branch-free binary search whose steps read all four
    // lists together.  Lane l holds pool entries l and l + 64.
    const int pool = kChunkWaves * k;  // <= 128
    const uint64_t c0 = lane < pool ? s_wl[lane / k][lane % k] : 0;
    const uint64_t c1 = lane + kWave < pool ? s_wl[(lane + kWave) / k][(lane + kWave) % k] : 0;
    auto larger_in_pool = [&](uint64_t key) {
        int lo[kChunkWaves];
#pragma unroll
        for (int w = 0; w < kChunkWaves; ++w) lo[w] = 0;
#pragma unroll
        for (int step = EAGLE_MAX_TOPK; step > 0; step >>= 1) {
            if (step > k) continue;  // uniform
#pragma unroll
            for (int w = 0; w < kChunkWaves; ++w)
                if (lo[w] + step <= k && s_wl[w][lo[w] + step - 1] > key) lo[w] += step;
        }
        return lo[0] + lo[1] + lo[2] + lo[3];
    };
    static_assert(kChunkWaves == 4, "four wave lists");
    const int r0 = c0 != 0 ? larger_in_pool(c0) : 2 * kWave;
    const int r1 = c1 != 0 ? larger_in_pool(c1) : 2 * kWave;
    const int nz = __popcll(__ballot(c0 != 0)) + __popcll(__ballot(c1 != 0));
    uint64_t* out = ckeys + (row * C + c) * (size_t)k;
    if (c0 != 0 && r0 < k) out[r0] = c0;
    if (c1 != 0 && r1 < k) out[r1] = c1;
    if (lane >= nz && lane < k) out[lane] = 0;  // fewer than k tokens in the chunk
    // chunk max = the top key's logit; chunk sum = sum over waves of
    // (wave sum) * exp(wave max - chunk max), all in fp64
    uint64_t top = s_wl[0][0];
#pragma unroll
    for (int w = 1; w < kChunkWaves; ++w) top = s_wl[w][0] > top ? s_wl[w][0] : top;
    double part = 0.0;
    if (lane < kChunkWaves && top != 0) {
        const uint64_t wk = s_wl[lane][0];
        if (wk != 0) part = s_ws[lane] * exp((double)logit_key_value(wk) - (double)logit_key_value(top));
    }
    part = wave_sum_f64(part);
    if (lane == 0) {
        cmax[row * C + c] = top != 0 ? logit_key_value(top) : 0.0f;
        csum[row * C + c] = part;
    }
}

// ---------------------------------------------------------------------------
// K1b: one workgroup per sequence.  One wave per draft row merges the row's C
// sorted chunk lists (head pointers over an LDS copy) into its top-k, forms
// lse = log(sum_c csum_c * exp(cmax_c - max)) in fp64 rounded once to fp32, and
// writes the k children at ids base + j*k + rank.  Then, below the last layer,
// the new layer's nodes are sorted by (value desc, id asc) in LDS and the first
// min(m, layer size) become the next frontier.  Advances n_nodes.
// ---------------------------------------------------------------------------
constexpr int kFinishThreads = 1024;
constexpr int kFinishWaves = kFinishThreads / kWave;
constexpr int kMergeLdsKeys = 8192;  // 64 KB of chunk lists per pass
constexpr int kMaxChunkHeads = 4;    // chunk lists per lane: C <= 256
constexpr int kFrontierRounds = 32;  // up to this many frontier nodes: one wave selects them
constexpr int kCopyBatch = 8;       // chunk-list loads per lane in flight together
static_assert((EAGLE_MAX_VOCAB + kChunk - 1) / kChunk <= kMaxChunkHeads * kWave, "chunk lists per lane");
static_assert(((EAGLE_MAX_VOCAB + kChunk - 1) / kChunk) * EAGLE_MAX_TOPK <= kMergeLdsKeys, "one row's lists fit");

// A draft row's top-k by k rounds of a wave maximum over the heads of its sorted
// chunk lists in LDS; lane q owns chunks q, q + 64, ... (NH of them).  Lane r ends
// holding the r-th key.
template <int NH>
__device__ __forceinline__ uint64_t merge_chunk_lists(const uint64_t* lists, int C, int k, int lane) {
    int pos[NH];
    uint64_t h[NH], nx[NH];  // head and the entry after it (read ahead, so an advance waits on no LDS read)
#pragma unroll
    for (int u = 0; u < NH; ++u) {
        pos[u] = 0;
        const bool own = lane + u * kWave < C;
        h[u] = own ? lists[(lane + u * kWave) * k] : 0;
        nx[u] = own && k > 1 ? lists[(lane + u * kWave) * k + 1] : 0;
    }
    uint64_t mykey = 0;
    for (int r = 0; r < k; ++r) {
        uint64_t loc = h[0];
#pragma unroll
        for (int u = 1; u < NH; ++u) loc = h[u] > loc ? h[u] : loc;
        const uint64_t best = wave_max_key_u64(loc);
#pragma unroll
        for (int u = 0; u < NH; ++u)
            if (best != 0 && h[u] == best) {  // keys are unique: one owner, which moves to its next key
                ++pos[u];
                h[u] = nx[u];
                nx[u] = pos[u] + 1 < k ? lists[(lane + u * kWave) * k + pos[u] + 1] : 0;
            }
        if (lane == r) mykey = best;
    }
    return mykey;
}

// The first `keep` of L candidate keys (held NQ per lane, lane + 64 q) by that many
// rounds of a wave maximum; lane r ends holding the r-th.
template <int NQ>
__device__ __forceinline__ uint64_t select_top(uint64_t (&cand)[NQ], int keep, int lane) {
    uint64_t pick = 0;
    for (int r = 0; r < keep; ++r) {
        uint64_t loc = cand[0];
#pragma unroll
        for (int q = 1; q < NQ; ++q) loc = cand[q] > loc ? cand[q] : loc;
        const uint64_t best = wave_max_key_u64(loc);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            if (cand[q] == best) cand[q] = 0;  // keys are unique: one owner
        if (lane == r) pick = best;
    }
    return pick;
}

template <int NQ>
__device__ __forceinline__ uint64_t frontier_pick(const float* s_val, int L, int base, int keep, int lane) {
    uint64_t cand[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i = lane + q * kWave;
        cand[q] = i < L ? ((uint64_t)float_order_key(s_val[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(base + i))
                        : 0;
    }
    return select_top<NQ>(cand, keep, lane);
}

// The first `keep` of L <= kRankNodes new nodes by rank: eight threads per node count
// the keys above it (keys are unique, so ranks are distinct) and the node of rank r
// lands in frontier slot r.  All threads of the workgroup take part.
constexpr int kRankNodes = kFinishThreads / 8;
__device__ __forceinline__ void frontier_by_rank(const float* s_val, int L, int base, int keep, int tid,
                                                 int32_t* __restrict__ frontier_out) {
    const int i = tid >> 3, part = tid & 7;
    auto key_of = [&](int x) {
        return ((uint64_t)float_order_key(s_val[x]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(base + x));
    };
    const uint64_t mine = i < L ? key_of(i) : 0;
    uint32_t above = 0;
    for (int x = part; x < L; x += 8) above += key_of(x) > mine;
    above += dpp_u32<kDppXor1>(above);        // the eight counts of node i sit in
    above += dpp_u32<kDppXor2>(above);        // lanes 8q .. 8q + 7 of one row
    above += dpp_u32<kDppHalfMirror>(above);
    if (part == 0 && i < L && (int)above < keep) frontier_out[above] = base + i;
}

__global__ __launch_bounds__(kFinishThreads) void expand_finish_kernel(
    int rows, int k, int C, int layer, int depth_total, const uint64_t* __restrict__ ckeys,
    const float* __restrict__ cmax, const double* __restrict__ csum,
    const int32_t* __restrict__ root_token, const float* __restrict__ fval_in, int cap, int m,
    int32_t* __restrict__ token,
    int32_t* __restrict__ parent, int32_t* __restrict__ depth, float* __restrict__ value,
    int32_t* __restrict__ frontier, int32_t* __restrict__ n_nodes) {
    __shared__ uint64_t lists[kMergeLdsKeys];
    __shared__ uint64_t fkeys[EAGLE_MAX_LAYER_NODES];
    __shared__ float s_val[EAGLE_MAX_LAYER_NODES];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
    const int base = (layer == 1) ? 1 : n_nodes[b];
    const int L = rows * k;
    const int per_row = C * k;
    int waves = kMergeLdsKeys / per_row;  // rows merged at once
    if (waves > kFinishWaves) waves = kFinishWaves;

    if (layer == 1 && tid == 0) {
        const size_t r0 = (size_t)b * cap;
        token[r0] = root_token[b];
        parent[r0] = -1;
        depth[r0] = 0;
        value[r0] = 0.0f;
    }
    for (int j0 = 0; j0 < rows; j0 += waves) {
        const int j = j0 + wid;
        const bool active = wid < waves && j < rows;
        uint64_t* mine = lists + wid * per_row;
        const size_t row = (size_t)b * rows + j;
        // everything this row needs from memory is requested before the merge:
        // its chunk lists, chunk maxima and sums, its frontier node and that node's value
        double cs[kMaxChunkHeads];
        float cm[kMaxChunkHeads];
        int f = 0;
        float fval = 0.0f;
        if (active) {
#pragma unroll
            for (int u = 0; u < kMaxChunkHeads; ++u) {
                const int cu = lane + u * kWave;
                cs[u] = cu < C ? csum[row * C + cu] : 0.0;
                cm[u] = cu < C ? cmax[row * C + cu] : 0.0f;
            }
            if (layer != 1) {
                f = frontier[(size_t)b * m + j];
                fval = fval_in[(size_t)b * rows + j];
            }
            // the lists: a batch of loads in flight before any LDS store (a load-store
            // loop would pay one memory round trip per 64 keys)
            for (int i0 = lane; i0 < per_row; i0 += kCopyBatch * kWave) {
                uint64_t t[kCopyBatch];
#pragma unroll
                for (int q = 0; q < kCopyBatch; ++q) {
                    const int i = i0 + q * kWave;
                    t[q] = i < per_row ? ckeys[row * per_row + i] : 0;
                }
#pragma unroll
                for (int q = 0; q < kCopyBatch; ++q) {
                    const int i = i0 + q * kWave;
                    if (i < per_row) mine[i] = t[q];
                }
            }
        }
        __syncthreads();
        if (active) {
            const uint64_t mykey = C <= kWave       ? merge_chunk_lists<1>(mine, C, k, lane)
                                   : C <= 2 * kWave ? merge_chunk_lists<2>(mine, C, k, lane)
                                                    : merge_chunk_lists<4>(mine, C, k, lane);
            const uint64_t top = __shfl(mykey, 0, kWave);
            const float row_max = logit_key_value(top);
            double s = 0.0;
#pragma unroll
            for (int u = 0; u < kMaxChunkHeads; ++u)
                if (lane + u * kWave < C) s += cs[u] * exp((double)cm[u] - (double)row_max);
            s = wave_sum_f64(s);
            const float lse32 = (float)log(s);
            if (lane < k) {
                const uint32_t tok = logit_key_token(mykey);
                const float shifted = logit_key_value(mykey) - row_max;  // fp32
                const float logq = shifted - lse32;                      // fp32
                const float val = fval + logq;                           // fp32
                const size_t idx = (size_t)b * cap + base + (size_t)j * k + lane;
                token[idx] = (int32_t)tok;
                parent[idx] = f;
                depth[idx] = layer;
                value[idx] = val;
                s_val[j * k + lane] = val;
            }
        }
        // the lists area is reused by the next pass and s_val is read below; every
        // frontier entry of this pass was read (its parent ids are in the stores)
        barrier_lds();
    }
    if (layer < depth_total && L <= kRankNodes) {
        frontier_by_rank(s_val, L, base, L < m ? L : m, tid, frontier + (size_t)b * m);
    } else if (layer < depth_total && (L < m ? L : m) <= kFrontierRounds) {
        // frontier = the first min(m, L) new nodes in (value desc, id asc): by that
        // many rounds of a wave maximum over the layer
        if (wid == 0) {
            const int keep = L < m ? L : m;
            const uint64_t pick = L <= 2 * kWave ? frontier_pick<2>(s_val, L, base, keep, lane)
                                                 : frontier_pick<EAGLE_MAX_LAYER_NODES / kWave>(s_val, L, base, keep, lane);
            if (lane < keep) frontier[(size_t)b * m + lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)(pick & 0xFFFFFFFFu));
        }
    } else if (layer < depth_total) {
        const int P = next_pow2(L);
        for (int i = tid; i < P; i += kFinishThreads) {
            uint64_t key = 0;
            if (i < L) {
                const uint32_t id = (uint32_t)(base + i);
                key = ((uint64_t)float_order_key(s_val[i]) << 32) | (uint64_t)(0xFFFFFFFFu - id);
            }
            fkeys[i] = key;
        }
        __syncthreads();
        lds_bitonic_sort_desc(fkeys, P);
        const int keep = L < m ? L : m;
        for (int i = tid; i < keep; i += kFinishThreads)
            frontier[(size_t)b * m + i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(fkeys[i] & 0xFFFFFFFFu));
    }
    if (tid == 0) n_nodes[b] = base + L;
}

// ---------------------------------------------------------------------------
// K3: per sequence, the n first non-root nodes in (value desc, depth asc, id asc),
// written in ascending id.  Node keys pack the three into one unique 64-bit
// value, larger = earlier.  Up to kRankMax candidates (one per thread): the n-th
// largest key is found by an 8-pass radix select (8-bit digits from the top, an
// LDS histogram per pass), the n nodes whose keys are at least that are kept, and
// a kept node's output slot is the number of kept nodes with a smaller id (a
// block prefix count of ballots).  Larger trees: one LDS bitonic sort, then the n first ids sorted
// again ascending.
// ---------------------------------------------------------------------------
constexpr int kRankMax = 1024;  // a multiple of 16, at most EAGLE_MAX_CAPACITY / 2
static_assert(kRankMax % 16 == 0 && 2 * kRankMax <= EAGLE_MAX_CAPACITY, "rank path layout");

__device__ __forceinline__ uint64_t rerank_key(const float* value, const int32_t* depth, int b, int cap, int id) {
    const uint32_t dep = (uint32_t)depth[(size_t)b * cap + id];
    return ((uint64_t)float_order_key(value[(size_t)b * cap + id]) << 32) | ((uint64_t)(255u - dep) << 24) |
           (uint64_t)(0xFFFFFFu - (uint32_t)id);
}

__global__ __launch_bounds__(1024) void rerank_kernel(int cap, int n, const float* __restrict__ value,
                                                       const int32_t* __restrict__ depth,
                                                       int32_t* __restrict__ kept) {
    __shared__ __attribute__((aligned(16))) uint64_t keys[EAGLE_MAX_CAPACITY];
    __shared__ uint64_t sel[EAGLE_MAX_TREE_ROWS];
    __shared__ int s_wave_kept[1024 / kWave];
    __shared__ int s_pick[2];  // radix select: chosen digit, remaining rank
    const int b = blockIdx.x, tid = threadIdx.x;
    const int N = cap - 1;
    if (N <= kRankMax) {
        const int lane = tid & (kWave - 1), wid = tid / kWave;
        const uint64_t mine = tid < N ? rerank_key(value, depth, b, cap, tid + 1) : 0;  // real keys are > 0
        // radix select of the n-th largest key, 8 bits a pass from the top: each pass
        // counts the candidates (keys agreeing with the digits chosen so far) per next
        // digit, and wave 0 picks the digit holding the remaining rank
        uint32_t* hist = reinterpret_cast<uint32_t*>(keys);  // two 256-bin histograms
        for (int i = tid; i < 512; i += blockDim.x) hist[i] = 0;
        __syncthreads();
        uint64_t prefix = 0;
        int need = n;  // rank (from the top, 1-based) of the wanted key among the candidates
        for (int pass = 0; pass < 8; ++pass) {
            const int shift = 56 - 8 * pass;
            uint32_t* h = hist + 256 * (pass & 1);
            const bool cand = tid < N && (pass == 0 || (mine >> (shift + 8)) == (prefix >> (shift + 8)));
            if (cand) atomicAdd(&h[(mine >> shift) & 255u], 1u);
            __syncthreads();
            if (wid == 0) {
                uint32_t c[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) c[u] = h[4 * lane + u];
                const uint32_t tot = c[0] + c[1] + c[2] + c[3];
                // keys in the bins above this lane's four: suffix sum over the lanes above
                uint32_t above = 0, run = tot;
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) {
                    const uint32_t o = __shfl_down(run, off, kWave);
                    if (lane + off < kWave) run += o;
                }
                above = run - tot;
#pragma unroll
                for (int u = 3; u >= 0; --u) {
                    if ((int)above < need && (int)(above + c[u]) >= need) {
                        s_pick[0] = 4 * lane + u;
                        s_pick[1] = need - (int)above;
                    }
                    above += c[u];
                }
                // the other histogram is cleared for the next pass
                uint32_t* hn = hist + 256 * ((pass + 1) & 1);
#pragma unroll
                for (int u = 0; u < 4; ++u) hn[4 * lane + u] = 0;
            }
            __syncthreads();
            prefix |= (uint64_t)(uint32_t)s_pick[0] << shift;
            need = s_pick[1];
        }
        // keys are unique: exactly n of them are >= the n-th largest
        const bool keep = tid < N && mine >= prefix;
        const uint64_t bal = __ballot(keep);
        if (lane == 0) s_wave_kept[wid] = __popcll(bal);
        __syncthreads();
        int before = __popcll(bal & ((1ull << lane) - 1ull));
        for (int w = 0; w < wid; ++w) before += s_wave_kept[w];
        if (keep) kept[(size_t)b * n + before] = tid + 1;
        return;
    }
    const int P = next_pow2(N);
    for (int i = tid; i < P; i += blockDim.x) keys[i] = i < N ? rerank_key(value, depth, b, cap, i + 1) : 0;
    __syncthreads();
    lds_bitonic_sort_desc(keys, P);
    const int P2 = next_pow2(n > 0 ? n : 1);
    for (int i = tid; i < P2; i += blockDim.x) {
        uint64_t key = 0;
        if (i < n) {
            const uint32_t id = 0xFFFFFFu - (uint32_t)(keys[i] & 0xFFFFFFu);
            key = (uint64_t)(0xFFFFFFFFu - id);
        }
        sel[i] = key;
    }
    __syncthreads();
    lds_bitonic_sort_desc(sel, P2);
    for (int i = tid; i < n; i += blockDim.x)
        kept[(size_t)b * n + i] = (int32_t)(0xFFFFFFFFu - (uint32_t)sel[i]);
}

// ---------------------------------------------------------------------------
// K4: one wave per sequence; lane i owns flattened row i.  Parent rows come from
// a node -> row table in LDS; the ancestor mask is built by walking parent rows,
// at most T steps.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void mask_kernel(int cap, int n, const int32_t* __restrict__ token,
                                                   const int32_t* __restrict__ parent,
                                                   const int32_t* __restrict__ depth,
                                                   const int32_t* __restrict__ kept,
                                                   const int32_t* __restrict__ ctx_len,
                                                   int32_t* __restrict__ flat_token,
                                                   int32_t* __restrict__ flat_parent,
                                                   int32_t* __restrict__ flat_depth,
                                                   int32_t* __restrict__ position,
                                                   uint64_t* __restrict__ mask) {
    __shared__ int32_t fnode[EAGLE_MAX_TREE_ROWS];
    __shared__ int32_t fpar[EAGLE_MAX_TREE_ROWS];
    __shared__ int16_t row_of[EAGLE_MAX_CAPACITY];  // node -> flattened row, kept nodes only
    const int b = blockIdx.x, i = threadIdx.x;
    const int T = n + 1;
    int node = 0, p = -1;
    if (i < T) {
        node = (i == 0) ? 0 : kept[(size_t)b * n + (i - 1)];
        if (node < 0 || node >= cap) node = 0;  // not a node id: memory-safe, result unspecified
        p = parent[(size_t)b * cap + node];
        fnode[i] = node;
        row_of[node] = (int16_t)i;
    }
    __syncthreads();
    // The kept set is ancestor-closed, so a kept node's parent has its entry; the
    // entry is checked against the row's node so a stale one reads as no parent.
    if (i < T) {
        int pr = p >= 0 && p < cap ? row_of[p] : -1;
        if (pr < 0 || pr >= T || fnode[pr] != p) pr = -1;
        fpar[i] = pr;
    }
    __syncthreads();
    if (i < T) {
        uint64_t bits = 0;
        int r = i;
        for (int steps = 0; r >= 0 && steps < T; ++steps) {
            bits |= 1ull << r;
            r = fpar[r];
        }
        const size_t o = (size_t)b * T + i;
        const int dep = depth[(size_t)b * cap + node];
        flat_token[o] = token[(size_t)b * cap + node];
        flat_parent[o] = fpar[i];
        flat_depth[o] = dep;
        position[o] = ctx_len[b] + dep;
        mask[o] = bits;
    }
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
// Expand workspace: per (sequence, draft row, chunk) the chunk's k keys, its max
// logit and its fp64 exp sum; per (sequence, draft row) the frontier node's value;
// draft rows <= m.
struct ExpandWs {
    size_t keys, max, sum, fval, total;
};
static ExpandWs expand_ws(const eagle_tree_cfg& cfg) {
    const size_t C = (size_t)expand_chunks(cfg.vocab);
    const size_t cells = (size_t)cfg.batch * (size_t)(cfg.m > 0 ? cfg.m : 1) * C;
    ExpandWs w;
    w.keys = 0;
    w.max = (cells * (size_t)cfg.topk * 8 + 255) & ~(size_t)255;
    w.sum = w.max + ((cells * 4 + 255) & ~(size_t)255);
    w.fval = w.sum + ((cells * 8 + 255) & ~(size_t)255);
    w.total = w.fval + (size_t)cfg.batch * (size_t)(cfg.m > 0 ? cfg.m : 1) * 4;
    return w;
}

int expand_chunks(int vocab) { return (vocab + kChunk - 1) / kChunk; }
size_t expand_workspace_bytes(const eagle_tree_cfg& cfg) { return expand_ws(cfg).total; }

hipError_t launch_expand(const eagle_tree_cfg& cfg, int layer, int rows, int cap,
                         const float* logits, const int32_t* root_token,
                         const eagle_tree_state& st, void* workspace, hipStream_t stream) {
    const int C = expand_chunks(cfg.vocab), k = cfg.topk;
    const ExpandWs w = expand_ws(cfg);
    unsigned char* ws = (unsigned char*)workspace;
    uint64_t* ckeys = (uint64_t*)(ws + w.keys);
    float* cmax = (float*)(ws + w.max);
    double* csum = (double*)(ws + w.sum);
    float* fval = (float*)(ws + w.fval);
    expand_chunk_kernel<<<dim3(C, rows, cfg.batch), kChunkThreads, 0, stream>>>(
        logits, cfg.vocab, rows, k, C, ckeys, cmax, csum, layer, cap, cfg.m, st.frontier, st.value, fval);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    expand_finish_kernel<<<cfg.batch, kFinishThreads, 0, stream>>>(
        rows, k, C, layer, cfg.depth, ckeys, cmax, csum, root_token, fval, cap, cfg.m, st.token, st.parent,
        st.depth, st.value, st.frontier, st.n_nodes);
    return hipGetLastError();
}

hipError_t launch_rerank(const eagle_tree_cfg& cfg, int cap, const eagle_tree_state& st,
                         int32_t* kept, hipStream_t stream) {
    rerank_kernel<<<cfg.batch, 1024, 0, stream>>>(cap, cfg.n, st.value, st.depth, kept);
    return hipGetLastError();
}

hipError_t launch_mask(const eagle_tree_cfg& cfg, int cap, const eagle_tree_state& st,
                       const int32_t* kept, const int32_t* ctx_len, int32_t* flat_token,
                       int32_t* flat_parent, int32_t* flat_depth, int32_t* position,
                       uint64_t* mask, hipStream_t stream) {
    mask_kernel<<<cfg.batch, 64, 0, stream>>>(cap, cfg.n, st.token, st.parent, st.depth, kept,
                                              ctx_len, flat_token, flat_parent, flat_depth,
                                              position, mask);
    return hipGetLastError();
}

}  // namespace eagle
