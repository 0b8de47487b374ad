// Dynamic draft-tree kernels for gfx950: Expand (per draft row and per layer),
// Rerank, and flatten + ancestor mask + positions.
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
// K1: one workgroup per (draft row, sequence).  Pass 1 keeps each thread's best
// KCAP (logit, token) keys in registers; every wave then emits its top-k by k
// rounds of wave-wide maxima; the waves' lists are merged by an LDS bitonic sort.
// Pass 2 sums exp(z - zmax) in fp64 (zmax = best key's logit) and rounds the
// log once to fp32.  The k children are written at ids base + j*k + rank.
// ---------------------------------------------------------------------------
constexpr int kExpandThreads = 1024;
constexpr int kExpandWaves = kExpandThreads / kWave;

template <int KCAP>
__global__ __launch_bounds__(kExpandThreads) void expand_rows_kernel(
    const float* __restrict__ logits, int V, int rows, int k, int layer,
    const int32_t* __restrict__ root_token, int cap, int m, int32_t* __restrict__ token,
    int32_t* __restrict__ parent, int32_t* __restrict__ depth, float* __restrict__ value,
    const int32_t* __restrict__ frontier, const int32_t* __restrict__ n_nodes) {
    constexpr int P = kExpandWaves * KCAP;  // power of two
    __shared__ uint64_t cand[P];
    __shared__ double red[kExpandWaves];
    __shared__ float s_lse32;

    const int j = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
    const float* z = logits + ((size_t)b * rows + j) * (size_t)V;
    const int f = (layer == 1) ? 0 : frontier[(size_t)b * m + j];
    const int base = (layer == 1) ? 1 : n_nodes[b];
    const float fval = (layer == 1) ? 0.0f : value[(size_t)b * cap + f];

    // Pass 1: per-thread sorted (descending) top-KCAP keys; 0 marks an empty slot.
    uint64_t list[KCAP];
#pragma unroll
    for (int i = 0; i < KCAP; ++i) list[i] = 0;
    for (int t = tid; t < V; t += kExpandThreads) {
        const uint64_t key = logit_key(z[t], (uint32_t)t);
        if (key > list[KCAP - 1]) {
            list[KCAP - 1] = key;
#pragma unroll
            for (int i = KCAP - 1; i > 0; --i) {
                if (list[i] > list[i - 1]) {
                    const uint64_t x = list[i];
                    list[i] = list[i - 1];
                    list[i - 1] = x;
                }
            }
        }
    }
    // Wave stage: k rounds of the wave maximum; the winning lane pops its head.
    for (int r = 0; r < KCAP; ++r) {
        uint64_t best = 0;
        if (r < k) {
            best = wave_max_u64(list[0]);
            if (best != 0 && list[0] == best) {
#pragma unroll
                for (int i = 0; i < KCAP - 1; ++i) list[i] = list[i + 1];
                list[KCAP - 1] = 0;
            }
        }
        if (lane == 0) cand[wid * KCAP + r] = best;
    }
    __syncthreads();
    lds_bitonic_sort_desc(cand, P);  // cand[0..k-1]: the row's top-k

    // Pass 2: fp64 normaliser from the row maximum (the best key's logit).
    const uint32_t top_tok = logit_key_token(cand[0]);
    const float row_max = z[top_tok];
    double s = 0.0;
    for (int t = tid; t < V; t += kExpandThreads) s += exp((double)z[t] - (double)row_max);
    s = block_sum_f64(s, red);
    if (tid == 0) s_lse32 = (float)log(s);
    __syncthreads();

    if (layer == 1 && j == 0 && tid == 0) {
        const size_t r0 = (size_t)b * cap;
        token[r0] = root_token[b];
        parent[r0] = -1;
        depth[r0] = 0;
        value[r0] = 0.0f;
    }
    if (tid < k) {
        const uint32_t tok = logit_key_token(cand[tid]);
        const float shifted = z[tok] - row_max;  // fp32
        const float logq = shifted - s_lse32;    // fp32
        const float val = fval + logq;           // fp32
        const size_t idx = (size_t)b * cap + base + (size_t)j * k + tid;
        token[idx] = (int32_t)tok;
        parent[idx] = f;
        depth[idx] = layer;
        value[idx] = val;
    }
}

// ---------------------------------------------------------------------------
// K2: per sequence, the new layer's nodes sorted by (value desc, id asc) in LDS;
// the first min(m, layer size) become the next frontier.  Advances n_nodes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void frontier_kernel(int layer, int depth_total, int rows, int k,
                                                         int m, int cap,
                                                         const float* __restrict__ value,
                                                         int32_t* __restrict__ frontier,
                                                         int32_t* __restrict__ n_nodes) {
    __shared__ uint64_t keys[EAGLE_MAX_LAYER_NODES];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int base = (layer == 1) ? 1 : n_nodes[b];
    const int L = rows * k;
    if (layer < depth_total) {
        const int P = next_pow2(L);
        for (int i = tid; i < P; i += blockDim.x) {
            uint64_t key = 0;
            if (i < L) {
                const uint32_t id = (uint32_t)(base + i);
                key = ((uint64_t)float_order_key(value[(size_t)b * cap + id]) << 32) |
                      (uint64_t)(0xFFFFFFFFu - id);
            }
            keys[i] = key;
        }
        __syncthreads();
        lds_bitonic_sort_desc(keys, P);
        const int keep = L < m ? L : m;
        for (int i = tid; i < keep; i += blockDim.x)
            frontier[(size_t)b * m + i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(keys[i] & 0xFFFFFFFFu));
    }
    __syncthreads();
    if (tid == 0) n_nodes[b] = base + L;
}

// ---------------------------------------------------------------------------
// K3: per sequence, all non-root nodes sorted by (value desc, depth asc, id asc)
// with one LDS bitonic sort; the first n ids are sorted again ascending.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void rerank_kernel(int cap, int n, const float* __restrict__ value,
                                                       const int32_t* __restrict__ depth,
                                                       int32_t* __restrict__ kept) {
    __shared__ uint64_t keys[EAGLE_MAX_CAPACITY];
    __shared__ uint64_t sel[EAGLE_MAX_TREE_ROWS];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int N = cap - 1;
    const int P = next_pow2(N);
    for (int i = tid; i < P; i += blockDim.x) {
        uint64_t key = 0;
        if (i < N) {
            const uint32_t id = (uint32_t)(i + 1);
            const uint32_t dep = (uint32_t)depth[(size_t)b * cap + id];
            key = ((uint64_t)float_order_key(value[(size_t)b * cap + id]) << 32) |
                  ((uint64_t)(255u - dep) << 24) | (uint64_t)(0xFFFFFFu - id);
        }
        keys[i] = key;
    }
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
// K4: one wave per sequence; lane i owns flattened row i.  Parent rows are found
// among the (ascending) kept ids; the ancestor mask is built by walking parent
// rows, at most T steps.
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
    const int b = blockIdx.x, i = threadIdx.x;
    const int T = n + 1;
    if (i < T) fnode[i] = (i == 0) ? 0 : kept[(size_t)b * n + (i - 1)];
    __syncthreads();
    int node = 0;
    if (i < T) {
        node = fnode[i];
        const int p = parent[(size_t)b * cap + node];
        int pr = -1;
        if (p >= 0) {
            for (int r = 0; r < T; ++r)
                if (fnode[r] == p) { pr = r; break; }
        }
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
hipError_t launch_expand(const eagle_tree_cfg& cfg, int layer, int rows, int cap,
                         const float* logits, const int32_t* root_token,
                         const eagle_tree_state& st, hipStream_t stream) {
    const dim3 grid(rows, cfg.batch);
    const int k = cfg.topk;
    if (k <= 8) {
        expand_rows_kernel<8><<<grid, kExpandThreads, 0, stream>>>(
            logits, cfg.vocab, rows, k, layer, root_token, cap, cfg.m, st.token, st.parent,
            st.depth, st.value, st.frontier, st.n_nodes);
    } else if (k <= 16) {
        expand_rows_kernel<16><<<grid, kExpandThreads, 0, stream>>>(
            logits, cfg.vocab, rows, k, layer, root_token, cap, cfg.m, st.token, st.parent,
            st.depth, st.value, st.frontier, st.n_nodes);
    } else {
        expand_rows_kernel<32><<<grid, kExpandThreads, 0, stream>>>(
            logits, cfg.vocab, rows, k, layer, root_token, cap, cfg.m, st.token, st.parent,
            st.depth, st.value, st.frontier, st.n_nodes);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    frontier_kernel<<<cfg.batch, 1024, 0, stream>>>(layer, cfg.depth, rows, k, cfg.m, cap, st.value,
                                                    st.frontier, st.n_nodes);
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
