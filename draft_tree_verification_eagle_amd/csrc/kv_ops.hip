// Kernels around the verification step: the mask of a caller-given static tree,
// rotary position encoding of the tree rows at their positions, the KV commit of
// the accepted path, the rows of the draft-side attention and a row gather into
// the KV cache.  All are small (tens of KB to a few MB per call) and
// latency-bound; each is one launch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.hpp"
#include "launchers.hpp"

namespace eagle {
namespace {

// ---------------------------------------------------------------------------
// Static tree: one wave per sequence, lane i = row i.  Row i's ancestors are
// found by walking parent links; a walk that meets a parent entry which is not an
// earlier row (or a root entry other than -1) marks the row invalid.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void mask_static_kernel(int T, const int32_t* __restrict__ flat_parent,
                                                         const int32_t* __restrict__ ctx_len,
                                                         int32_t* __restrict__ flat_depth,
                                                         int32_t* __restrict__ position,
                                                         uint64_t* __restrict__ mask) {
    __shared__ int32_t par[EAGLE_MAX_TREE_ROWS];
    const int b = blockIdx.x, i = threadIdx.x;
    if (i < T) par[i] = flat_parent[(size_t)b * T + i];
    __syncthreads();
    if (i >= T) return;
    uint64_t bits = 0;
    int depth = 0;
    bool ok = true;
    int r = i;
    // each step moves to a strictly earlier row, so the walk ends within T steps
    while (true) {
        bits |= 1ull << r;
        const int p = par[r];
        if (r == 0) {
            ok = (p == -1);
            break;
        }
        if (p < 0 || p >= r) {
            ok = false;
            break;
        }
        r = p;
        ++depth;
    }
    const size_t o = (size_t)b * T + i;
    flat_depth[o] = ok ? depth : -1;
    position[o] = ok ? ctx_len[b] + depth : -1;
    mask[o] = ok ? bits : 0ull;
}

// ---------------------------------------------------------------------------
// Rotary position encoding of the tree rows.  One workgroup per (tree row,
// sequence, slice of kRopeHeads heads), the query heads of the row followed by
// the KV heads' tree row.  Thread t takes coordinate pair d = t mod (D/2) of every
// (256 / (D/2))-th head of the slice: it computes the pair's angle, cosine and
// sine once (fp64) and rotates that pair in each of its heads; consecutive threads
// take consecutive coordinates, so each head row is read and written in
// coalesced sweeps.  The frequencies base^(-2d/D) arrive as launch arguments,
// computed once on the host.
// ---------------------------------------------------------------------------
constexpr int kRopeHeads = 16;

__device__ __forceinline__ double load_elt(const float* p) { return (double)*p; }
__device__ __forceinline__ double load_elt(const uint16_t* p) {
    return (double)__uint_as_float((uint32_t)*p << 16);
}
__device__ __forceinline__ void store_elt(float* p, float x) { *p = x; }
__device__ __forceinline__ void store_elt(uint16_t* p, float x) { *p = bf16_bits_rne(x); }

constexpr int kRopeHostRows = 32;  // sequences whose K row may ride in the launch arguments

struct RopeArgs {
    double f[128];                     // base^(-2d/D), d < D/2
    int64_t k_row0[kRopeHostRows];     // kv_row_off[b] + ctx_len[b], when the host has them
};

// Every load a thread needs is issued before it waits for any: the position of
// its row and both halves of its coordinate pair in each of its heads, so one
// memory round trip covers the kernel.
template <typename Elt, bool HOST_ROWS>
__global__ __launch_bounds__(256) void rope_kernel(int T, int Hq, int Hkv, int D,
                                                   const int32_t* __restrict__ position,
                                                   const int32_t* __restrict__ ctx_len,
                                                   const int64_t* __restrict__ kv_row_off,
                                                   int64_t kv_rows_total, RopeArgs ra, Elt* q, Elt* k) {
    constexpr int kMaxPer = kRopeHeads / 2;  // groups >= 2 since D/2 <= 128
    const int i = blockIdx.x, b = blockIdx.y;
    const int half = D >> 1;
    const int groups = blockDim.x / half;
    const int d = threadIdx.x % half, grp = threadIdx.x / half;
    if (grp >= groups) return;
    const int nq = q ? Hq : 0;
    const int h0 = blockIdx.z * kRopeHeads;
    const int h_end = min(h0 + kRopeHeads, nq + (k ? Hkv : 0));
    int64_t krow = -1;
    if (k && h_end > nq) {
        krow = HOST_ROWS ? ra.k_row0[b] + i : kv_row_off[b] + (int64_t)ctx_len[b] + i;
        if (krow < 0 || krow >= kv_rows_total) krow = -1;  // outside the cache: K is not rotated
    }
    const int32_t pos = position[(size_t)b * T + i];
    Elt* rows[kMaxPer];
    double x[kMaxPer], y[kMaxPer];
#pragma unroll
    for (int s = 0; s < kMaxPer; ++s) {
        const int h = h0 + grp + s * groups;
        rows[s] = nullptr;
        if (h < h_end) {
            if (h < nq)
                rows[s] = q + (((size_t)b * T + i) * Hq + h) * D;
            else if (krow >= 0)
                rows[s] = k + ((size_t)(h - nq) * kv_rows_total + krow) * D;
        }
        if (rows[s]) {
            x[s] = load_elt(rows[s] + d);
            y[s] = load_elt(rows[s] + d + half);
        }
    }
    double sn, cs;
    sincos((double)pos * ra.f[d], &sn, &cs);
#pragma unroll
    for (int s = 0; s < kMaxPer; ++s) {
        if (rows[s]) {
            float xr, yr;
            rope_rotate_f64(x[s], y[s], cs, sn, xr, yr);
            store_elt(rows[s] + d, xr);
            store_elt(rows[s] + d + half, yr);
        }
    }
}

// ---------------------------------------------------------------------------
// KV commit.  One wave per (KV head, layer x {K, V}, sequence).  Accepted rows
// r_1 < ... < r_a satisfy r_j >= j, and once r_j > j every later r_i > i: the
// rows that stay put form a prefix, and the rows that move are j0..a.  They are
// copied in batches of up to 256 16-byte chunks in ascending j: a batch's chunks
// are all loaded and staged in LDS before the barrier, then stored.  A batch's
// sources (rows r_j > j) never lie among the rows written by earlier batches
// (rows < j), and within a batch every load has completed before the barrier, so
// no row is overwritten before it is read.
// ---------------------------------------------------------------------------
constexpr int kCommitChunks = 256;  // 16-byte chunks staged per batch (4 KB of LDS)

struct CommitLayers {
    char* k[kCommitMaxLayers];
    char* v[kCommitMaxLayers];
};

__global__ __launch_bounds__(64) void kv_commit_kernel(int T, int depth, int row_chunks,
                                                       int64_t kv_rows_total,
                                                       const int32_t* __restrict__ ctx_len,
                                                       const int64_t* __restrict__ kv_row_off,
                                                       const int32_t* __restrict__ accept_len,
                                                       const int32_t* __restrict__ accept_path,
                                                       int32_t* __restrict__ new_ctx_len, int write_ctx,
                                                       CommitLayers L) {
    __shared__ uint4 stage[kCommitChunks];
    __shared__ int32_t path[256];
    const int g = blockIdx.x, layer = blockIdx.y >> 1, is_v = blockIdx.y & 1, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int a = accept_len[b];
    const int amax = depth < T - 1 ? depth : T - 1;
    const int64_t ctx = ctx_len[b], off = kv_row_off[b];
    bool ok = a >= 0 && a <= amax && ctx >= 0 && off >= 0 && off + ctx + T <= kv_rows_total;
    int bad = 0;
    if (ok) {
        for (int j = lane; j < a; j += 64) {
            const int r = accept_path[(size_t)b * depth + j];
            path[j] = r;
            bad |= (r < 1 || r >= T);
        }
    }
    __syncthreads();
    if (ok) {
        for (int j = 1 + lane; j < a; j += 64) bad |= (path[j] <= path[j - 1]);
    }
    const int any_bad = __syncthreads_or(bad);  // every lane reaches this barrier
    ok = ok && !any_bad;
    if (write_ctx && g == 0 && blockIdx.y == 0 && lane == 0) new_ctx_len[b] = ok ? (int32_t)(ctx + 1 + a) : -1;
    if (!ok) return;
    int stay = 0;  // rows with r_j == j form a prefix
    while (stay < a && path[stay] == stay + 1) ++stay;
    const int moved = a - stay;
    if (moved == 0) return;
    char* cache = is_v ? L.v[layer] : L.k[layer];
    if (!cache) return;  // launched only to report the new context lengths
    const size_t row_bytes = (size_t)row_chunks * 16;
    char* base = cache + ((size_t)g * kv_rows_total + off + ctx) * row_bytes;
    const int total = moved * row_chunks;
    for (int e0 = 0; e0 < total; e0 += kCommitChunks) {
        const int n = total - e0 < kCommitChunks ? total - e0 : kCommitChunks;
        for (int e = lane; e < n; e += 64) {
            const int idx = e0 + e;
            const int j = stay + idx / row_chunks, c = idx - (idx / row_chunks) * row_chunks;
            stage[e] = *reinterpret_cast<const uint4*>(base + (size_t)path[j] * row_bytes + (size_t)c * 16);
        }
        __syncthreads();
        for (int e = lane; e < n; e += 64) {
            const int idx = e0 + e;
            const int j = stay + idx / row_chunks, c = idx - (idx / row_chunks) * row_chunks;
            *reinterpret_cast<uint4*>(base + (size_t)(j + 1) * row_bytes + (size_t)c * 16) = stage[e];
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Draft-side attention rows.  One workgroup per sequence.  Each frontier node
// marks its root path in an LDS bitmap over the nodes created so far; a node's
// row is the number of marked nodes below it (per-word prefix of popcounts plus
// the bits below it in its word), so rows follow ascending node id.  Rows whose
// ids rank past T_sub are dropped (never the case for a consistent tree: the
// frontier's root paths hold at most 1 + F (layer - 1) nodes), and since
// ancestors have smaller ids the kept rows stay ancestor-closed.
// ---------------------------------------------------------------------------
constexpr int kSubThreads = 256;
constexpr int kFlagWords = EAGLE_MAX_CAPACITY / 32;

__global__ __launch_bounds__(kSubThreads) void draft_subtree_kernel(
    int cap, int m, int F, int T_sub, int root_only, const int32_t* __restrict__ parent, const int32_t* __restrict__ depth,
    const int32_t* __restrict__ frontier, const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ ctx_len,
    int32_t* __restrict__ sub_node, int32_t* __restrict__ sub_parent, int32_t* __restrict__ position,
    uint64_t* __restrict__ mask, int32_t* __restrict__ query_row) {
    __shared__ uint32_t flags[kFlagWords];
    __shared__ int base[kFlagWords + 1];
    __shared__ int32_t s_par[EAGLE_MAX_TREE_ROWS];
    __shared__ int32_t s_node[EAGLE_MAX_TREE_ROWS];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1);
    if (root_only) {
        // draft layer 1: the root is the only query and the only row; the tree state
        // is not read (the first expand has not run yet)
        if (tid == 0) {
            sub_node[b] = 0;
            sub_parent[b] = -1;
            position[b] = ctx_len[b];
            mask[b] = 1ull;
        }
        for (int j = tid; j < m; j += kSubThreads) query_row[(size_t)b * m + j] = j == 0 ? 0 : -1;
        return;
    }
    int n = n_nodes[b];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const int nw = (n + 31) >> 5;
    for (int w = tid; w < kFlagWords; w += kSubThreads) flags[w] = 0;
    if (tid < T_sub) s_node[tid] = -1;
    __syncthreads();
    if (tid < F) {  // F <= T_sub <= 64 past layer 1
        int x = frontier[(size_t)b * m + tid];
        for (int steps = 0; x >= 0 && x < n && steps <= 255; ++steps) {
            atomicOr(&flags[x >> 5], 1u << (x & 31));
            x = parent[(size_t)b * cap + x];
        }
    }
    __syncthreads();
    // exclusive prefix of the words' popcounts (kFlagWords = 128: two words per lane of wave 0)
    if (tid < kWave) {
        const int c0 = __popc(flags[2 * lane]), c1 = __popc(flags[2 * lane + 1]);
        int incl = c0 + c1;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int o = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += o;
        }
        base[2 * lane] = incl - c0 - c1;
        base[2 * lane + 1] = incl - c1;
        if (lane == kWave - 1) base[kFlagWords] = incl;
    }
    __syncthreads();
    auto row_of = [&](int x) {
        return base[x >> 5] + __popc(flags[x >> 5] & ((1u << (x & 31)) - 1u));
    };
    auto marked = [&](int x) { return x >= 0 && x < n && ((flags[x >> 5] >> (x & 31)) & 1u); };
    for (int x = tid; x < nw * 32; x += kSubThreads) {
        if (marked(x)) {
            const int r = row_of(x);
            if (r < T_sub) s_node[r] = x;
        }
    }
    __syncthreads();
    if (tid < T_sub) {
        const int x = s_node[tid];
        int pr = -1;
        if (x >= 0) {
            const int p = parent[(size_t)b * cap + x];
            if (marked(p)) pr = row_of(p);
            if (pr >= T_sub) pr = -1;
        }
        s_par[tid] = pr;
    }
    __syncthreads();
    if (tid < T_sub) {
        const int x = s_node[tid];
        uint64_t bits = 1ull << tid;
        if (x >= 0) {
            // each step moves to an earlier row, so the walk ends within T_sub steps
            for (int r = s_par[tid]; r >= 0; r = s_par[r]) bits |= 1ull << r;
        }
        const size_t o = (size_t)b * T_sub + tid;
        sub_node[o] = x;
        sub_parent[o] = s_par[tid];
        position[o] = ctx_len[b] + (x >= 0 ? depth[(size_t)b * cap + x] : 0);
        mask[o] = bits;
    }
    for (int j = tid; j < m; j += kSubThreads) {
        int qr = -1;
        if (j < F) {
            const int f = frontier[(size_t)b * m + j];
            if (marked(f)) {
                const int r = row_of(f);
                qr = r < T_sub ? r : -1;
            }
        }
        query_row[(size_t)b * m + j] = qr;
    }
}

// ---------------------------------------------------------------------------
// Row gather: one wave per (row, KV head, sequence); lane = 16-byte chunk of the
// row, K and V.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void kv_gather_kernel(int T, int row_chunks, int64_t kv_rows_total,
                                                       const int32_t* __restrict__ ctx_len,
                                                       const int64_t* __restrict__ kv_row_off,
                                                       int64_t src_rows_per_seq, int64_t src_rows_total,
                                                       const int32_t* __restrict__ rows,
                                                       const char* __restrict__ src_k,
                                                       const char* __restrict__ src_v, char* k, char* v) {
    const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int64_t dst = kv_row_off[b] + (int64_t)ctx_len[b] + r;
    if (dst < 0 || dst >= kv_rows_total) return;
    int64_t x = rows[(size_t)b * T + r];
    if (x < 0 || x >= src_rows_per_seq) x = 0;
    const int64_t src = (int64_t)b * src_rows_per_seq + x;
    if (src >= src_rows_total) return;
    const size_t row_bytes = (size_t)row_chunks * 16;
    const size_t so = ((size_t)g * src_rows_total + src) * row_bytes, dofs = ((size_t)g * kv_rows_total + dst) * row_bytes;
    for (int c = lane; c < row_chunks; c += 64) {
        const uint4 kk = *reinterpret_cast<const uint4*>(src_k + so + (size_t)c * 16);
        const uint4 vv = *reinterpret_cast<const uint4*>(src_v + so + (size_t)c * 16);
        *reinterpret_cast<uint4*>(k + dofs + (size_t)c * 16) = kk;
        *reinterpret_cast<uint4*>(v + dofs + (size_t)c * 16) = vv;
    }
}

}  // namespace

hipError_t launch_draft_subtree(const eagle_tree_cfg& cfg, int layer, int cap, int F, int T_sub,
                                const eagle_tree_state& st, const int32_t* ctx_len, int32_t* sub_node,
                                int32_t* sub_parent, int32_t* position, uint64_t* mask, int32_t* query_row,
                                hipStream_t stream) {
    draft_subtree_kernel<<<cfg.batch, kSubThreads, 0, stream>>>(cap, cfg.m, F, T_sub, layer == 1 ? 1 : 0,
                                                                 st.parent, st.depth,
                                                                 st.frontier, st.n_nodes, ctx_len, sub_node,
                                                                 sub_parent, position, mask, query_row);
    return hipGetLastError();
}

hipError_t launch_kv_gather(const eagle_attn_desc& d, const int32_t* rows, int64_t src_rows_per_seq,
                            int64_t src_rows_total, const void* src_k, const void* src_v, void* k, void* v,
                            hipStream_t stream) {
    const int elt = d.dtype == EAGLE_BF16 ? 2 : 4;
    const int row_chunks = d.head_dim * elt / 16;
    kv_gather_kernel<<<dim3(d.T, d.n_kv_heads, d.batch), 64, 0, stream>>>(
        d.T, row_chunks, d.kv_rows_total, d.ctx_len, d.kv_row_off, src_rows_per_seq, src_rows_total, rows,
        (const char*)src_k, (const char*)src_v, (char*)k, (char*)v);
    return hipGetLastError();
}


hipError_t launch_mask_static(int batch, int T, const int32_t* flat_parent, const int32_t* ctx_len,
                              int32_t* flat_depth, int32_t* position, uint64_t* mask, hipStream_t stream) {
    mask_static_kernel<<<batch, 64, 0, stream>>>(T, flat_parent, ctx_len, flat_depth, position, mask);
    return hipGetLastError();
}

hipError_t launch_rope(const eagle_attn_desc& d, const int32_t* position, double base, void* q, void* k,
                       hipStream_t stream) {
    RopeArgs ra{};
    const int half = d.head_dim / 2;
    for (int j = 0; j < half; ++j) ra.f[j] = pow(base, -2.0 * j / d.head_dim);
    const bool host_rows = d.ctx_len_host && d.kv_row_off_host && d.batch <= kRopeHostRows;
    if (host_rows)
        for (int b = 0; b < d.batch; ++b) ra.k_row0[b] = d.kv_row_off_host[b] + d.ctx_len_host[b];
    const int heads = (q ? d.n_q_heads : 0) + (k ? d.n_kv_heads : 0);
    const dim3 grid(d.T, d.batch, (heads + kRopeHeads - 1) / kRopeHeads);
    if (d.dtype == EAGLE_BF16) {
        auto kern = host_rows ? rope_kernel<uint16_t, true> : rope_kernel<uint16_t, false>;
        kern<<<grid, 256, 0, stream>>>(d.T, d.n_q_heads, d.n_kv_heads, d.head_dim, position, d.ctx_len,
                                       d.kv_row_off, d.kv_rows_total, ra, (uint16_t*)q, (uint16_t*)k);
    } else {
        auto kern = host_rows ? rope_kernel<float, true> : rope_kernel<float, false>;
        kern<<<grid, 256, 0, stream>>>(d.T, d.n_q_heads, d.n_kv_heads, d.head_dim, position, d.ctx_len,
                                       d.kv_row_off, d.kv_rows_total, ra, (float*)q, (float*)k);
    }
    return hipGetLastError();
}

hipError_t launch_kv_commit(const eagle_commit_desc& d, const int32_t* accept_len, const int32_t* accept_path,
                            void* const* k_layers, void* const* v_layers, int32_t* new_ctx_len,
                            hipStream_t stream) {
    const int elt = d.dtype == EAGLE_BF16 ? 2 : 4;
    const int row_chunks = d.head_dim * elt / 16;
    // with no layers one launch still writes new_ctx_len (null cache pointers: no copies)
    for (int l0 = 0; l0 == 0 || l0 < d.n_layers; l0 += kCommitMaxLayers) {
        const int nl = d.n_layers - l0 < kCommitMaxLayers ? d.n_layers - l0 : kCommitMaxLayers;
        CommitLayers L{};
        for (int l = 0; l < nl; ++l) {
            L.k[l] = (char*)k_layers[l0 + l];
            L.v[l] = (char*)v_layers[l0 + l];
        }
        const dim3 grid(nl > 0 ? d.n_kv_heads : 1, nl > 0 ? 2 * nl : 1, d.batch);
        kv_commit_kernel<<<grid, 64, 0, stream>>>(d.T, d.depth, row_chunks, d.kv_rows_total, d.ctx_len,
                                                  d.kv_row_off, accept_len, accept_path, new_ctx_len,
                                                  l0 == 0 ? 1 : 0, L);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace eagle
