// Lossless acceptance over the target logits of the flattened tree (gfx950).
//
// Pages: CSDN page "论文解读：eagle/eagle2" sections 1.1 / 1.2 and the abstract of
// "EAGLE: Speculative Sampling Requires Rethinking Feature Uncertainty" -- the
// verification must leave the target's output distribution unchanged, under
// greedy and under sampled decoding.
//
// Greedy: follow the child whose token is the row's argmax (lowest id on ties).
// Sampled: each child proposes its own token as a point mass; the children of the
// current row are tested in flattened order with acceptance probability
// p(tok) / (mass of tokens not yet rejected at this row); rejected tokens are
// removed; the bonus token is drawn from the remaining mass by inverse CDF.
//
// K6 (one workgroup per row) computes argmax, row max and, for sampling, the fp64
// masses exp((z - zmax) / temperature) of every child token plus the fp64 mass of
// all other tokens, summed directly (never as 1 - sum of removed).  K7 (one
// workgroup per sequence) walks the tree with Philox4x32-10 uniforms and draws
// the bonus token by inverse CDF over a block-wide prefix sum of the residual
// masses, taken in 2^-48 fixed point so the sum is exact in any order.
#include "device_common.hpp"
#include "launchers.hpp"

namespace eagle {

constexpr int kKids = EAGLE_MAX_TOPK;

// Per-row statistics in the workspace.
struct RowStats {
    double rest;        // mass of tokens that are not children of the row
    double kid_e[kKids];  // mass of each child's token, flattened order
    int32_t kid_row[kKids];
    float zmax;
    int32_t argmax;
    int32_t n_kids;
    int32_t pad;
};

// ---------------------------------------------------------------------------
// K6
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 256;

__global__ __launch_bounds__(kRowThreads) void verify_rows_kernel(
    const float* __restrict__ target, int T, int V, const int32_t* __restrict__ flat_token,
    const int32_t* __restrict__ flat_parent, float temperature, RowStats* __restrict__ stats) {
    __shared__ int32_t s_kid_row[kKids];
    __shared__ int32_t s_kid_tok[kKids];
    __shared__ int s_nk;
    __shared__ uint64_t s_key[kRowThreads / kWave];
    __shared__ double s_red[kRowThreads / kWave];
    const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    const float* z = target + ((size_t)b * T + i) * (size_t)V;
    if (tid == 0) {
        int nk = 0;
        for (int j = 0; j < T && nk < kKids; ++j) {
            if (flat_parent[(size_t)b * T + j] == i) {
                s_kid_row[nk] = j;
                s_kid_tok[nk] = flat_token[(size_t)b * T + j];
                ++nk;
            }
        }
        s_nk = nk;
    }
    uint64_t best = 0;
    for (int t = tid; t < V; t += kRowThreads) {
        const uint64_t key = logit_key(z[t], (uint32_t)t);
        best = key > best ? key : best;
    }
    best = wave_max_u64(best);
    if (lane == 0) s_key[wid] = best;
    __syncthreads();
    for (int w = 0; w < kRowThreads / kWave; ++w) best = s_key[w] > best ? s_key[w] : best;
    const int amax = (int)logit_key_token(best);
    const float zmax = z[amax];
    const int nk = s_nk;
    RowStats* out = stats + (size_t)b * T + i;
    if (temperature > 0.0f) {
        const double temp = (double)temperature;
        double s = 0.0;
        for (int t = tid; t < V; t += kRowThreads) {
            bool kid = false;
            for (int c = 0; c < nk; ++c) kid |= (s_kid_tok[c] == t);
            if (!kid) s += exp(((double)z[t] - (double)zmax) / temp);
        }
        s = block_sum_f64(s, s_red);
        if (tid < nk) out->kid_e[tid] = exp(((double)z[s_kid_tok[tid]] - (double)zmax) / temp);
        if (tid == 0) out->rest = s;
    }
    if (tid < nk) out->kid_row[tid] = s_kid_row[tid];
    if (tid == 0) {
        out->zmax = zmax;
        out->argmax = amax;
        out->n_kids = nk;
    }
}

// ---------------------------------------------------------------------------
// K7
// ---------------------------------------------------------------------------
constexpr int kWalkThreads = 1024;

// Exclusive block prefix sum of one uint64 per thread (exact, order-free);
// returns the thread's exclusive prefix and the block total.  Contains
// __syncthreads.
__device__ uint64_t block_exclusive_scan_u64(uint64_t v, uint64_t* s_wave, uint64_t* total) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    uint64_t incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t lo = __shfl_up((uint32_t)incl, off, kWave);
        const uint32_t hi = __shfl_up((uint32_t)(incl >> 32), off, kWave);
        if (lane >= off) incl += ((uint64_t)hi << 32) | lo;
    }
    if (lane == kWave - 1) s_wave[wid] = incl;
    __syncthreads();
    uint64_t before = 0, all = 0;
    for (int w = 0; w < nw; ++w) {
        if (w < wid) before += s_wave[w];
        all += s_wave[w];
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

// Token mass in 2^-48 fixed point (masses are <= 1: the row maximum has mass 1),
// so prefix sums are exact whatever the summation order.
__device__ __forceinline__ uint64_t fixed_mass(double e) {
    return (uint64_t)(e * 281474976710656.0);
}

__global__ __launch_bounds__(kWalkThreads) void verify_walk_kernel(
    const float* __restrict__ target, int T, int V, int depth, const int32_t* __restrict__ flat_token,
    float temperature, uint64_t seed, uint64_t step, const RowStats* __restrict__ stats,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_path,
    int32_t* __restrict__ out_tokens) {
    __shared__ int s_bonus_row, s_len;
    __shared__ int32_t s_removed[kKids];
    __shared__ int s_n_removed;
    __shared__ uint64_t s_wave[kWalkThreads / kWave];
    const int b = blockIdx.x, tid = threadIdx.x;
    const bool sampled = temperature > 0.0f;
    const RowStats* rs = stats + (size_t)b * T;
    int32_t* path = accept_path + (size_t)b * depth;
    int32_t* outt = out_tokens + (size_t)b * (depth + 1);

    if (tid == 0) {
        for (int d = 0; d < depth; ++d) path[d] = -1;
        for (int d = 0; d <= depth; ++d) outt[d] = -1;
        int cur = 0, len = 0;
        while (true) {
            const RowStats& R = rs[cur];
            int next = -1;
            if (len < depth) {
                if (!sampled) {
                    for (int c = 0; c < R.n_kids; ++c)
                        if (flat_token[(size_t)b * T + R.kid_row[c]] == R.argmax) { next = R.kid_row[c]; break; }
                } else {
                    for (int c = 0; c < R.n_kids; ++c) {
                        double denom = R.rest;
                        for (int s2 = c; s2 < R.n_kids; ++s2) denom += R.kid_e[s2];
                        const double ratio = R.kid_e[c] / denom;
                        const double u = decision_uniform(seed, step, (uint32_t)b, (uint32_t)cur, (uint32_t)c);
                        if (u < ratio) { next = R.kid_row[c]; break; }
                    }
                }
            }
            if (next >= 0) {
                path[len] = next;
                outt[len] = flat_token[(size_t)b * T + next];
                ++len;
                cur = next;
                continue;
            }
            if (!sampled) outt[len] = R.argmax;
            // every child of the final row was tested and rejected (none when it is a leaf)
            const int nrem = (len < depth) ? R.n_kids : 0;
            for (int c = 0; c < nrem; ++c) s_removed[c] = flat_token[(size_t)b * T + R.kid_row[c]];
            s_n_removed = nrem;
            s_bonus_row = cur;
            s_len = len;
            break;
        }
        accept_len[b] = s_len;
    }
    if (!sampled) return;
    __syncthreads();

    // Bonus draw: smallest t whose running residual mass exceeds u * total, the
    // masses in 2^-48 fixed point.  Thread tid owns tokens [t0, t1); the integer
    // intervals [prefix, prefix + mass) partition [0, total) exactly, so exactly
    // one thread holds the crossing.
    const int row = s_bonus_row, nrem = s_n_removed;
    const float* z = target + ((size_t)b * T + row) * (size_t)V;
    const double zmax = (double)rs[row].zmax, temp = (double)temperature;
    const int chunk = (V + kWalkThreads - 1) / kWalkThreads;
    const int t0 = min(V, tid * chunk), t1 = min(V, t0 + chunk);
    uint64_t cs = 0;
    for (int t = t0; t < t1; ++t) {
        bool rem = false;
        for (int c = 0; c < nrem; ++c) rem |= (s_removed[c] == t);
        if (!rem) cs += fixed_mass(exp(((double)z[t] - zmax) / temp));
    }
    uint64_t total = 0;
    const uint64_t prefix = block_exclusive_scan_u64(cs, s_wave, &total);
    const Philox4x32 word = philox4x32_10(Philox4x32{kBonusSlot, (uint32_t)row, (uint32_t)b, (uint32_t)step},
                                          (uint32_t)seed, (uint32_t)(seed >> 32));
    const uint64_t u24 = (uint64_t)(word.c0 >> 8);
    const uint64_t goal = __umul64hi(total, u24 << 40);  // floor(total * u24 / 2^24)
    if (cs > 0 && prefix <= goal && goal < prefix + cs) {
        uint64_t run = prefix;
        for (int t = t0; t < t1; ++t) {
            bool rem = false;
            for (int c = 0; c < nrem; ++c) rem |= (s_removed[c] == t);
            if (rem) continue;
            run += fixed_mass(exp(((double)z[t] - zmax) / temp));
            if (run > goal) {
                outt[s_len] = t;
                break;
            }
        }
    }
}

// ---------------------------------------------------------------------------
size_t verify_workspace_bytes(const eagle_tree_cfg& cfg) {
    return (size_t)cfg.batch * (size_t)(cfg.n + 1) * sizeof(RowStats);
}

hipError_t launch_verify(const eagle_tree_cfg& cfg, const float* target, const int32_t* flat_token,
                         const int32_t* flat_parent, float temperature, uint64_t seed,
                         uint64_t step, int32_t* accept_len, int32_t* accept_path,
                         int32_t* out_tokens, void* workspace, hipStream_t stream) {
    const int T = cfg.n + 1;
    RowStats* stats = (RowStats*)workspace;
    verify_rows_kernel<<<dim3(T, cfg.batch), kRowThreads, 0, stream>>>(
        target, T, cfg.vocab, flat_token, flat_parent, temperature, stats);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    verify_walk_kernel<<<cfg.batch, kWalkThreads, 0, stream>>>(
        target, T, cfg.vocab, cfg.depth, flat_token, temperature, seed, step, stats, accept_len,
        accept_path, out_tokens);
    return hipGetLastError();
}

}  // namespace eagle
