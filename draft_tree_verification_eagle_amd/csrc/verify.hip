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
// all other tokens, summed directly (never as 1 - sum of removed), and the
// fixed-point mass of each of 1024 contiguous token chunks.  K7 (one workgroup
// per sequence) walks the tree with Philox4x32-10 uniforms and draws the bonus
// token by inverse CDF: a block-wide prefix sum over the final row's chunk masses
// (minus the removed tokens) finds the chunk holding u * total, and one wave
// rescans that chunk token by token.  Masses are taken in 2^-s fixed point (s = 48
// for vocabularies up to 32768, lower above so no sum can overflow), so every sum
// is exact in any order and the two kernels agree bit for bit.
#include "device_common.hpp"
#include "launchers.hpp"

namespace eagle {

constexpr int kKids = EAGLE_MAX_TOPK;

// Token mass in fixed point: masses are <= 1 (the row maximum has mass 1); with
// 2^s, s = 63 - ceil(log2 V), a row total stays below 2^63, so prefix sums are
// exact whatever the summation order.
__host__ __device__ inline int fixed_shift(int V) {
    int k = 0;
    while ((1 << k) < V) ++k;
    const int sh = 63 - k;
    return sh < 48 ? sh : 48;
}
__device__ __forceinline__ uint64_t fixed_mass(double e, double scale) { return (uint64_t)(e * scale); }

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
// K6: one workgroup of 1024 threads per (row, sequence).  Wave 0 finds the row's
// children with one ballot (flattened order = lane order).  The argmax pass reads
// token t = tid + 1024 * it (coalesced); the mass pass gives thread tid the
// contiguous chunk [tid * ch, tid * ch + ch), ch = ceil(V / 1024) <= 256 (re-read,
// from L2), with a 256-bit mask of the children in it, and stores the chunk's
// fixed-point mass (children included) for the bonus draw.
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kRowBatch = 32;       // tokens per thread loaded together
constexpr int kMaxChunkTokens = 256;  // ceil(EAGLE_MAX_VOCAB / 1024)
static_assert((EAGLE_MAX_VOCAB + kRowThreads - 1) / kRowThreads <= kMaxChunkTokens, "chunk mask");

__global__ __launch_bounds__(kRowThreads) void verify_rows_kernel(
    const float* __restrict__ target, int T, int V, const int32_t* __restrict__ flat_token,
    const int32_t* __restrict__ flat_parent, float temperature, RowStats* __restrict__ stats,
    uint64_t* __restrict__ chunk_mass) {
    __shared__ int32_t s_kid_row[kKids];
    __shared__ int32_t s_kid_tok[kKids];
    __shared__ int s_nk;
    __shared__ uint64_t s_key[kRowWaves];
    __shared__ double s_red[kRowWaves];
    const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    const float* z = target + ((size_t)b * T + i) * (size_t)V;
    if (wid == 0) {
        const bool kid = lane < T && flat_parent[(size_t)b * T + lane] == i;
        const uint64_t bal = __ballot(kid);
        const int pos = __popcll(bal & ((1ull << lane) - 1ull));
        if (kid && pos < kKids) {
            s_kid_row[pos] = lane;
            s_kid_tok[pos] = flat_token[(size_t)b * T + lane];
        }
        if (lane == 0) s_nk = __popcll(bal) < kKids ? __popcll(bal) : kKids;
    }
    // Thread tid reads tokens t = tid + 1024 * it in unrolled batches of 32 (all
    // loads of a batch in flight together); with vocab <= 32768 the single batch
    // stays in registers for the second pass.
    const int iters = (V + kRowThreads - 1) / kRowThreads;  // <= 256
    float zr[kRowBatch];
    uint64_t best = 0;
    for (int it0 = 0; it0 < iters; it0 += kRowBatch) {
#pragma unroll
        for (int q = 0; q < kRowBatch; ++q) {
            const int t = (it0 + q) * kRowThreads + tid;
            zr[q] = t < V ? z[t] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < kRowBatch; ++q) {
            const int t = (it0 + q) * kRowThreads + tid;
            if (t < V) {
                const uint64_t key = logit_key(zr[q], (uint32_t)t);
                best = key > best ? key : best;
            }
        }
    }
    best = wave_max_u64(best);
    if (lane == 0) s_key[wid] = best;
    __syncthreads();
    for (int w = 0; w < kRowWaves; ++w) best = s_key[w] > best ? s_key[w] : best;
    const int amax = (int)logit_key_token(best);
    const float zmax = logit_key_value(best);
    const int nk = s_nk;
    RowStats* out = stats + (size_t)b * T + i;
    if (temperature > 0.0f) {
        const double temp = (double)temperature;
        const bool unit_temp = temperature == 1.0f;  // x / 1 == x: skip the fp64 divide
        const double fscale = ldexp(1.0, fixed_shift(V));
        const int ch = (V + kRowThreads - 1) / kRowThreads;
        const int c0 = min(V, tid * ch), c1 = min(V, c0 + ch);
        uint64_t km[4] = {0, 0, 0, 0};  // bit d: token c0 + d is a child of the row
        for (int c = 0; c < nk; ++c) {
            const int d = s_kid_tok[c] - c0;
            if (d >= 0 && d < c1 - c0) {
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    if ((d >> 6) == w) km[w] |= 1ull << (d & 63);
            }
        }
        double s = 0.0;
        uint64_t fm = 0;
        // 16-byte aligned chunk starts: vector loads
        const bool vec = (V & 3) == 0 && (ch & 3) == 0 && ((uintptr_t)target & 15) == 0;
        for (int a0 = c0; a0 < c1; a0 += kRowBatch) {
            float zz[kRowBatch];
            if (vec) {
#pragma unroll
                for (int q = 0; q < kRowBatch; q += 4) {
                    float4 v4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    if (a0 + q < c1) v4 = *reinterpret_cast<const float4*>(z + a0 + q);
                    zz[q] = v4.x; zz[q + 1] = v4.y; zz[q + 2] = v4.z; zz[q + 3] = v4.w;
                }
            } else {
#pragma unroll
                for (int q = 0; q < kRowBatch; ++q) zz[q] = a0 + q < c1 ? z[a0 + q] : 0.0f;
            }
            const int o = a0 - c0;  // a multiple of 32: bits o .. o + 31 of the mask
            uint64_t kw = km[0];
#pragma unroll
            for (int w = 1; w < 4; ++w)
                if ((o >> 6) == w) kw = km[w];
            const uint32_t kb = (uint32_t)(kw >> (o & 63));
#pragma unroll
            for (int q = 0; q < kRowBatch; ++q) {
                if (a0 + q < c1) {
                    const double x = (double)zz[q] - (double)zmax;
                    const double e = exp_nonpos_f64(unit_temp ? x : x / temp);
                    fm += fixed_mass(e, fscale);
                    if (!((kb >> q) & 1u)) s += e;
                }
            }
        }
        chunk_mass[((size_t)b * T + i) * kRowThreads + tid] = fm;
        s = block_sum_f64(s, s_red);
        if (tid < nk) out->kid_e[tid] = exp_nonpos_f64(((double)z[s_kid_tok[tid]] - (double)zmax) / temp);
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
static_assert(kWalkThreads == kRowThreads, "one chunk mass per walk thread");
constexpr int kMaxDepth = 255;  // the library's depth limit

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



__global__ __launch_bounds__(kWalkThreads) void verify_walk_kernel(
    const float* __restrict__ target, int T, int V, int depth, const int32_t* __restrict__ flat_token,
    float temperature, uint64_t seed, uint64_t step, const RowStats* __restrict__ stats,
    const uint64_t* __restrict__ chunk_mass, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ accept_path, int32_t* __restrict__ out_tokens) {
    __shared__ RowStats s_rs[EAGLE_MAX_TREE_ROWS];
    __shared__ int32_t s_tok[EAGLE_MAX_TREE_ROWS];
    __shared__ int32_t s_path[kMaxDepth];      // depth <= 255: accepted rows, -1 padded
    __shared__ int32_t s_out[kMaxDepth + 1];   // accepted tokens then the bonus, -1 padded
    __shared__ int s_bonus_row, s_len;
    __shared__ int32_t s_removed[kKids];
    __shared__ int s_n_removed;
    __shared__ uint64_t s_wave[kWalkThreads / kWave];
    __shared__ int s_hit_chunk;
    __shared__ uint64_t s_hit_prefix;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1);
    const bool sampled = temperature > 0.0f;

    // the row statistics and tokens of this sequence, in one round trip
    {
        static_assert(sizeof(RowStats) % 8 == 0, "copied as 8-byte words");
        const uint64_t* src = (const uint64_t*)(stats + (size_t)b * T);
        uint64_t* dst = (uint64_t*)s_rs;
        const int words = T * (int)(sizeof(RowStats) / 8);
        for (int w = tid; w < words; w += kWalkThreads) dst[w] = src[w];
        if (tid < T) s_tok[tid] = flat_token[(size_t)b * T + tid];
        if (tid < depth) s_path[tid] = -1;
        if (tid <= depth) s_out[tid] = -1;
    }
    __syncthreads();

    // The walk, by wave 0: lane c evaluates child c of the current row.  The
    // sequential rule takes the first child (flattened order) whose test passes,
    // and child c's test depends only on c (the children before it are the ones
    // already removed), so the lowest set bit of the ballot is that child.
    if (tid < kWave) {
        int cur = 0, len = 0;
        while (true) {
            const RowStats& R = s_rs[cur];
            const int nk = R.n_kids;
            int next = -1;
            if (len < depth && nk > 0) {
                bool pass = false;
                if (lane < nk) {
                    if (!sampled) {
                        pass = s_tok[R.kid_row[lane]] == R.argmax;
                    } else {
                        double denom = R.rest;
                        for (int c = lane; c < nk; ++c) denom += R.kid_e[c];
                        const double ratio = R.kid_e[lane] / denom;
                        const double u = decision_uniform(seed, step, (uint32_t)b, (uint32_t)cur, (uint32_t)lane);
                        pass = u < ratio;
                    }
                }
                const uint64_t bal = __ballot(pass);
                if (bal) next = R.kid_row[__ffsll((unsigned long long)bal) - 1];
            }
            if (next >= 0) {
                if (lane == 0) {
                    s_path[len] = next;
                    s_out[len] = s_tok[next];
                }
                ++len;
                cur = next;
                continue;
            }
            if (lane == 0) {
                if (!sampled) s_out[len] = R.argmax;
                s_bonus_row = cur;
                s_len = len;
                // every child of the final row was tested and rejected (none when it is a leaf)
                s_n_removed = (len < depth) ? nk : 0;
            }
            if (len < depth && lane < nk) s_removed[lane] = s_tok[R.kid_row[lane]];
            break;
        }
    }
    __syncthreads();

    if (sampled) {
        // Bonus draw: the smallest t whose running residual mass exceeds u * total.
        // Chunk tid = tokens [tid * ch, tid * ch + ch); its residual mass is the
        // chunk mass from K6 minus the removed tokens in it (the row's children,
        // whose masses K6 also kept).  The integer intervals [prefix, prefix + mass)
        // partition [0, total) exactly, so exactly one chunk holds the goal; wave 0
        // then rescans that chunk, lane l over its l-th slice of ceil(ch / 64)
        // tokens, with the same masses bit for bit.
        const int row = s_bonus_row, nrem = s_n_removed;
        const RowStats& R = s_rs[row];
        const float* z = target + ((size_t)b * T + row) * (size_t)V;
        const double zmax = (double)R.zmax, temp = (double)temperature;
        const bool unit_temp = temperature == 1.0f;  // x / 1 == x: skip the fp64 divide
        const double fscale = ldexp(1.0, fixed_shift(V));
        const int ch = (V + kWalkThreads - 1) / kWalkThreads;
        const int c0 = min(V, tid * ch), c1 = min(V, c0 + ch);
        uint64_t cs = chunk_mass[((size_t)b * T + row) * kWalkThreads + tid];
        for (int c = 0; c < nrem; ++c) {
            const int tok = s_removed[c];  // child c's token; its mass is R.kid_e[c]
            if (tok >= c0 && tok < c1) cs -= fixed_mass(R.kid_e[c], fscale);
        }
        const Philox4x32 word = philox4x32_10(Philox4x32{kBonusSlot, (uint32_t)row, (uint32_t)b, (uint32_t)step},
                                              (uint32_t)seed, (uint32_t)(seed >> 32));
        const uint64_t u24 = (uint64_t)(word.c0 >> 8);
        if (tid == 0) s_hit_chunk = -1;
        uint64_t total = 0;
        const uint64_t prefix = block_exclusive_scan_u64(cs, s_wave, &total);  // synchronises
        const uint64_t goal = __umul64hi(total, u24 << 40);  // floor(total * u24 / 2^24)
        if (cs > 0 && prefix <= goal && goal < prefix + cs) {
            s_hit_chunk = tid;
            s_hit_prefix = prefix;
        }
        __syncthreads();
        const int hc = s_hit_chunk;
        if (tid < kWave && hc >= 0) {
            const int per = (ch + kWave - 1) / kWave;  // <= 4
            const int h0 = hc * ch, h1 = min(V, h0 + ch);
            const int l0 = min(h1, h0 + lane * per), l1 = min(h1, l0 + per);
            auto mass_of = [&](int t) -> uint64_t {
                for (int c = 0; c < nrem; ++c)
                    if (s_removed[c] == t) return 0;
                const double x = (double)z[t] - zmax;
                return fixed_mass(exp_nonpos_f64(unit_temp ? x : x / temp), fscale);
            };
            uint64_t lm = 0;
            for (int t = l0; t < l1; ++t) lm += mass_of(t);
            uint64_t incl = lm;  // inclusive prefix over the lanes (exact)
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const uint32_t lo = __shfl_up((uint32_t)incl, off, kWave);
                const uint32_t hi = __shfl_up((uint32_t)(incl >> 32), off, kWave);
                if (lane >= off) incl += ((uint64_t)hi << 32) | lo;
            }
            const uint64_t base = s_hit_prefix + (incl - lm);
            if (lm > 0 && base <= goal && goal < base + lm) {
                uint64_t run = base;
                for (int t = l0; t < l1; ++t) {
                    run += mass_of(t);
                    if (run > goal) {
                        s_out[s_len] = t;
                        break;
                    }
                }
            }
        }
        __syncthreads();
    }
    // results, written once
    int32_t* path = accept_path + (size_t)b * depth;
    int32_t* outt = out_tokens + (size_t)b * (depth + 1);
    if (tid < depth) path[tid] = s_path[tid];
    if (tid <= depth) outt[tid] = s_out[tid];
    if (tid == 0) accept_len[b] = s_len;
}

// ---------------------------------------------------------------------------
// Workspace: RowStats [batch][T], then the chunk masses [batch][T][1024] (uint64).
static size_t stats_bytes(const eagle_tree_cfg& cfg) {
    return ((size_t)cfg.batch * (size_t)(cfg.n + 1) * sizeof(RowStats) + 255) & ~(size_t)255;
}
size_t verify_workspace_bytes(const eagle_tree_cfg& cfg) {
    return stats_bytes(cfg) + (size_t)cfg.batch * (size_t)(cfg.n + 1) * kRowThreads * sizeof(uint64_t);
}

hipError_t launch_verify(const eagle_tree_cfg& cfg, const float* target, const int32_t* flat_token,
                         const int32_t* flat_parent, float temperature, uint64_t seed,
                         uint64_t step, int32_t* accept_len, int32_t* accept_path,
                         int32_t* out_tokens, void* workspace, hipStream_t stream) {
    const int T = cfg.n + 1;
    RowStats* stats = (RowStats*)workspace;
    uint64_t* chunk_mass = (uint64_t*)((unsigned char*)workspace + stats_bytes(cfg));
    verify_rows_kernel<<<dim3(T, cfg.batch), kRowThreads, 0, stream>>>(
        target, T, cfg.vocab, flat_token, flat_parent, temperature, stats, chunk_mass);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    verify_walk_kernel<<<cfg.batch, kWalkThreads, 0, stream>>>(
        target, T, cfg.vocab, cfg.depth, flat_token, temperature, seed, step, stats, chunk_mass,
        accept_len, accept_path, out_tokens);
    return hipGetLastError();
}

}  // namespace eagle
