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
// K6 (four workgroups per row) computes argmax, row max and, for sampling, the fp64
// masses exp((z - zmax) / temperature) of every child token plus the fp64 mass of
// all other tokens, summed directly (never as 1 - sum of removed), and the
// fixed-point mass of each of 1024 contiguous token chunks.  A row may have up to
// T - 1 children (caller-given static trees), and siblings may carry the same
// token: a token already rejected at a row has no residual mass, so a later
// sibling carrying it has acceptance probability 0, and each removed token's
// mass leaves the residual once.  K7 (one workgroup
// per sequence) walks the tree with Philox4x32-10 uniforms and draws the bonus
// token by inverse CDF: a block-wide prefix sum over the final row's chunk masses
// (minus the removed tokens) finds the chunk holding u * total, and one wave
// rescans that chunk token by token.  Masses are taken in 2^-s fixed point (s = 48
// for vocabularies up to 32768, lower above so no sum can overflow), so every sum
// is exact in any order and the two kernels agree bit for bit.
#include "device_common.hpp"
#include "launchers.hpp"

namespace eagle {

// children of one row: every other row of the tree at most
constexpr int kKids = EAGLE_MAX_TREE_ROWS;
static_assert(kKids <= kWave, "one wave holds a row's children, lane = row");

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

// Per-row statistics in the workspace.  Every row but the root has exactly one
// parent, so a child's mass in its parent's row is kept with the child.
struct RowStats {
    double rest[4];  // mass of tokens that are not children of the row, per quarter of its chunks
    double e_kid;    // mass of this row's token in its parent row (sampled mode; unused for the root)
    float zmax;
    int32_t argmax;
};

// ---------------------------------------------------------------------------
// K6: kRowSplit workgroups of 512 threads per (row, sequence), all four on one
// XCD (blockIdx.x mod 8) so the row is fetched from HBM once and re-read from
// that XCD's L2.  Every workgroup finds the row's maximum and argmax over the
// whole row (float4 loads, all in flight together for vocabularies up to 32768);
// then, for sampling, workgroup q takes chunks [256 q, 256 q + 256) of the row's
// 1024 contiguous token chunks (ch = ceil(V / 1024) tokens each; two threads per
// chunk, re-read from L2), with a 256-bit mask of the row's children in the chunk: it
// stores each chunk's fixed-point mass (children included) for the bonus draw and
// the fp64 mass of the non-child tokens of its quarter.  Workgroup 0 also writes
// the argmax and the maximum, and each child's fp64 mass into the child's own
// statistics.  Wave 0 of each workgroup finds the children with one ballot
// (flattened order = lane order).
// ---------------------------------------------------------------------------
constexpr int kRowSplit = 4;
constexpr int kRowThreads = 512;
constexpr int kWgChunks = kRowThreads / 2;           // two threads per chunk
constexpr int kRowChunks = kRowSplit * kWgChunks;    // 1024 chunks per row
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kRowBatch = 16;       // tokens per thread per step of the mass pass (<= 32)
// float4 loads per thread in flight together in the maximum pass: a whole 32000-token
// row in one step.  With the mass pass's step this keeps the kernel at 78 VGPRs,
// three 512-thread workgroups per CU (a batch of many rows runs 3x as many at once)
constexpr int kMaxBatch = 16;
static_assert(kRowBatch <= 32, "one 32-bit window of the child mask per step");
constexpr int kMaxChunkTokens = 256;  // ceil(EAGLE_MAX_VOCAB / 1024)
static_assert((EAGLE_MAX_VOCAB + kRowChunks - 1) / kRowChunks <= kMaxChunkTokens, "chunk mask");
static_assert(kRowSplit == 4, "RowStats keeps four partial rest masses");
// From this many tree rows in a call (batch x T), one workgroup takes a whole row:
// it finds the maximum once and then does the four quarters' mass passes one after
// the other, each exactly as that quarter's workgroup would (same threads, same
// sums), so the statistics are the same bits; the row is read once for its maximum
// instead of four times, and there are enough rows to fill the GPU.
constexpr int kWholeRowsFrom = 256;

template <bool kWhole>
__global__ __launch_bounds__(kRowThreads) void verify_rows_kernel(
    const float* __restrict__ target, int T, int V, const int32_t* __restrict__ flat_token,
    const int32_t* __restrict__ flat_parent, float temperature, RowStats* __restrict__ stats,
    uint64_t* __restrict__ chunk_mass) {
    __shared__ int32_t s_kid_row[kKids];
    __shared__ int32_t s_kid_tok[kKids];
    __shared__ int s_nk;
    __shared__ uint64_t s_key[kRowWaves];
    __shared__ double s_red[kRowWaves];
    // kWhole: blockIdx.x = row i, quarters 0..3 in turn.  Otherwise blockIdx.x =
    // 8 * (kRowSplit * (i / 8) + q) + i % 8: the quarters of row i share an XCD.
    const int xb = blockIdx.x;
    const int i = kWhole ? xb : 8 * (xb / (8 * kRowSplit)) + (xb & 7);
    const int q_first = kWhole ? 0 : (xb >> 3) % kRowSplit, q_end = kWhole ? kRowSplit : q_first + 1;
    const int b = blockIdx.y, tid = threadIdx.x;
    if (i >= T || (q_first > 0 && !(temperature > 0.0f))) return;  // greedy needs the argmax only
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    const float* z = target + ((size_t)b * T + i) * (size_t)V;
    if (wid == 0) {
        const bool kid = lane < T && flat_parent[(size_t)b * T + lane] == i;
        const uint64_t bal = __ballot(kid);
        const int pos = __popcll(bal & ((1ull << lane) - 1ull));
        if (kid) {  // pos < 64 = kKids
            s_kid_row[pos] = lane;
            s_kid_tok[pos] = flat_token[(size_t)b * T + lane];
        }
        if (lane == 0) s_nk = __popcll(bal);
    }
    // maximum and argmax over the whole row: (logit, ~token) keys, order-free
    uint64_t best = 0;
    const bool vec = (V & 3) == 0 && ((uintptr_t)target & 15) == 0;
    if (vec) {
        const int n4 = V >> 2;
        const float4* z4 = reinterpret_cast<const float4*>(z);
        for (int j0 = 0; j0 < n4; j0 += kMaxBatch * kRowThreads) {
            float4 zr[kMaxBatch];
#pragma unroll
            for (int u = 0; u < kMaxBatch; ++u) {
                const int j = j0 + u * kRowThreads + tid;
                zr[u] = j < n4 ? z4[j] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
#pragma unroll
            for (int u = 0; u < kMaxBatch; ++u) {
                const int j = j0 + u * kRowThreads + tid;
                if (j < n4) {
                    const uint32_t t = 4u * (uint32_t)j;
                    uint64_t k0 = logit_key(zr[u].x, t), k1 = logit_key(zr[u].y, t + 1);
                    uint64_t k2 = logit_key(zr[u].z, t + 2), k3 = logit_key(zr[u].w, t + 3);
                    k0 = k1 > k0 ? k1 : k0;
                    k2 = k3 > k2 ? k3 : k2;
                    k0 = k2 > k0 ? k2 : k0;
                    best = k0 > best ? k0 : best;
                }
            }
        }
    } else {
        for (int t0 = 0; t0 < V; t0 += kRowBatch * kRowThreads) {
            float zr[kRowBatch];
#pragma unroll
            for (int u = 0; u < kRowBatch; ++u) {
                const int t = t0 + u * kRowThreads + tid;
                zr[u] = t < V ? z[t] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < kRowBatch; ++u) {
                const int t = t0 + u * kRowThreads + tid;
                if (t < V) {
                    const uint64_t key = logit_key(zr[u], (uint32_t)t);
                    best = key > best ? key : best;
                }
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
    // the children's logits, requested now so their latency overlaps the mass pass
    const float z_kid = q_first == 0 && temperature > 0.0f && tid < nk ? z[s_kid_tok[tid]] : 0.0f;
    if (temperature > 0.0f) {
        const double temp = (double)temperature;
        const bool unit_temp = temperature == 1.0f;  // x / 1 == x: skip the fp64 divide
        const double fscale = ldexp(1.0, fixed_shift(V));
        const int ch = (V + kRowChunks - 1) / kRowChunks;
        for (int q = q_first; q < q_end; ++q) {
            const int chunk = q * kWgChunks + (tid >> 1), half = tid & 1;
            const int c0 = min(V, chunk * ch), c1 = min(V, c0 + ch);
            // the pair of threads splits the chunk: the first takes the first
            // ceil(ch / 2) tokens rounded up to a multiple of 4, the second the rest
            const int hc = (((ch + 1) >> 1) + 3) & ~3;
            const int s0 = half == 0 ? c0 : min(c1, c0 + hc), s1 = half == 0 ? min(c1, c0 + hc) : c1;
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
            const bool cvec = vec && (ch & 3) == 0;
            for (int a0 = s0; a0 < s1; a0 += kRowBatch) {
                float zz[kRowBatch];
                if (cvec) {
    #pragma unroll
                    for (int u = 0; u < kRowBatch; u += 4) {
                        float4 v4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                        if (a0 + u < s1) v4 = *reinterpret_cast<const float4*>(z + a0 + u);
                        zz[u] = v4.x; zz[u + 1] = v4.y; zz[u + 2] = v4.z; zz[u + 3] = v4.w;
                    }
                } else {
    #pragma unroll
                    for (int u = 0; u < kRowBatch; ++u) zz[u] = a0 + u < s1 ? z[a0 + u] : 0.0f;
                }
                // bits o .. o + 31 of the chunk's child mask, which may straddle two words
                const int o = a0 - c0, wo = o >> 6, sh = o & 63;
                uint64_t lo = km[0], hi = km[1];
    #pragma unroll
                for (int w = 1; w < 4; ++w)
                    if (wo == w) {
                        lo = km[w];
                        hi = w + 1 < 4 ? km[w + 1] : 0;
                    }
                const uint32_t kb = (uint32_t)(sh == 0 ? lo : (lo >> sh) | (hi << (64 - sh)));
    #pragma unroll
                for (int u = 0; u < kRowBatch; ++u) {
                    if (a0 + u < s1) {
                        const double x = (double)zz[u] - (double)zmax;
                        const double e = exp_nonpos_f64(unit_temp ? x : x / temp);
                        fm += fixed_mass(e, fscale);
                        if (!((kb >> u) & 1u)) s += e;
                    }
                }
            }
            // the pair's integer masses add exactly
            const uint32_t flo = __shfl_xor((uint32_t)fm, 1, kWave), fhi = __shfl_xor((uint32_t)(fm >> 32), 1, kWave);
            fm += ((uint64_t)fhi << 32) | flo;
            if (half == 0) chunk_mass[((size_t)b * T + i) * kRowChunks + chunk] = fm;
            s = block_sum_f64(s, s_red);
            if (tid == 0) out->rest[q] = s;
            // the same expression as the chunk masses' (x / 1 == x exactly), so the bonus
            // draw can take a removed token's fixed-point mass out of its chunk exactly
            if (q == 0 && tid < nk)
                stats[(size_t)b * T + s_kid_row[tid]].e_kid = exp_nonpos_f64(((double)z_kid - (double)zmax) / temp);
        }  // quarters
    }
    if (q_first != 0) return;
    if (tid == 0) {
        out->zmax = zmax;
        out->argmax = amax;
    }
}

// ---------------------------------------------------------------------------
// K7
// ---------------------------------------------------------------------------
constexpr int kWalkThreads = 1024;
static_assert(kWalkThreads == kRowChunks, "one chunk mass per walk thread");
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
    const int32_t* __restrict__ flat_parent, float temperature, uint64_t seed, uint64_t step,
    const RowStats* __restrict__ stats,
    const uint64_t* __restrict__ chunk_mass, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ accept_path, int32_t* __restrict__ out_tokens) {
    __shared__ RowStats s_rs[EAGLE_MAX_TREE_ROWS];
    __shared__ int32_t s_tok[EAGLE_MAX_TREE_ROWS];
    __shared__ int32_t s_par[EAGLE_MAX_TREE_ROWS];
    __shared__ int32_t s_path[kMaxDepth];      // depth <= 255: accepted rows, -1 padded
    __shared__ int32_t s_out[kMaxDepth + 1];   // accepted tokens then the bonus, -1 padded
    __shared__ int s_bonus_row, s_len;
    __shared__ int32_t s_removed[kKids];   // distinct tokens rejected at the final row
    __shared__ double s_removed_e[kKids];  // and their fp64 masses
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
        if (tid < T) {
            s_tok[tid] = flat_token[(size_t)b * T + tid];
            s_par[tid] = flat_parent[(size_t)b * T + tid];
        }
        if (tid < depth) s_path[tid] = -1;
        if (tid <= depth) s_out[tid] = -1;
    }
    __syncthreads();

    // The walk, by wave 0: lane j evaluates row j when it is a child of the
    // current row; its slot is its index among the row's children (flattened
    // order).  The sequential rule takes the first child whose test passes, and
    // child c's test depends only on c (the children before it are the ones
    // already rejected), so the lowest set bit of the ballot is that child.  The
    // tokens not yet rejected when child c is tested are the non-children (mass
    // `rest`) and the tokens whose first carrier among the children is c or later;
    // a child whose token an earlier sibling carried has probability 0.
    if (tid < kWave) {
        // bit j: no earlier sibling of row j carries row j's token.  Each row (but the
        // root) has the key parent * 2^tb + token; the rows sharing a lane's key are
        // found bit by bit (for every key bit, the rows that agree with the lane on
        // it, from one ballot), with no per-row loop.
        int tb = 0;
        while ((1 << tb) < V) ++tb;  // token bits (V <= 2^18, parent < 64: 24 bits at most)
        const bool row_ok = lane >= 1 && lane < T;
        const uint32_t key = row_ok ? ((uint32_t)s_par[lane] << tb) | (uint32_t)s_tok[lane] : 0u;
        uint64_t same = __ballot(row_ok);
        for (int bit = 0; bit < tb + 6; ++bit) {
            const bool on = (key >> bit) & 1u;
            const uint64_t with_bit = __ballot(on);
            same &= on ? with_bit : ~with_bit;
        }
        const bool first = lane < T && (lane == 0 || (same & ((1ull << lane) - 1ull)) == 0);
        const uint64_t firsts = __ballot(first);
        int cur = 0, len = 0;
        while (true) {
            const RowStats& R = s_rs[cur];
            const bool is_kid = lane < T && s_par[lane] == cur;
            const uint64_t kids = __ballot(is_kid);
            int next = -1;
            if (len < depth && kids) {
                bool pass = false;
                if (is_kid) {
                    if (!sampled) {
                        pass = s_tok[lane] == R.argmax;
                    } else {
                        double denom = ((R.rest[0] + R.rest[1]) + R.rest[2]) + R.rest[3];
                        for (uint64_t m = (kids & firsts) >> lane; m; m &= m - 1) {
                            const int j = lane + __ffsll((unsigned long long)m) - 1;
                            denom += s_rs[j].e_kid;
                        }
                        const double ratio = ((firsts >> lane) & 1) ? s_rs[lane].e_kid / denom : 0.0;
                        const int slot = __popcll(kids & ((1ull << lane) - 1ull));
                        const double u = decision_uniform(seed, step, (uint32_t)b, (uint32_t)cur, (uint32_t)slot);
                        pass = u < ratio;
                    }
                }
                const uint64_t bal = __ballot(pass);
                if (bal) next = __ffsll((unsigned long long)bal) - 1;
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
            // every child of the final row was tested and rejected (none when it is a
            // leaf, or when the path has reached the depth limit): its distinct tokens
            const bool rem = len < depth && is_kid && ((firsts >> lane) & 1);
            const uint64_t rbal = __ballot(rem);
            if (rem) {
                const int c = __popcll(rbal & ((1ull << lane) - 1ull));
                s_removed[c] = s_tok[lane];
                s_removed_e[c] = s_rs[lane].e_kid;
            }
            if (lane == 0) {
                if (!sampled) s_out[len] = R.argmax;
                s_bonus_row = cur;
                s_len = len;
                s_n_removed = __popcll(rbal);
            }
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
            const int tok = s_removed[c];  // distinct tokens: each leaves its chunk once
            if (tok >= c0 && tok < c1) cs -= fixed_mass(s_removed_e[c], fscale);
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
    return stats_bytes(cfg) + (size_t)cfg.batch * (size_t)(cfg.n + 1) * kRowChunks * sizeof(uint64_t);
}

hipError_t launch_verify(const eagle_tree_cfg& cfg, const float* target, const int32_t* flat_token,
                         const int32_t* flat_parent, float temperature, uint64_t seed,
                         uint64_t step, int32_t* accept_len, int32_t* accept_path,
                         int32_t* out_tokens, void* workspace, hipStream_t stream) {
    const int T = cfg.n + 1;
    RowStats* stats = (RowStats*)workspace;
    uint64_t* chunk_mass = (uint64_t*)((unsigned char*)workspace + stats_bytes(cfg));
    if ((int64_t)cfg.batch * T >= kWholeRowsFrom) {
        verify_rows_kernel<true><<<dim3(T, cfg.batch), kRowThreads, 0, stream>>>(
            target, T, cfg.vocab, flat_token, flat_parent, temperature, stats, chunk_mass);
    } else {
        // rows padded to a multiple of 8 so the quarters of a row share an XCD
        const int row_groups = (T + 7) / 8;
        verify_rows_kernel<false><<<dim3(8 * kRowSplit * row_groups, cfg.batch), kRowThreads, 0, stream>>>(
            target, T, cfg.vocab, flat_token, flat_parent, temperature, stats, chunk_mass);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    verify_walk_kernel<<<cfg.batch, kWalkThreads, 0, stream>>>(
        target, T, cfg.vocab, cfg.depth, flat_token, flat_parent, temperature, seed, step, stats, chunk_mass,
        accept_len, accept_path, out_tokens);
    return hipGetLastError();
}

}  // namespace eagle
