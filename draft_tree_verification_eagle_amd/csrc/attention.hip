// Tree attention for gfx950 (MI355X).
//
// Page: EAGLE-2 page (news write-up of "EAGLE-2: Faster Inference of Language
// Models with Dynamic Draft Trees"), the passage after the two stages: every
// flattened draft token attends to the whole context and, inside the tree, to its
// own ancestors only (the It / is / a / has example), so one target pass verifies
// every branch at once.
//
// BF16 kernel design (head_dim 128):
//  * Work unit = (sequence, KV head, group of 64 packed query rows); the packed
//    rows of a KV head are its G = Hq/Hkv query heads x T tree rows.  Each unit's
//    keys are cut into 64-key tiles.  All (unit, tile) pairs form one linear list
//    that is split evenly over exactly 256 workgroups (one per CU), so the work
//    is balanced whatever the context lengths.  Workgroup index -> position in the
//    list is XCD-aware: workgroups on one XCD (blockIdx % 8) take one contiguous
//    stretch, so the few units they share merge through one L2.
//  * K, V (and, at a unit's first tile, Q and the 64 mask words) are streamed
//    HBM -> LDS by direct 16-byte global_load_lds, three stages deep, every load
//    instruction covering 1 KB of contiguous rows.  Rows are stored with a 16-byte
//    chunk XOR swizzle that keeps the MFMA operand reads conflict-free.
//  * 4 waves = 2 query halves x 2 key halves of each tile.  S^T = K Q^T and
//    O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16; V^T operands come straight
//    from the row-major V tile through ds_read_b64_tr_b16.  The key order inside
//    the S^T block is permuted so each half-wave's probabilities are the PV
//    operand's 8 consecutive keys, with no register shuffles.
//  * Online softmax in fp32 (base 2), probabilities rounded to bf16 for PV.
//  * A workgroup whose stretch covers a whole unit writes the output directly;
//    otherwise it writes an fp32 partial (m, l, O) and the last workgroup to
//    arrive at that unit (atomic counter) merges the partials and resets the
//    counter.
#include "device_common.hpp"
#include "launchers.hpp"

namespace eagle {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_ADDR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kD = 128;
constexpr int kTileKeys = 64;
constexpr int kUnitRows = 64;
constexpr int kThreads = 256;
constexpr int kStages = 3;
constexpr int kRowBytes = kD * 2;                    // 256
constexpr int kTileBytes = kTileKeys * kRowBytes;    // 16 KB
constexpr int kQBytes = kUnitRows * kRowBytes;       // 16 KB
constexpr int kMaskBytes = kUnitRows * 8;            // 512 B
constexpr int kOffV = kTileBytes;
constexpr int kOffQ = 2 * kTileBytes;
constexpr int kOffMask = 2 * kTileBytes + kQBytes;
constexpr int kStageBytes = kOffMask + kMaskBytes;   // 49664 B
constexpr int kKVLoadsPerTile = 2 * kTileBytes / (kThreads * 16);  // 8 per thread
constexpr int kGridWG = 256;                         // multiple of the 8 XCDs
constexpr int kMaxAttnBatch = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

static_assert(kKVLoadsPerTile == 8 && kStages == 3,
              "the stage barrier assumes one 8-load stage may stay in flight");
static_assert(2 * kTileBytes <= kStageBytes, "merge buffer must fit in one stage");

// 16-byte chunk position of logical chunk c in LDS row r: c ^ swz(r).
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// S^T block row i holds key (i with bits 2 and 3 exchanged).
__device__ __forceinline__ int key_of_row(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// Direct HBM -> LDS loads and the pipeline barrier are written as inline asm so
// the compiler neither tracks them nor serialises LDS reads behind them; the
// explicit s_waitcnt vmcnt(n) before each barrier is what orders a stage's
// loads before its use.  Nothing else in this kernel uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_b128(const void* gptr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gptr)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const void* gptr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gptr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most one stage's K/V loads (8 per thread) are in flight, then
// barrier; the tail of the loop waits for everything.
__device__ __forceinline__ void stage_barrier_one_in_flight() {
    asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void stage_barrier_drained() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

struct AttnArgs {
    const __bf16* q;
    const __bf16* k;
    const __bf16* v;
    const uint64_t* mask;
    __bf16* o;
    float* lse;
    const int32_t* ctx_len;
    const int64_t* kv_row_off;
    float* part_o;       // [slots][64][128]
    float* part_ml;      // [slots][2][64]
    uint32_t* counters;  // [units]
    int64_t kv_rows_total;
    int B, T, Hq, Hkv, G, RG;
    float scale_log2;
};

struct TileRef {
    int b, unit, kt, ntiles;  // unit: index inside the sequence (g * RG + rg)
    int64_t unit_begin;       // linear index of the unit's first tile
};

__device__ __forceinline__ TileRef decode_tile(int64_t t, const int64_t* seq_off, const int* ntiles,
                                               int B) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seq_off[mid] <= t) lo = mid; else hi = mid - 1;
    }
    TileRef r;
    r.b = lo;
    r.ntiles = ntiles[lo];
    const int64_t local = t - seq_off[lo];
    r.unit = (int)(local / r.ntiles);
    r.kt = (int)(local - (int64_t)r.unit * r.ntiles);
    r.unit_begin = seq_off[lo] + (int64_t)r.unit * r.ntiles;
    return r;
}

// Workgroup (in list order) whose stretch [total*v/n, total*(v+1)/n) holds tile t.
__device__ __forceinline__ int stretch_of(int64_t t, int64_t total, int nwg) {
    int v = (int)((t * nwg) / total);
    while (v + 1 < nwg && total * (v + 1) / nwg <= t) ++v;
    while (v > 0 && total * v / nwg > t) --v;
    return v;
}

__device__ __forceinline__ int64_t shfl_up_i64(int64_t x, int off) {
    const uint32_t lo = __shfl_up((uint32_t)x, off, kWave);
    const uint32_t hi = __shfl_up((uint32_t)((uint64_t)x >> 32), off, kWave);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int64_t shfl_i64(int64_t x, int src) {
    const uint32_t lo = __shfl((uint32_t)x, src, kWave);
    const uint32_t hi = __shfl((uint32_t)((uint64_t)x >> 32), src, kWave);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Issue the direct-to-LDS loads of one tile (and, at a unit's first tile in this
// workgroup, its Q rows and mask words) into stage memory `st`.
__device__ __forceinline__ void issue_tile(const AttnArgs& a, const TileRef& r, bool with_q,
                                           unsigned char* st, int wid, int lane, const int* s_ctx,
                                           const int64_t* s_row0) {
    const int g = r.unit / a.RG, rg = r.unit - g * a.RG;
    const int ctx = s_ctx[r.b];
    const int S = ctx + a.T;
    const int64_t row0 = s_row0[r.b];
    const int key0 = r.kt * kTileKeys;
    const __bf16* kb = a.k + ((int64_t)g * a.kv_rows_total + row0) * kD;
    const __bf16* vb = a.v + ((int64_t)g * a.kv_rows_total + row0) * kD;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int blk = n * 4 + wid;  // 16 blocks of 4 rows
        const int lrow = blk * 4 + (lane >> 4);
        int key = key0 + lrow;
        key = key < S ? key : S - 1;
        const int c = (lane & 15) ^ swz(lrow);
        dma_b128(kb + (int64_t)key * kD + c * 8, lds_u32(st + blk * 1024));
        dma_b128(vb + (int64_t)key * kD + c * 8, lds_u32(st + kOffV + blk * 1024));
    }
    if (with_q) {
        const int rows = a.G * a.T;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int blk = n * 4 + wid;
            const int rho = blk * 4 + (lane >> 4);
            int rp = rg * kUnitRows + rho;
            rp = rp < rows ? rp : 0;
            const int gi = rp / a.T, i = rp - gi * a.T;
            const int hq = g * a.G + gi;
            const __bf16* qrow = a.q + (((int64_t)r.b * a.T + i) * a.Hq + hq) * kD;
            const int c = (lane & 15) ^ swz(rho);
            dma_b128(qrow + c * 8, lds_u32(st + kOffQ + blk * 1024));
        }
        if (wid == 0) {
            int rp = rg * kUnitRows + lane;
            rp = rp < rows ? rp : 0;
            const int i = rp % a.T;
            const uint32_t* mw = (const uint32_t*)(a.mask + (int64_t)r.b * a.T + i);
            dma_b32(mw, lds_u32(st + kOffMask));
            dma_b32(mw + 1, lds_u32(st + kOffMask + 256));
        }
    }
}

__global__ __launch_bounds__(kThreads, 1) void tree_attn_bf16_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStageBytes];
    __shared__ int64_t s_seq_off[kMaxAttnBatch + 1];
    __shared__ int s_ntiles[kMaxAttnBatch];
    __shared__ int s_ctx[kMaxAttnBatch];
    __shared__ int64_t s_row0[kMaxAttnBatch];
    __shared__ float s_ml[2][2][kWave];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
    const int rb = wid & 1, ks = wid >> 1;
    const int l32 = lane & 31, h2 = lane >> 5;
    const int B = a.B, T = a.T;
    const int units_per_seq = a.Hkv * a.RG;

    // ---- schedule: tiles per sequence, prefix over the (unit, tile) list ----
    // (context lengths and cache offsets are cached in LDS: the tile loop issues no
    // vector-memory loads of its own besides the staged DMA)
    for (int b = tid; b < B; b += kThreads) {
        const int c = a.ctx_len[b];
        s_ctx[b] = c;
        s_row0[b] = a.kv_row_off[b];
        s_ntiles[b] = (c + T + kTileKeys - 1) / kTileKeys;
    }
    __syncthreads();
    if (wid == 0) {
        int64_t run = 0;
        for (int base = 0; base < B; base += kWave) {
            const int b = base + lane;
            const int64_t v = (b < B) ? (int64_t)s_ntiles[b] * units_per_seq : 0;
            int64_t incl = v;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const int64_t o = shfl_up_i64(incl, off);
                if (lane >= off) incl += o;
            }
            if (b < B) s_seq_off[b] = run + incl - v;
            run += shfl_i64(incl, kWave - 1);
        }
        if (lane == 0) s_seq_off[B] = run;
    }
    __syncthreads();
    const int64_t total = s_seq_off[B];
    // Workgroups taking part: at most one per tile, so that every stretch is
    // non-empty and the workgroups overlapping a unit are exactly stretch_of(first
    // tile) .. stretch_of(last tile).
    const int nwg = total < (int64_t)gridDim.x ? (int)total : (int)gridDim.x;
    const int vwg = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    if (vwg >= nwg) return;
    const int64_t t_begin = total * vwg / nwg, t_end = total * (vwg + 1) / nwg;
    const int ntile = (int)(t_end - t_begin);

    // ---- prologue: first kStages-1 tiles in flight ----
    for (int s = 0; s < kStages - 1 && s < ntile; ++s) {
        const TileRef r = decode_tile(t_begin + s, s_seq_off, s_ntiles, B);
        issue_tile(a, r, s == 0 || r.kt == 0, smem + s * kStageBytes, wid, lane, s_ctx, s_row0);
    }

    f32x16 oacc[4];
    bf16x8 qcur[8];
    uint64_t mword = 0;
    float m_run = -INFINITY, l_run = 0.0f;
    const int krow = 32 * ks + key_of_row(l32);
    const int g16 = lane >> 4, i16 = lane & 15, rr = i16 >> 2, cc = i16 & 3, dh = g16 & 1;

    for (int it = 0; it < ntile; ++it) {
        const int64_t t = t_begin + it;
        if (it + 1 < ntile) stage_barrier_one_in_flight(); else stage_barrier_drained();
        if (it + kStages - 1 < ntile) {
            const TileRef rn = decode_tile(t + kStages - 1, s_seq_off, s_ntiles, B);
            issue_tile(a, rn, rn.kt == 0, smem + ((it + kStages - 1) % kStages) * kStageBytes, wid, lane,
                       s_ctx, s_row0);
        }
        const TileRef r = decode_tile(t, s_seq_off, s_ntiles, B);
        unsigned char* st = smem + (it % kStages) * kStageBytes;
        const bool seg_start = (it == 0) || (r.kt == 0);
        const bool seg_end = (it == ntile - 1) || (r.kt == r.ntiles - 1);
        const int ctx = s_ctx[r.b];
        const int S = ctx + T;
        const int key0 = r.kt * kTileKeys;

        if (seg_start) {
            const int rho = 32 * rb + l32;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int c = (2 * kk + h2) ^ swz(rho);
                qcur[kk] = *(const bf16x8*)(st + kOffQ + rho * kRowBytes + c * 16);
            }
            const uint32_t* mw = (const uint32_t*)(st + kOffMask);
            mword = (uint64_t)mw[rho] | ((uint64_t)mw[64 + rho] << 32);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
            m_run = -INFINITY;
            l_run = 0.0f;
        }

        // ---- S^T = K Q^T for this wave's 32 keys x 32 query rows ----
        f32x16 sacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int c = (2 * kk + h2) ^ swz(krow);
            const bf16x8 ka = *(const bf16x8*)(st + krow * kRowBytes + c * 16);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qcur[kk], sacc, 0, 0, 0);
        }

        // ---- online softmax (base 2); lane = one query, 16 of its keys ----
        float sv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) sv[e] = sacc[e] * a.scale_log2;
        if (key0 + kTileKeys > ctx) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = key0 + 32 * ks + 16 * (e >> 3) + 8 * h2 + (e & 7);
                bool vis = key < ctx;
                if (!vis && key < S) vis = (mword >> (key - ctx)) & 1ull;
                if (!vis) sv[e] = -INFINITY;
            }
        }
        float mx = sv[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sv[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float psum = 0.0f;
        bf16x8 pb[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float p = exp2f(sv[e] - m_use);
            psum += p;
            pb[e >> 3][e & 7] = (__bf16)p;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;

        // ---- O^T += V^T P^T; V^T operands by LDS transpose reads ----
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int vr1 = 32 * ks + 16 * j + 8 * h2 + rr;
            const int vr2 = vr1 + 4;
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const int c = 4 * db + 2 * dh + (cc >> 1);
                const int off = (cc & 1) * 8;
                const unsigned char* p1 = st + kOffV + vr1 * kRowBytes + ((c ^ swz(vr1)) << 4) + off;
                const unsigned char* p2 = st + kOffV + vr2 * kRowBytes + ((c ^ swz(vr2)) << 4) + off;
                const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_ADDR(i16x4, p1));
                const i16x4 a2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_ADDR(i16x4, p2));
                const i16x8 a8 = {a1[0], a1[1], a1[2], a1[3], a2[0], a2[1], a2[2], a2[3]};
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb[j],
                                                                   oacc[db], 0, 0, 0);
            }
        }

        if (!seg_end) continue;

        // ---- end of this workgroup's part of a unit: merge the two key halves ----
        __syncthreads();  // every wave is done with this stage: reuse it
        float* mb = (float*)st;
        if (ks == 1) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) mb[((rb * 64) + db * 16 + e) * kWave + lane] = oacc[db][e];
            s_ml[rb][0][lane] = m_run;
            s_ml[rb][1][lane] = l_run;
        }
        __syncthreads();
        const int g = r.unit / a.RG, rg = r.unit - g * a.RG;
        const int unit_global = r.b * units_per_seq + r.unit;
        const bool whole = r.unit_begin >= t_begin && r.unit_begin + r.ntiles <= t_end;
        const int rows = a.G * T;
        const int rho = 32 * rb + l32;
        const int rp = rg * kUnitRows + rho;
        if (ks == 0) {
            const float m1 = s_ml[rb][0][lane], l1 = s_ml[rb][1][lane];
            const float M = fmaxf(m_run, m1);
            const float Mu = (M == -INFINITY) ? 0.0f : M;
            const float a0 = exp2f(m_run - Mu), a1 = exp2f(m1 - Mu);
            const float lsum = l_run * a0 + l1 * a1;
            const float ltot = lsum + __shfl_xor(lsum, 32, kWave);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    oacc[db][e] = oacc[db][e] * a0 + mb[((rb * 64) + db * 16 + e) * kWave + lane] * a1;
            if (whole) {
                if (rp < rows) {
                    const int gi = rp / T, i = rp - gi * T;
                    const int hq = g * a.G + gi;
                    const float inv = 1.0f / ltot;
                    __bf16* orow = a.o + (((int64_t)r.b * T + i) * a.Hq + hq) * kD;
#pragma unroll
                    for (int db = 0; db < 4; ++db)
#pragma unroll
                        for (int qd = 0; qd < 4; ++qd) {
                            bf16x4 w;
#pragma unroll
                            for (int x = 0; x < 4; ++x) w[x] = (__bf16)(oacc[db][4 * qd + x] * inv);
                            *(bf16x4*)(orow + 32 * db + 8 * qd + 4 * h2) = w;
                        }
                    if (h2 == 0 && a.lse)
                        a.lse[((int64_t)r.b * T + i) * a.Hq + hq] = (M + log2f(ltot)) * kLn2;
                }
            } else {
                const int64_t slot = (int64_t)unit_global + vwg;
                float* po = a.part_o + slot * (kUnitRows * kD) + (int64_t)rho * kD;
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        f32x4 w;
#pragma unroll
                        for (int x = 0; x < 4; ++x) w[x] = oacc[db][4 * qd + x];
                        *(f32x4*)(po + 32 * db + 8 * qd + 4 * h2) = w;
                    }
                if (h2 == 0) {
                    a.part_ml[slot * 128 + rho] = M;
                    a.part_ml[slot * 128 + 64 + rho] = ltot;
                }
            }
        }
        if (whole) continue;

        // ---- partial written: the last workgroup on this unit merges ----
        __threadfence();
        __syncthreads();
        const int vf = stretch_of(r.unit_begin, total, nwg);
        const int vl = stretch_of(r.unit_begin + r.ntiles - 1, total, nwg);
        if (tid == 0) {
            const uint32_t old = atomicAdd(&a.counters[unit_global], 1u);
            s_last = (old == (uint32_t)(vl - vf));
        }
        __syncthreads();
        if (!s_last) continue;
        __threadfence();
        {
            const int row = tid >> 2, dq = tid & 3;  // 64 rows x 4 quarters of 32 dims
            const int rpm = rg * kUnitRows + row;
            if (rpm < rows) {
                float M = -INFINITY;
                for (int v = vf; v <= vl; ++v)
                    M = fmaxf(M, __builtin_nontemporal_load(&a.part_ml[((int64_t)unit_global + v) * 128 + row]));
                float L = 0.0f;
                float acc[32];
#pragma unroll
                for (int x = 0; x < 32; ++x) acc[x] = 0.0f;
                for (int v = vf; v <= vl; ++v) {
                    const int64_t slot = (int64_t)unit_global + v;
                    const float ms = __builtin_nontemporal_load(&a.part_ml[slot * 128 + row]);
                    const float ls = __builtin_nontemporal_load(&a.part_ml[slot * 128 + 64 + row]);
                    const float w = exp2f(ms - M);
                    L += ls * w;
                    const float* po = a.part_o + slot * (kUnitRows * kD) + (int64_t)row * kD + 32 * dq;
#pragma unroll
                    for (int x = 0; x < 32; x += 4) {
                        const f32x4 pv = __builtin_nontemporal_load((const f32x4*)(po + x));
                        acc[x] += pv[0] * w;
                        acc[x + 1] += pv[1] * w;
                        acc[x + 2] += pv[2] * w;
                        acc[x + 3] += pv[3] * w;
                    }
                }
                const int gi = rpm / T, i = rpm - gi * T;
                const int hq = g * a.G + gi;
                const float inv = 1.0f / L;
                __bf16* orow = a.o + (((int64_t)r.b * T + i) * a.Hq + hq) * kD + 32 * dq;
#pragma unroll
                for (int x = 0; x < 32; x += 8) {
                    bf16x8 w;
#pragma unroll
                    for (int y = 0; y < 8; ++y) w[y] = (__bf16)(acc[x + y] * inv);
                    *(bf16x8*)(orow + x) = w;
                }
                if (dq == 0 && a.lse) a.lse[((int64_t)r.b * T + i) * a.Hq + hq] = (M + log2f(L)) * kLn2;
            }
            if (tid == 0) a.counters[unit_global] = 0u;
        }
    }
}

// ---------------------------------------------------------------------------
// FP32 path: one wave per (tree row, query head); lane = head dimension.
// ---------------------------------------------------------------------------
struct AttnF32Args {
    const float* q;
    const float* k;
    const float* v;
    const uint64_t* mask;
    float* o;
    float* lse;
    const int32_t* ctx_len;
    const int64_t* kv_row_off;
    int64_t kv_rows_total;
    int T, Hq, G, D;
    float scale;
};

__global__ __launch_bounds__(256) void tree_attn_f32_kernel(AttnF32Args a) {
    const int i = blockIdx.x, b = blockIdx.z;
    const int wid = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int hq = blockIdx.y * 4 + wid;
    if (hq >= a.Hq) return;
    const int g = hq / a.G;
    const int ctx = a.ctx_len[b], S = ctx + a.T, D = a.D;
    const uint64_t mword = a.mask[(int64_t)b * a.T + i];
    const float* qrow = a.q + (((int64_t)b * a.T + i) * a.Hq + hq) * D;
    const float q0 = lane < D ? qrow[lane] : 0.0f;
    const float q1 = lane + kWave < D ? qrow[lane + kWave] : 0.0f;
    const int64_t base = ((int64_t)g * a.kv_rows_total + a.kv_row_off[b]) * D;
    float m = -INFINITY, l = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int c = 0; c < S; ++c) {
        if (c >= ctx && !((mword >> (c - ctx)) & 1ull)) continue;
        const float* kr = a.k + base + (int64_t)c * D;
        const float* vr = a.v + base + (int64_t)c * D;
        float part = 0.0f;
        if (lane < D) part += q0 * kr[lane];
        if (lane + kWave < D) part += q1 * kr[lane + kWave];
        const float s = wave_sum_f32(part) * a.scale;
        const float m_new = fmaxf(m, s);
        const float alpha = expf(m - m_new);
        const float p = expf(s - m_new);
        l = l * alpha + p;
        o0 = o0 * alpha + (lane < D ? p * vr[lane] : 0.0f);
        o1 = o1 * alpha + (lane + kWave < D ? p * vr[lane + kWave] : 0.0f);
        m = m_new;
    }
    float* orow = a.o + (((int64_t)b * a.T + i) * a.Hq + hq) * D;
    if (lane < D) orow[lane] = o0 / l;
    if (lane + kWave < D) orow[lane + kWave] = o1 / l;
    if (lane == 0 && a.lse) a.lse[((int64_t)b * a.T + i) * a.Hq + hq] = m + logf(l);
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
    size_t part_o, part_ml, counters, total;
};

WsLayout ws_layout(const eagle_attn_desc& d) {
    WsLayout w{0, 0, 0, 0};
    if (d.dtype != EAGLE_BF16) return w;
    const int G = d.n_q_heads / d.n_kv_heads;
    const int RG = (G * d.T + kUnitRows - 1) / kUnitRows;
    const size_t units = (size_t)d.batch * d.n_kv_heads * RG;
    const size_t slots = units + kGridWG;
    w.part_o = 0;
    w.part_ml = align_up(slots * kUnitRows * kD * sizeof(float));
    w.counters = w.part_ml + align_up(slots * 2 * kUnitRows * sizeof(float));
    w.total = w.counters + align_up(units * sizeof(uint32_t));
    return w;
}

}  // namespace

size_t attention_workspace_bytes(const eagle_attn_desc& d) { return ws_layout(d).total; }

hipError_t launch_attention(const eagle_attn_desc& d, const void* q, const void* k, const void* v,
                            const uint64_t* mask, void* o, float* lse, void* workspace,
                            hipStream_t stream) {
    const float scale = d.scale != 0.0f ? d.scale : 1.0f / sqrtf((float)d.head_dim);
    const int G = d.n_q_heads / d.n_kv_heads;
    if (d.dtype == EAGLE_F32) {
        AttnF32Args a;
        a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v;
        a.mask = mask; a.o = (float*)o; a.lse = lse;
        a.ctx_len = d.ctx_len; a.kv_row_off = d.kv_row_off; a.kv_rows_total = d.kv_rows_total;
        a.T = d.T; a.Hq = d.n_q_heads; a.G = G; a.D = d.head_dim; a.scale = scale;
        tree_attn_f32_kernel<<<dim3(d.T, (d.n_q_heads + 3) / 4, d.batch), 256, 0, stream>>>(a);
        return hipGetLastError();
    }
    const WsLayout w = ws_layout(d);
    unsigned char* ws = (unsigned char*)workspace;
    AttnArgs a;
    a.q = (const __bf16*)q; a.k = (const __bf16*)k; a.v = (const __bf16*)v;
    a.mask = mask; a.o = (__bf16*)o; a.lse = lse;
    a.ctx_len = d.ctx_len; a.kv_row_off = d.kv_row_off;
    a.part_o = (float*)(ws + w.part_o);
    a.part_ml = (float*)(ws + w.part_ml);
    a.counters = (uint32_t*)(ws + w.counters);
    a.kv_rows_total = d.kv_rows_total;
    a.B = d.batch; a.T = d.T; a.Hq = d.n_q_heads; a.Hkv = d.n_kv_heads; a.G = G;
    a.RG = (G * d.T + kUnitRows - 1) / kUnitRows;
    a.scale_log2 = scale * kLog2e;
    tree_attn_bf16_kernel<<<kGridWG, kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

int attention_max_batch() { return kMaxAttnBatch; }

}  // namespace eagle
