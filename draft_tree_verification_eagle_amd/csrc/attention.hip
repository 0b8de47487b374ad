// Tree attention for gfx950 (MI355X).
//
// Page: EAGLE-2 page (news write-up of "EAGLE-2: Faster Inference of Language
// Models with Dynamic Draft Trees"), the passage after the two stages: every
// flattened draft token attends to the whole context and, inside the tree, to its
// own ancestors only (the It / is / a / has example), so one target pass verifies
// every branch at once.
//
// BF16 path (head_dim 128): per sequence, a main kernel and a merge kernel.
//  * Work unit = (KV head, group of 64 packed query rows); the packed rows of a KV
//    head are its G = Hq/Hkv query heads x T tree rows.  The keys of all units
//    (ctx + T each) form one linear list split evenly over 256 workgroups, one per
//    CU, so every workgroup streams the same number of K/V bytes.  Workgroup
//    index -> list position is XCD-aware (blockIdx % 8 picks the XCD): each XCD
//    takes one contiguous stretch, so the units that share K/V rows (GQA) read
//    them through one L2.  A workgroup walks its stretch in tiles of <= 64 keys.
//  * K and V stream HBM -> LDS by direct 16-byte global_load_lds (no register
//    staging), four stages deep: three tiles (96 KB) in flight per CU while one
//    is computed.  Each load instruction covers 1 KB of contiguous rows.  Every
//    tile issues the same 8 loads per thread (the stage barriers count them):
//    lanes for rows past a short tile re-read the tile's last row, which the
//    softmax masks out and which costs no extra HBM traffic.  LDS rows use a
//    16-byte chunk XOR swizzle that keeps the MFMA operand reads conflict-free.
//  * Q stays in registers for a whole segment.  The first segment's Q is loaded
//    directly; a later segment's Q rides into an LDS slot with its first tile.
//  * 4 waves = 2 query halves x 2 key halves of a tile.  S^T = K Q^T and
//    O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16; V^T operands come straight
//    from the row-major V tile through ds_read_b64_tr_b16.  The key order inside
//    the S^T block is permuted so each half-wave's probabilities are the PV
//    operand's 8 consecutive keys, with no register shuffles.  Online softmax in
//    fp32 (base 2); probabilities rounded to bf16 for PV.
//  * A workgroup whose stretch holds a whole unit writes the output; otherwise
//    it writes a partial: row max and row sum in fp32 and the normalised row in
//    fp16 (relative rounding 2^-11, inside the bf16 output's own).  The merge
//    kernel, on the same stream, combines the partials of split units, so no
//    workgroup ever waits for another.
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
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_ADDR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kD = 128;
constexpr int kTileKeys = 64;
constexpr int kUnitRows = 64;
constexpr int kThreads = 256;
constexpr int kStages = 4;
constexpr int kGridWG = 256;                         // one per CU, multiple of the 8 XCDs
constexpr int kRowBytes = kD * 2;                    // 256
constexpr int kTileBytes = kTileKeys * kRowBytes;    // 16 KB
constexpr int kStageBytes = 2 * kTileBytes;          // K tile | V tile
constexpr int kQBytes = kUnitRows * kRowBytes;       // 16 KB
constexpr int kKVLoads = 2 * kTileBytes / (kThreads * 16);  // 8 per thread per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

static_assert(kKVLoads == 8 && kStages == 4, "the stage barriers assume 8 loads per tile, 4 stages");

// 16-byte chunk position of logical chunk c in LDS row r: c ^ swz(r).
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// S^T block row i holds key (i with bits 2 and 3 exchanged).
__device__ __forceinline__ int key_of_row(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Direct HBM -> LDS loads and the pipeline barriers are inline asm: the compiler
// neither tracks these loads nor serialises LDS reads behind them.  The stage
// barrier's explicit vmcnt(n) is what orders a stage's loads before its use:
// loads complete in issue order, so waiting until at most n loads are in flight,
// with n the loads issued after the stage's own, makes that stage complete.
// Nothing else in this kernel uses M0.
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
__device__ __forceinline__ void barrier_vm16() { asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void barrier_vm8() { asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void barrier_vm0() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Barrier for LDS traffic only (leaves the K/V loads in flight).
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt vmcnt(0) as the compiler sees it: after this, registers filled by
// ordinary loads count as complete, so no wait for them is carried into the
// tile loop (where any vmcnt wait would also drain the K/V pipeline).
__device__ __forceinline__ void wait_direct_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

// One sequence.  Pointers are already offset to the sequence.
struct AttnArgs {
    const __bf16* q;           // [T][Hq][D]
    const __bf16* k;           // cache base; the sequence's rows start at *kv_row_off
    const __bf16* v;
    const uint64_t* mask;      // [T]
    __bf16* o;                 // [T][Hq][D]
    float* lse;                // [T][Hq] or null
    const int32_t* ctx_len;    // [1]
    const int64_t* kv_row_off; // [1]
    _Float16* part_o;          // [slots][64][128], normalised rows
    float* part_ml;            // [slots][2][64]: row max (base 2), row sum
    int64_t kv_rows_total;
    int T, Hq, Hkv, G, RG;
    float scale_log2;
};

// Workgroup (in list order) whose stretch [total*v/n, total*(v+1)/n) holds key x.
__device__ __forceinline__ int stretch_of(int64_t x, int64_t total, int nwg) {
    int v = (int)((x * nwg) / total);
    while (v + 1 < nwg && total * (v + 1) / nwg <= x) ++v;
    while (v > 0 && total * v / nwg > x) --v;
    return v;
}

// Tile at list position x: unit, first key, key count, segment flags.
struct Tile {
    int unit, key0, nkeys;
    bool seg_start, seg_end;
};
__device__ __forceinline__ Tile tile_at(int64_t x, int64_t x_begin, int64_t x_end, int S) {
    Tile t;
    t.unit = uni((int)(x / S));
    t.key0 = uni((int)(x - (int64_t)t.unit * S));
    int n = kTileKeys;
    if (S - t.key0 < n) n = S - t.key0;
    if (x_end - x < n) n = (int)(x_end - x);
    t.nkeys = uni(n);
    t.seg_start = (x == x_begin) || (t.key0 == 0);
    t.seg_end = (x + t.nkeys == x_end) || (t.key0 + t.nkeys == S);
    return t;
}

// Packed query row -> (tree row, query head); rows past G*T map to row 0.
__device__ __forceinline__ void query_row(const AttnArgs& a, int g, int rp, int& i, int& hq) {
    if (rp >= a.G * a.T) rp = 0;
    const int gi = rp / a.T;
    i = rp - gi * a.T;
    hq = g * a.G + gi;
}

// Direct-to-LDS loads of one tile's K and V rows: always 8 per thread; rows
// past nkeys re-read row nkeys - 1.
__device__ __forceinline__ void issue_kv(const AttnArgs& a, const Tile& t, int64_t row0, unsigned char* st,
                                         int wid, int lane) {
    const int g = t.unit / a.RG;
    const int64_t base = ((int64_t)g * a.kv_rows_total + row0 + t.key0) * kD;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int blk = n * 4 + wid;  // 16 blocks of 4 rows
        const int lrow = blk * 4 + (lane >> 4);
        const int grow = lrow < t.nkeys ? lrow : t.nkeys - 1;
        const int c = (lane & 15) ^ swz(lrow);
        dma_b128(a.k + base + (int64_t)grow * kD + c * 8, lds_u32(st + blk * 1024));
        dma_b128(a.v + base + (int64_t)grow * kD + c * 8, lds_u32(st + kTileBytes + blk * 1024));
    }
}

// Direct-to-LDS loads of a unit's 64 packed Q rows and their mask words.
__device__ __forceinline__ void issue_q(const AttnArgs& a, int unit, unsigned char* qslot, uint32_t* mslot,
                                        int wid, int lane) {
    const int g = unit / a.RG, rg = unit - g * a.RG;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int blk = n * 4 + wid;
        const int rho = blk * 4 + (lane >> 4);
        int i, hq;
        query_row(a, g, rg * kUnitRows + rho, i, hq);
        const int c = (lane & 15) ^ swz(rho);
        dma_b128(a.q + ((int64_t)i * a.Hq + hq) * kD + c * 8, lds_u32(qslot + blk * 1024));
    }
    if (wid == 0) {
        int i, hq;
        query_row(a, g, rg * kUnitRows + lane, i, hq);
        const uint32_t* mw = (const uint32_t*)(a.mask + i);
        dma_b32(mw, lds_u32(mslot));
        dma_b32(mw + 1, lds_u32(mslot + kWave));
    }
}

__global__ __launch_bounds__(kThreads, 1) void tree_attn_bf16_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStageBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char qslot[kQBytes];
    __shared__ uint32_t mslot[2 * kWave];
    __shared__ float s_ml[2][2][kWave];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
    const int rb = wid & 1, ks = wid >> 1;
    const int l32 = lane & 31, h2 = lane >> 5;
    const int T = a.T;
    const int ctx = a.ctx_len[0];
    const int S = ctx + T;
    const int64_t row0 = a.kv_row_off[0];
    const int units = a.Hkv * a.RG;
    const int64_t total = (int64_t)units * S;
    const int nwg = total < (int64_t)gridDim.x ? (int)total : (int)gridDim.x;
    const int vwg = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    if (vwg >= nwg) return;
    const int64_t x_begin = total * vwg / nwg, x_end = total * (vwg + 1) / nwg;

    // ---- first segment's Q and mask word, straight into registers ----
    const int qrow = 32 * rb + l32;  // this lane's packed query row inside the unit
    bf16x8 qcur[8];
    uint64_t mword;
    {
        const Tile t0 = tile_at(x_begin, x_begin, x_end, S);
        const int g = t0.unit / a.RG, rg = t0.unit - g * a.RG;
        int i, hq;
        query_row(a, g, rg * kUnitRows + qrow, i, hq);
        const __bf16* qp = a.q + ((int64_t)i * a.Hq + hq) * kD;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qcur[kk] = *(const bf16x8*)(qp + 16 * kk + 8 * h2);
        mword = a.mask[i];
        wait_direct_loads();
    }

    // ---- prologue: tiles 0..2 in flight; a later segment's Q goes to the slot ----
    int64_t xl = x_begin;     // list position of the next tile to fetch
    int nl = 0;               // tiles fetched so far
    int q_slot_tile = -1;     // tile whose Q is in (or on its way to) the Q slot
    // A later segment's Q rides with its first tile into the slot when the slot is
    // free; otherwise that tile loads its Q directly when it is computed.
    auto fetch = [&]() {
        const Tile t = tile_at(xl, x_begin, x_end, S);
        issue_kv(a, t, row0, smem + (nl % kStages) * kStageBytes, wid, lane);
        if (t.seg_start && nl > 0 && q_slot_tile < 0) {
            issue_q(a, t.unit, qslot, mslot, wid, lane);
            q_slot_tile = nl;
        }
        xl += t.nkeys;
        ++nl;
    };
    for (int s = 0; s < kStages - 1 && xl < x_end; ++s) fetch();

    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    int seg_key0 = 0;
    const int krow = 32 * ks + key_of_row(l32);
    const int g16 = lane >> 4, i16 = lane & 15, rr = i16 >> 2, cc = i16 & 3, dh = g16 & 1;

    int64_t xc = x_begin;     // list position of the tile being computed
    for (int it = 0; xc < x_end; ++it) {
        // tiles fetched after this one: nl - 1 - it (at most 2)
        const int after = nl - 1 - it;
        if (after >= 2) barrier_vm16(); else if (after == 1) barrier_vm8(); else barrier_vm0();
        if (xl < x_end) fetch();

        const Tile tc = tile_at(xc, x_begin, x_end, S);
        unsigned char* st = smem + (it % kStages) * kStageBytes;
        const unsigned char* sK = st;
        const unsigned char* sV = st + kTileBytes;

        if (tc.seg_start) {
            if (it > 0) {
                if (q_slot_tile == it) {
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk) {
                        const int c = (2 * kk + h2) ^ swz(qrow);
                        qcur[kk] = *(const bf16x8*)(qslot + qrow * kRowBytes + c * 16);
                    }
                    mword = (uint64_t)mslot[qrow] | ((uint64_t)mslot[kWave + qrow] << 32);
                    q_slot_tile = -1;  // free once every wave has passed the next barrier
                } else {
                    const int g = tc.unit / a.RG, rg = tc.unit - g * a.RG;
                    int i, hq;
                    query_row(a, g, rg * kUnitRows + qrow, i, hq);
                    const __bf16* qp = a.q + ((int64_t)i * a.Hq + hq) * kD;
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk) qcur[kk] = *(const bf16x8*)(qp + 16 * kk + 8 * h2);
                    mword = a.mask[i];
                    wait_direct_loads();  // drains the K/V loads too: rare (short segments)
                }
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
                m_run = -INFINITY;
                l_run = 0.0f;
            }
            seg_key0 = tc.key0;
        }

        // ---- S^T = K Q^T: this wave's 32 keys x 32 query rows, two MFMA chains ----
        f32x16 s0, s1;
#pragma unroll
        for (int e = 0; e < 16; ++e) { s0[e] = 0.0f; s1[e] = 0.0f; }
#pragma unroll
        for (int kk = 0; kk < 8; kk += 2) {
            const int c0 = (2 * kk + h2) ^ swz(krow), c1 = (2 * kk + 2 + h2) ^ swz(krow);
            const bf16x8 k0 = *(const bf16x8*)(sK + krow * kRowBytes + c0 * 16);
            const bf16x8 k1 = *(const bf16x8*)(sK + krow * kRowBytes + c1 * 16);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qcur[kk], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qcur[kk + 1], s1, 0, 0, 0);
        }

        // ---- online softmax (base 2): lane = one query row, 16 of its keys ----
        float sv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) sv[e] = (s0[e] + s1[e]) * a.scale_log2;
        if (tc.key0 + kTileKeys > ctx || tc.nkeys < kTileKeys) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = 32 * ks + 16 * (e >> 3) + 8 * h2 + (e & 7);
                const int key = tc.key0 + j;
                bool vis = j < tc.nkeys;
                if (vis && key >= ctx) vis = (mword >> (key - ctx)) & 1ull;
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
        if (__any(alpha != 1.0f && m_run != -INFINITY)) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
        }
        m_run = m_new;

        // ---- O^T += V^T P^T; V^T operands by LDS transpose reads ----
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int vr1 = 32 * ks + 16 * j + 8 * h2 + rr;
            const int vr2 = vr1 + 4;
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const int c = 4 * db + 2 * dh + (cc >> 1);
                const int off = (cc & 1) * 8;
                const unsigned char* p1 = sV + vr1 * kRowBytes + ((c ^ swz(vr1)) << 4) + off;
                const unsigned char* p2 = sV + vr2 * kRowBytes + ((c ^ swz(vr2)) << 4) + off;
                const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_ADDR(i16x4, p1));
                const i16x4 a2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_ADDR(i16x4, p2));
                const i16x8 a8 = {a1[0], a1[1], a1[2], a1[3], a2[0], a2[1], a2[2], a2[3]};
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb[j],
                                                                   oacc[db], 0, 0, 0);
            }
        }

        if (tc.seg_end) {
            // ---- merge the two key halves through this stage's LDS (its tile is
            // consumed; the stage is refilled only after the next stage barrier) ----
            barrier_lds();
            float* mb = (float*)st;
            if (ks == 1) {
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) mb[((rb * 64) + db * 16 + e) * kWave + lane] = oacc[db][e];
                s_ml[rb][0][lane] = m_run;
                s_ml[rb][1][lane] = l_run;
            }
            barrier_lds();
            if (ks == 0) {
                const int g = tc.unit / a.RG, rg = tc.unit - g * a.RG;
                const bool whole = seg_key0 == 0 && tc.key0 + tc.nkeys == S;
                const int rp = rg * kUnitRows + qrow;
                const float m1 = s_ml[rb][0][lane], l1 = s_ml[rb][1][lane];
                const float M = fmaxf(m_run, m1);
                const float Mu = (M == -INFINITY) ? 0.0f : M;
                const float a0 = exp2f(m_run - Mu), a1 = exp2f(m1 - Mu);
                const float lsum = l_run * a0 + l1 * a1;
                const float ltot = lsum + __shfl_xor(lsum, 32, kWave);
                // a row that sees none of this segment's keys has ltot = 0: its partial
                // is all zeros, and its merge weight is zero
                const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        oacc[db][e] = (oacc[db][e] * a0 + mb[((rb * 64) + db * 16 + e) * kWave + lane] * a1) * inv;
                if (rp < a.G * T) {
                    if (whole) {
                        int i, hq;
                        query_row(a, g, rp, i, hq);
                        __bf16* orow = a.o + ((int64_t)i * a.Hq + hq) * kD;
#pragma unroll
                        for (int db = 0; db < 4; ++db)
#pragma unroll
                            for (int qd = 0; qd < 4; ++qd) {
                                bf16x4 w;
#pragma unroll
                                for (int x = 0; x < 4; ++x) w[x] = (__bf16)oacc[db][4 * qd + x];
                                *(bf16x4*)(orow + 32 * db + 8 * qd + 4 * h2) = w;
                            }
                        if (h2 == 0 && a.lse) a.lse[(int64_t)i * a.Hq + hq] = (M + log2f(ltot)) * kLn2;
                    } else {
                        const int64_t slot = (int64_t)tc.unit + vwg;
                        _Float16* po = a.part_o + slot * (kUnitRows * kD) + (int64_t)qrow * kD;
#pragma unroll
                        for (int db = 0; db < 4; ++db)
#pragma unroll
                            for (int qd = 0; qd < 4; ++qd) {
                                f16x4 w;
#pragma unroll
                                for (int x = 0; x < 4; ++x) w[x] = (_Float16)oacc[db][4 * qd + x];
                                *(f16x4*)(po + 32 * db + 8 * qd + 4 * h2) = w;
                            }
                        if (h2 == 0) {
                            a.part_ml[slot * 128 + qrow] = M;
                            a.part_ml[slot * 128 + 64 + qrow] = ltot;
                        }
                    }
                }
            }
        }
        xc += tc.nkeys;
    }
}

// ---------------------------------------------------------------------------
// Merge: one workgroup per (unit, 16 query rows); thread = (row, 8 dims).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(AttnArgs a, int grid_wg) {
    const int tid = threadIdx.x;
    const int unit = blockIdx.x;
    const int g = unit / a.RG, rg = unit - g * a.RG;
    const int S = a.ctx_len[0] + a.T;
    const int64_t total = (int64_t)a.Hkv * a.RG * S;
    const int nwg = total < (int64_t)grid_wg ? (int)total : grid_wg;
    const int64_t U0 = (int64_t)unit * S;
    const int vf = stretch_of(U0, total, nwg), vl = stretch_of(U0 + S - 1, total, nwg);
    if (vf == vl) return;  // written directly by the main kernel
    const int row = blockIdx.y * 16 + (tid >> 4);
    const int d0 = (tid & 15) * 8;
    const int rp = rg * kUnitRows + row;
    if (rp >= a.G * a.T) return;
    float M = -INFINITY;
    for (int v = vf; v <= vl; ++v) M = fmaxf(M, a.part_ml[((int64_t)unit + v) * 128 + row]);
    float L = 0.0f;
    f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
#pragma unroll 4
    for (int v = vf; v <= vl; ++v) {
        const int64_t slot = (int64_t)unit + v;
        const float w = exp2f(a.part_ml[slot * 128 + row] - M) * a.part_ml[slot * 128 + 64 + row];
        L += w;
        const f16x8 o8 = *(const f16x8*)(a.part_o + slot * (kUnitRows * kD) + (int64_t)row * kD + d0);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            acc0[x] += (float)o8[x] * w;
            acc1[x] += (float)o8[4 + x] * w;
        }
    }
    int i, hq;
    query_row(a, g, rp, i, hq);
    const float inv = 1.0f / L;
    bf16x8 out;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        out[x] = (__bf16)(acc0[x] * inv);
        out[4 + x] = (__bf16)(acc1[x] * inv);
    }
    *(bf16x8*)(a.o + ((int64_t)i * a.Hq + hq) * kD + d0) = out;
    if (d0 == 0 && a.lse) a.lse[(int64_t)i * a.Hq + hq] = (M + log2f(L)) * kLn2;
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
    size_t part_o, part_ml, total;
};

// Partial slots for one sequence (reused, in stream order, by the next one).
WsLayout ws_layout(const eagle_attn_desc& d) {
    WsLayout w{0, 0, 0};
    if (d.dtype != EAGLE_BF16) return w;
    const int G = d.n_q_heads / d.n_kv_heads;
    const int RG = (G * d.T + kUnitRows - 1) / kUnitRows;
    const size_t slots = (size_t)d.n_kv_heads * RG + kGridWG;
    w.part_o = 0;
    w.part_ml = align_up(slots * kUnitRows * kD * sizeof(_Float16));
    w.total = w.part_ml + align_up(slots * 2 * kUnitRows * sizeof(float));
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
    const int RG = (G * d.T + kUnitRows - 1) / kUnitRows;
    const size_t seq_q = (size_t)d.T * d.n_q_heads * kD;
    // One sequence per launch pair: the kernels never walk across sequences.
    for (int b = 0; b < d.batch; ++b) {
        AttnArgs a;
        a.q = (const __bf16*)q + b * seq_q;
        a.k = (const __bf16*)k;
        a.v = (const __bf16*)v;
        a.mask = mask + (size_t)b * d.T;
        a.o = (__bf16*)o + b * seq_q;
        a.lse = lse ? lse + (size_t)b * d.T * d.n_q_heads : nullptr;
        a.ctx_len = d.ctx_len + b;
        a.kv_row_off = d.kv_row_off + b;
        a.part_o = (_Float16*)(ws + w.part_o);
        a.part_ml = (float*)(ws + w.part_ml);
        a.kv_rows_total = d.kv_rows_total;
        a.T = d.T; a.Hq = d.n_q_heads; a.Hkv = d.n_kv_heads; a.G = G; a.RG = RG;
        a.scale_log2 = scale * kLog2e;
        tree_attn_bf16_kernel<<<kGridWG, kThreads, 0, stream>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        tree_attn_merge_kernel<<<dim3(d.n_kv_heads * RG, kUnitRows / 16), 256, 0, stream>>>(a, kGridWG);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int attention_max_batch() { return 1024; }

}  // namespace eagle
