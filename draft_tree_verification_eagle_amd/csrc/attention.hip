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
//    head are its G = Hq/Hkv query heads x T tree rows.  The 64-key tiles of all
//    units (ctx + T keys each) form one list, split over 256 workgroups, one per
//    CU, on tile boundaries and weighted so that a workgroup spanning two units
//    (two segments to merge and write) takes fewer tiles.  Workgroup index ->
//    list position is XCD-aware (blockIdx % 8 picks the XCD): each XCD takes one
//    contiguous run of stretches, so the units that share K/V rows (GQA) read
//    them through one L2, and the partials of a unit land mostly in one L2.
//  * Eight waves per workgroup: four compute, four only load.  K and V stream HBM ->
//    LDS by direct 16-byte global_load_lds (no register staging), four stages
//    deep, issued and waited for by the loader waves alone (each issues a quarter
//    of every tile's 1 KB row blocks, K before V).  A wave that issues a burst of such loads
//    stalls until the memory pipeline takes them, and one wave alone cannot keep
//    enough of them in flight, so the computing waves never issue one and four
//    loaders share the stream.  Every wave runs the same tile walk and meets the
//    same barriers.  Lanes for rows past a short tile re-read the tile's last
//    row, which the softmax masks out and which costs no extra HBM traffic.  LDS
//    rows use a 16-byte chunk XOR swizzle that keeps the MFMA operand reads
//    conflict-free.
//  * Q stays in registers for a whole segment; each segment's Q rides into an
//    LDS slot ahead of its first tile (or, when the slot is still busy, is loaded
//    directly when that tile's scores are computed).
//  * The 4 computing waves = 2 query halves x 2 key halves of a tile.  S^T = K Q^T
//    and O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16; V^T operands come
//    straight from the row-major V tile through ds_read_b64_tr_b16.  The key
//    order inside the S^T block is permuted so each half-wave's probabilities are
//    the PV operand's 8 consecutive keys, with no register shuffles.  Online
//    softmax in fp32 (base 2) with a lazy reference max: O is rescaled only when
//    a row's max grows by more than 2^8, so the common tile does no rescale;
//    probabilities are rounded to bf16 for PV.  The MFMA accumulators live in
//    VGPRs (the library is built with the VGPR form of MFMA), so the softmax and
//    rescale read them without accumulator-register copies.
//  * A workgroup whose stretch holds a whole unit writes the output; otherwise
//    it writes a partial: row max and row sum in fp32 and the normalised row in
//    fp16 (relative rounding 2^-11, inside the bf16 output's own).  The merge
//    kernel, on the same stream, combines the partials of split units, so no
//    workgroup ever waits for another; each unit is merged on the XCD whose
//    stretches hold the middle of it, where most of its partials are still in
//    L2 (written back, not dropped, when the main kernel ends).
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
constexpr int kComputeWaves = 4;                     // 2 query halves x 2 key halves
#ifndef EAGLE_LOADERS
#define EAGLE_LOADERS 4
#endif
constexpr int kLoaders = EAGLE_LOADERS;              // waves that issue the loads
constexpr int kThreads = (kComputeWaves + kLoaders) * 64;
constexpr int kStages = 4;
constexpr int kGridWG = 256;                         // one per CU, multiple of the 8 XCDs
static_assert(kGridWG % 8 == 0, "workgroups are dealt to the 8 XCDs in turn");

// Workgroup b of a launch runs on XCD b % 8 (the dispatcher deals workgroups to
// the XCDs in turn).  Of n stretches, XCD x takes [xcd_first(x, n),
// xcd_first(x + 1, n)): one contiguous run each, sizes differing by at most one.
__host__ __device__ inline int xcd_first(int x, int n) { return (x * n + 7) >> 3; }
// Unit u's middle lies at fraction (u + 1/2) / units of the cost line, which
// XCD floor((8u + 4) / units) holds; XCD x merges units [merge_unit_first(x),
// merge_unit_first(x + 1)), at most ceil(units / 8) of them.
__host__ __device__ inline int merge_unit_first(int x, int units) {
    const int t = x * units - 4;
    return t <= 0 ? 0 : (t + 7) >> 3;
}
constexpr int kRowBytes = kD * 2;                    // 256
constexpr int kTileBytes = kTileKeys * kRowBytes;    // 16 KB
constexpr int kStageBytes = 2 * kTileBytes;          // K tile | V tile
constexpr int kQBytes = kUnitRows * kRowBytes;       // 16 KB
constexpr int kTileLoads = 2 * kTileBytes / (64 * 16) / kLoaders;  // per loader lane per tile (K and V)
constexpr int kQLoads = kQBytes / (64 * 16) / kLoaders + 2;         // per loader lane (+ mask words)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;  // log2 of the largest unnormalised probability

static_assert(kStages == 4 && 16 % kLoaders == 0, "4 stages; the loaders split the 16 blocks of a tile evenly");

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
// 16 bytes per lane from base + off (scalar base, 32-bit lane offset) to LDS
// address lds + 16 * lane.
// The base is the same in every lane; readfirstlane makes that visible to the
// compiler so the operand is always an SGPR pair.
__device__ __forceinline__ void dma_b128(const void* base, uint32_t off, uint32_t lds_addr) {
    // readfirstlane returns int: widen through uint32_t (a sign extension of the
    // low word would corrupt the high word of the address)
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t bu = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(off), "s"((const void*)(uintptr_t)bu)
                 : "memory", "m0");
}
// Same, non-temporal: K and V are streamed once.
__device__ __forceinline__ void dma_b128_nt(const void* base, uint32_t off, uint32_t lds_addr) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t bu = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(off), "s"((const void*)(uintptr_t)bu)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const void* gptr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gptr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop
// Loader wave: wait until at most `tiles_after` tiles' loads (0 or 1) are still
// in flight; loads complete in issue order, so everything issued before them has
// landed.
template <int N>
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void loader_wait(int tiles_after) {
    if (tiles_after >= 1) vm_wait<kTileLoads>();
    else vm_wait<0>();
}

// s_waitcnt vmcnt(0) as the compiler sees it: after this, registers filled by
// ordinary loads count as complete, so no wait for them is carried into the
// tile loop (where any vmcnt wait would also drain the K/V pipeline).
__device__ __forceinline__ void wait_direct_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// A lane value the compiler must treat as unknown here: addresses derived from it
// in the rarely taken paths (segment starts and ends) are recomputed there instead
// of being hoisted out of the tile loop, where they would only hold registers.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

// max / sum of a value over the lane pair (l, l ^ 32)
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One sequence.  Pointers are already offset to the sequence.
struct AttnArgs {
    const __bf16* q;           // [T][Hq][D]
    const __bf16* k;           // cache base; the sequence's rows start at *kv_row_off
    const __bf16* v;
    const uint64_t* mask;      // [T]
    __bf16* o;                 // [T][Hq][D]
    float* lse;                // [T][Hq] or null
    const int32_t* ctx_len;    // [1], read when ctx_h < 0
    const int64_t* kv_row_off; // [1], read when ctx_h < 0
    _Float16* part_o;          // [slots][64][128], normalised rows
    float* part_ml;            // [slots][2][64]: row reference max (base 2), row sum
    int64_t kv_rows_total;
    int T, Hq, Hkv, G, RG;
    float scale_log2;
    int ctx_h;                 // the sequence's context length from the host, or -1
    int64_t row0_h;            // its first cache row from the host (when ctx_h >= 0)
};

// Work split.  Each unit's keys form nt = ceil(S / 64) tiles; the tiles are laid
// on a cost line, unit after unit, each tile 4 cost steps long and each unit
// preceded by kSegCost4 steps that stand for the fixed work of a segment (its
// key-half merge and its output).  The line is cut into nwg equal stretches and a
// workgroup takes the tiles that start in its stretch, so stretches end on tile
// boundaries and a workgroup that spans two units takes fewer tiles.  Every
// stretch is at least one tile long, so one that lies inside a unit's tiles holds
// a tile start; one that falls wholly in the steps before a unit's first tile is
// empty (its workgroup exits).  The workgroups holding a unit's tiles are
// consecutive, none of them empty.
constexpr int kSegCost4 = 16;
// All in 32-bit steps: the host checks that the cost line fits in 31 bits.
struct Split {
    uint32_t W;      // cost steps per unit
    uint32_t Wt;     // cost steps in all
    uint32_t q, r;   // Wt = q * nwg + r
    int nt;          // tiles per unit
    int nwg;         // workgroups that take part
};
__host__ __device__ inline Split make_split(int S, int units, int grid) {
    Split sp;
    sp.nt = (S + kTileKeys - 1) / kTileKeys;
    sp.W = 4u * (uint32_t)sp.nt + kSegCost4;
    sp.Wt = (uint32_t)units * sp.W;
    const uint32_t most = sp.Wt / 4;
    sp.nwg = most < (uint32_t)grid ? (most > 0 ? (int)most : 1) : grid;
    sp.q = sp.Wt / (uint32_t)sp.nwg;
    sp.r = sp.Wt - sp.q * (uint32_t)sp.nwg;
    return sp;
}
// First cost step of stretch v: floor(Wt * v / nwg).
__host__ __device__ inline uint32_t stretch_start(const Split& sp, int v) {
    return sp.q * (uint32_t)v + (sp.r * (uint32_t)v) / (uint32_t)sp.nwg;
}
// First tile (unit, tile) starting at or after cost step p; (units, 0) past the last.
struct TilePos {
    int unit, tile;
};
__device__ __forceinline__ TilePos split_tile(const Split& sp, uint32_t p) {
    TilePos tp;
    tp.unit = (int)(p / sp.W);
    const uint32_t r = p - (uint32_t)tp.unit * sp.W;
    tp.tile = r <= kSegCost4 ? 0 : (int)((r - kSegCost4 + 3) / 4);
    if (tp.tile >= sp.nt) {
        ++tp.unit;
        tp.tile = 0;
    }
    return tp;
}
// Workgroup (in list order) whose stretch holds cost step p.
__host__ __device__ inline int stretch_of(const Split& sp, uint32_t p) {
    int v = (int)((double)p * (double)sp.nwg / (double)sp.Wt);
    if (v > sp.nwg - 1) v = sp.nwg - 1;
    while (v + 1 < sp.nwg && stretch_start(sp, v + 1) <= p) ++v;
    while (v > 0 && stretch_start(sp, v) > p) --v;
    return v;
}

// Position in a workgroup's stretch: keys walked since the stretch start (a
// stretch is far below 2^31 keys), unit and key inside the unit.  Advanced tile by
// tile without division; all bookkeeping is 32-bit scalar work.
struct Walker {
    int x;
    int unit, key0;
};
struct Tile {
    int unit, key0, nkeys;
    bool seg_start, seg_end;
};
// `len` = keys in the stretch.
__device__ __forceinline__ Tile peek(const Walker& w, int len, int S) {
    Tile t;
    t.unit = w.unit;
    t.key0 = w.key0;
    int n = kTileKeys;
    if (S - w.key0 < n) n = S - w.key0;
    if (len - w.x < n) n = len - w.x;
    t.nkeys = n;
    t.seg_start = (w.x == 0) || (w.key0 == 0);
    t.seg_end = (w.x + n == len) || (w.key0 + n == S);
    return t;
}
__device__ __forceinline__ void advance(Walker& w, int nkeys, int S) {
    w.x += nkeys;
    w.key0 += nkeys;
    if (w.key0 == S) {
        w.key0 = 0;
        ++w.unit;
    }
}

// Packed query row -> (tree row, query head); rows past G*T map to row 0.
__device__ __forceinline__ void query_row(const AttnArgs& a, int g, int rp, int& i, int& hq) {
    if (rp >= a.G * a.T) rp = 0;
    const int gi = rp / a.T;
    i = rp - gi * a.T;
    hq = g * a.G + gi;
}

// Direct-to-LDS loads of one tile's K and V rows, all issued by the loader wave:
// 16 blocks of 4 rows each for K and for V, 32 loads per lane.  In a full tile,
// block b starts 1 KB * b in and off4[b & 3] is the lane's offset inside it; for a
// short tile, rows past
// nkeys re-read row nkeys - 1 (masked out by the softmax, no extra HBM traffic).
__device__ __forceinline__ void load_tile(const AttnArgs& a, const Tile& t, int64_t row0, unsigned char* st,
                                          const uint32_t (&off4)[4], int li, int lane) {
    // keep the wave's outstanding-load count within the 63 its counter holds
    vm_wait<63 - kTileLoads>();
    const int g = t.unit / a.RG;
    const int64_t elt0 = ((int64_t)g * a.kv_rows_total + row0 + t.key0) * kD;
    const __bf16* kb = a.k + elt0;
    const __bf16* vb = a.v + elt0;
    if (t.nkeys == kTileKeys) {
        // K first, then V: the first tile's scores can start before its V lands.
        // The block's 1 KB step goes into the scalar base, the lane part stays in 4 VGPRs.
#pragma unroll
        for (int bi = 0; bi < 16 / kLoaders; ++bi) {
            const int blk = bi * kLoaders + li;
            dma_b128_nt(kb + blk * 512, off4[blk & 3], lds_u32(st + blk * 1024));
        }
#pragma unroll
        for (int bi = 0; bi < 16 / kLoaders; ++bi) {
            const int blk = bi * kLoaders + li;
            dma_b128_nt(vb + blk * 512, off4[blk & 3], lds_u32(st + kTileBytes + blk * 1024));
        }
    } else {
        uint32_t off[16 / kLoaders];
#pragma unroll
        for (int bi = 0; bi < 16 / kLoaders; ++bi) {
            const int lrow = (bi * kLoaders + li) * 4 + (lane >> 4);
            const int grow = lrow < t.nkeys ? lrow : t.nkeys - 1;
            off[bi] = (uint32_t)(grow * kRowBytes + (((lane & 15) ^ swz(lrow)) << 4));
        }
#pragma unroll
        for (int bi = 0; bi < 16 / kLoaders; ++bi)
            dma_b128_nt(kb, off[bi], lds_u32(st + (bi * kLoaders + li) * 1024));
#pragma unroll
        for (int bi = 0; bi < 16 / kLoaders; ++bi)
            dma_b128_nt(vb, off[bi], lds_u32(st + kTileBytes + (bi * kLoaders + li) * 1024));
    }
}

// Direct-to-LDS loads of a unit's 64 packed Q rows and their mask words, by the
// loader wave: 16 + 2 loads per lane.
__device__ __forceinline__ void load_q(const AttnArgs& a, int unit, unsigned char* qslot, uint32_t* mslot,
                                       int li, int lane) {
    vm_wait<63 - kQLoads>();  // at most 63 loads in flight
    const int g = unit / a.RG, rg = unit - g * a.RG;
#pragma unroll
    for (int bi = 0; bi < 16 / kLoaders; ++bi) {
        const int blk = bi * kLoaders + li;
        const int rho = blk * 4 + (lane >> 4);
        int i, hq;
        query_row(a, g, rg * kUnitRows + rho, i, hq);
        const uint32_t off = (uint32_t)((((int64_t)i * a.Hq + hq) * kD) * 2 + (((lane & 15) ^ swz(rho)) << 4));
        dma_b128(a.q, off, lds_u32(qslot + blk * 1024));
    }
    if (li == 0) {
        int i, hq;
        query_row(a, g, rg * kUnitRows + lane, i, hq);
        const uint32_t* mw = (const uint32_t*)(a.mask + i);
        dma_b32(mw, lds_u32(mslot));
        dma_b32(mw + 1, lds_u32(mslot + kWave));
    }
}

// The tile walk of one workgroup, for the loader wave (kLoader) or a computing
// wave.  Both instantiations share every branch that reaches a barrier, so the
// five waves always meet the same barriers in the same order.
template <bool kLoader>
__device__ __forceinline__ void tile_loop(const AttnArgs& a, unsigned char* smem, unsigned char* qslot,
                                          uint32_t* mslot, float (*s_ml)[2][2][kWave], int wid, int lane,
                                          int T, int ctx, int S, int64_t row0, int vwg, int len,
                                          TilePos tb) {
    constexpr bool loader = kLoader;
    const int rb = wid & 1, ks = (wid >> 1) & 1;
    const int l32 = lane & 31, h2 = lane >> 5;
    // lane offset inside a full tile's block b (rows 4b .. 4b + 3), without the
    // block's own 1 KB * b: the lane's row in the block and its swizzled chunk,
    // which depends on b only through b & 3
    uint32_t off4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        off4[j] = (uint32_t)((lane >> 4) * kRowBytes + (((lane & 15) ^ swz(j * 4 + (lane >> 4))) << 4));

    Walker w0;
    w0.x = 0;
    w0.unit = tb.unit;
    w0.key0 = tb.tile * kTileKeys;

    // ---- first segment's Q and mask word, straight into registers ----
    const int qrow = 32 * rb + l32;  // this lane's packed query row inside the unit
    bf16x8 qcur[8];
    uint64_t mword_n;
    auto load_q_direct = [&](int unit) {
        const int g = unit / a.RG, rg = unit - g * a.RG;
        int i, hq;
        query_row(a, g, rg * kUnitRows + qrow, i, hq);
        const __bf16* qp = a.q + ((int64_t)i * a.Hq + hq) * kD;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qcur[kk] = *(const bf16x8*)(qp + 16 * kk + 8 * h2);
        mword_n = a.mask[i];
        wait_direct_loads();
    };

    // this lane's Q row and mask word from the Q slot
    auto read_q_slot = [&]() {
        const int qr = opaque(qrow), hh = opaque(h2);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int c = (2 * kk + hh) ^ swz(qr);
            qcur[kk] = *(const bf16x8*)(qslot + qr * kRowBytes + c * 16);
        }
        mword_n = (uint64_t)mslot[qr] | ((uint64_t)mslot[kWave + qr] << 32);
    };

    // ---- prologue.  Every wave runs the same tile bookkeeping and barriers; only
    // the loader issues and waits for loads. ----
    Walker wf = w0;           // next tile to fetch
    int nl = 0;               // tiles fetched so far
    int q_slot_tile = -1;     // tile whose Q is in (or on its way to) the Q slot
    // The computing waves load the first segment's Q straight into registers: they
    // have nothing else in flight, and it lands while tile 0's K streams in.  That
    // keeps the slot free from the start for the next segment's Q, which rides with
    // that segment's first tile (a third segment starting while the slot is still
    // busy loads its Q directly when its scores are computed).
    if (!loader) load_q_direct(w0.unit);
    auto fetch = [&]() {
        const Tile t = peek(wf, len, S);
        if (loader) load_tile(a, t, row0, smem + (nl % kStages) * kStageBytes, off4, wid - kComputeWaves, lane);
        if (t.seg_start && nl > 0 && q_slot_tile < 0) {
            if (loader) load_q(a, t.unit, qslot, mslot, wid - kComputeWaves, lane);
            q_slot_tile = nl;
        }
        advance(wf, t.nkeys, S);
        ++nl;
    };
    fetch();
    if (wf.x < len) fetch();
    // tile 0's K; its V and tile 1 (with any Q that rode with it) may still be in
    // flight, since the first iteration's barrier waits for them.  A one-tile
    // stretch has no such barrier: there everything must land here.
    if (loader) {
        if (nl > 1) vm_wait<kTileLoads / 2 + kTileLoads>();
        else vm_wait<0>();
    }
    barrier_lds();
    if (wf.x < len) fetch();        // tile 2: its stage has not been used yet

    const int krow = 32 * ks + key_of_row(l32);
    const int g16 = lane >> 4, i16 = lane & 15, rr = i16 >> 2, cc = i16 & 3, dh = g16 & 1;

    // S^T = K Q^T for this wave's 32 keys x 32 query rows of the tile in stage st
    auto scores = [&](const unsigned char* st) {
        f32x16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int c = (2 * kk + h2) ^ swz(krow);
            const bf16x8 kv = *(const bf16x8*)(st + krow * kRowBytes + c * 16);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qcur[kk], acc, 0, 0, 0);
        }
        return acc;
    };

    // ---- tile 0: scores ----
    Walker wn = w0;           // tile whose scores are computed next
    Tile tc = peek(wn, len, S);
    advance(wn, tc.nkeys, S);
    f32x16 sacc;
    if (!loader) sacc = scores(smem);
    uint64_t mword_c = mword_n;
    bool from0_c = tc.key0 == 0;  // the current segment starts at the unit's first key

    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    // Software pipeline: iteration it computes the scores of tile it+1 (MFMA)
    // next to the softmax of tile it (VALU), then PV of tile it.
    for (int it = 0;; ++it) {
        const bool has_next = wn.x < len;
        Tile tn;
        bool from0_n = from0_c;
        if (has_next) {
            // tile it+1 has landed; tile it-1's stage is free
            if (loader) loader_wait(nl - it - 2);
            barrier_lds();
            if (wf.x < len) fetch();
            tn = peek(wn, len, S);
            if (tn.seg_start) {
                if (q_slot_tile == it + 1) {
                    if (!loader) {
                        read_q_slot();
                    }
                    q_slot_tile = -1;  // free once every wave has passed the next barrier
                } else if (!loader) {
                    load_q_direct(tn.unit);  // rare (short segments)
                }
                from0_n = tn.key0 == 0;
            }
        }

        f32x16 snext;
        if (!loader) {
        const unsigned char* sV = smem + (it % kStages) * kStageBytes + kTileBytes;

        // ---- online softmax (base 2): lane = one query row, 16 of its keys ----
        // Raw scores; the scale (> 0) is applied inside the exponent.
        if (tc.key0 + kTileKeys > ctx || tc.nkeys < kTileKeys) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = 32 * ks + 16 * (e >> 3) + 8 * h2 + (e & 7);
                const int key = tc.key0 + j;
                bool vis = j < tc.nkeys;
                if (vis && key >= ctx) vis = (mword_c >> (key - ctx)) & 1ull;
                if (!vis) sacc[e] = -INFINITY;
            }
        }
        float mx = fmaxf(sacc[0], sacc[1]);
#pragma unroll
        for (int e = 2; e < 16; ++e) mx = fmaxf(mx, sacc[e]);
        mx = pair_max(mx) * a.scale_log2;
        // Lazy rescaling: the running reference max moves only when a row's max
        // exceeds it by more than kLazy (so probabilities stay <= 2^kLazy).  Any
        // reference gives the same softmax; this keeps the O rescale off the
        // common path.
        if (__any(mx > m_run + kLazy)) {
            const bool bump = mx > m_run + kLazy;
            // exp2(-inf) = 0 when the row had no visible key yet (O and l are 0)
            const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
            if (bump) m_run = mx;
        }
        const float nm = (m_run == -INFINITY) ? 0.0f : -m_run;

        // ---- one branch-free block: the scores of tile it+1 on the matrix cores
        // interleaved with this tile's exponentials on the VALU.  After the last
        // tile the scores are computed from a stale stage and discarded. ----
        // V^T operands of this tile's PV, read first so their latency overlaps
        bf16x8 vop[2][4];
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
                vop[j][db] = __builtin_bit_cast(bf16x8, a8);
            }
        }
        const unsigned char* sKn = smem + ((it + 1) % kStages) * kStageBytes;
#pragma unroll
        for (int e = 0; e < 16; ++e) snext[e] = 0.0f;
        float psum = 0.0f;
        bf16x8 pb[2];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int c = (2 * kk + h2) ^ swz(krow);
            const bf16x8 kv = *(const bf16x8*)(sKn + krow * kRowBytes + c * 16);
            snext = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qcur[kk], snext, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int e = 2 * kk + u;
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], a.scale_log2, nm));
                psum += p;
                pb[e >> 3][e & 7] = (__bf16)p;
            }
        }
        l_run += psum;

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int db = 0; db < 4; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[j][db], pb[j], oacc[db], 0, 0, 0);
        }  // computing waves

        if (tc.seg_end) {
            // ---- close the segment.  Each key half normalises its rows by its own
            // row sum and hands the other half the 64 columns that half finishes
            // (fp16, relative rounding 2^-11) through this stage's K area, dead
            // since the scores of this tile.  Each wave then combines 32 rows x 64
            // columns, stages them row-major in this stage's V area, and all four
            // waves store whole 256-byte rows.  The stage is refilled only after
            // the next stage barrier. ----
            // Without a next tile no stage barrier has passed since the scores of
            // this tile were read from K: wait for every wave before overwriting it.
            if (!has_next) barrier_lds();
            unsigned char* const stg = smem + (it % kStages) * kStageBytes;
            f16x4* const xch = reinterpret_cast<f16x4*>(stg);  // [2 sender ks][2 rb][2 db&1][4 qd][64 lanes]
            unsigned char* const obuf = stg + kTileBytes;       // [64 rows][16 chunks of 16 B], swizzled
            const float lw = pair_sum(l_run);  // this wave's row sum over its keys
            if (!loader) {
                const float inv = lw > 0.0f ? 1.0f / lw : 0.0f;
                auto send = [&](const f32x16& acc, int jj) {
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        f16x4 w;
#pragma unroll
                        for (int x = 0; x < 4; ++x) w[x] = (_Float16)(acc[4 * qd + x] * inv);
                        xch[(((ks * 2 + rb) * 2 + jj) * 4 + qd) * kWave + lane] = w;
                    }
                };
                if (ks == 0) {  // the other half finishes columns 64..127
                    send(oacc[2], 0);
                    send(oacc[3], 1);
                } else {        // the other half finishes columns 0..63
                    send(oacc[0], 0);
                    send(oacc[1], 1);
                }
                s_ml[ks][rb][0][lane] = m_run;
                s_ml[ks][rb][1][lane] = lw;
            }
            barrier_lds();
            const int g = tc.unit / a.RG, rg = tc.unit - g * a.RG;
            const bool whole = from0_c && tc.key0 + tc.nkeys == S;
            if (!loader) {
                const float m1 = s_ml[ks ^ 1][rb][0][lane], l1 = s_ml[ks ^ 1][rb][1][lane];
                const float M = fmaxf(m_run, m1);
                const float Mu = (M == -INFINITY) ? 0.0f : M;
                const float a0 = __builtin_amdgcn_exp2f(m_run - Mu);
                const float w1 = __builtin_amdgcn_exp2f(m1 - Mu) * l1;
                const float ltot = lw * a0 + w1;
                // a row that sees none of this segment's keys has ltot = 0: its partial
                // is all zeros, and its merge weight is zero
                const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
                const int row = opaque(32 * rb + l32);
                // the other half's values for this wave's 64 columns, all read before
                // any staging write (the two areas share a stage)
                f16x4 o1[2][4];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd)
                        o1[jj][qd] = xch[((((ks ^ 1) * 2 + rb) * 2 + jj) * 4 + qd) * kWave + lane];
                // combine this wave's columns (block db) and stage them as 2-byte values:
                // bf16 for the output, fp16 for a partial
                auto finish = [&](const f32x16& acc, int db, auto tag) {
                    using V4 = decltype(tag);
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        V4 w;
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            w[x] = (acc[4 * qd + x] * a0 + (float)o1[db & 1][qd][x] * w1) * inv;
                        const int c = (4 * db + qd) ^ (row & 15);
                        *reinterpret_cast<V4*>(obuf + row * kRowBytes + c * 16 + h2 * 8) = w;
                    }
                };
                if (whole) {
                    if (ks == 0) {
                        finish(oacc[0], 0, bf16x4{});
                        finish(oacc[1], 1, bf16x4{});
                    } else {
                        finish(oacc[2], 2, bf16x4{});
                        finish(oacc[3], 3, bf16x4{});
                    }
                } else {
                    if (ks == 0) {
                        finish(oacc[0], 0, f16x4{});
                        finish(oacc[1], 1, f16x4{});
                    } else {
                        finish(oacc[2], 2, f16x4{});
                        finish(oacc[3], 3, f16x4{});
                    }
                }
                const int rp = rg * kUnitRows + qrow;
                if (ks == 0 && h2 == 0 && rp < a.G * T) {
                    if (whole) {
                        if (a.lse) {
                            int i, hq;
                            query_row(a, g, rp, i, hq);
                            a.lse[(int64_t)i * a.Hq + hq] = (M + log2f(ltot)) * kLn2;
                        }
                    } else {
                        const int64_t slot = (int64_t)tc.unit + vwg;
                        a.part_ml[slot * 128 + qrow] = M;
                        a.part_ml[slot * 128 + 64 + qrow] = ltot;
                    }
                }
            }
            barrier_lds();
            // ---- whole rows out: computing wave wid stores rows 16 wid .. 16 wid + 15 ----
            if (!loader) {
                const int ln = opaque(lane);
                u32x4 val[4];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int row = 16 * wid + 4 * r4 + (ln >> 4);
                    val[r4] = *reinterpret_cast<const u32x4*>(obuf + row * kRowBytes + (((ln & 15) ^ (row & 15)) << 4));
                }
                if (whole) {
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int rp = rg * kUnitRows + 16 * wid + 4 * r4 + (ln >> 4);
                        if (rp < a.G * T) {
                            int i, hq;
                            query_row(a, g, rp, i, hq);
                            *reinterpret_cast<u32x4*>(a.o + ((int64_t)i * a.Hq + hq) * kD + 8 * (ln & 15)) = val[r4];
                        }
                    }
                } else {
                    _Float16* const po = a.part_o + ((int64_t)tc.unit + vwg) * (kUnitRows * kD);
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int row = 16 * wid + 4 * r4 + (ln >> 4);
                        if (rg * kUnitRows + row < a.G * T)
                            *reinterpret_cast<u32x4*>(po + row * kD + 8 * (ln & 15)) = val[r4];
                    }
                }
            }
            // the next segment starts from an empty state
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
            m_run = -INFINITY;
            l_run = 0.0f;
        }
        if (!has_next) break;
        sacc = snext;
        tc = tn;
        advance(wn, tn.nkeys, S);
        mword_c = mword_n;
        from0_c = from0_n;
    }
}

// kHostLen: the sequence's context length and first row come as launch arguments
// (a separate instantiation, so every argument load issues at once).
template <bool kHostLen>
__global__ __launch_bounds__(kThreads, 1) void tree_attn_bf16_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStageBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char qslot[kQBytes];
    __shared__ uint32_t mslot[2 * kWave];
    __shared__ float s_ml[2][2][2][kWave];  // [key half][query half][max, sum][lane]

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int T = a.T;
    const int ctx = kHostLen ? a.ctx_h : a.ctx_len[0];
    const int S = ctx + T;
    const int64_t row0 = kHostLen ? a.row0_h : a.kv_row_off[0];
    const int units = a.Hkv * a.RG;
    const Split sp = make_split(S, units, (int)gridDim.x);
    const int xcd = blockIdx.x & 7;
    const int vwg = xcd_first(xcd, sp.nwg) + (blockIdx.x >> 3);
    if (vwg >= xcd_first(xcd + 1, sp.nwg)) return;  // nwg <= gridDim.x: every stretch has a workgroup
    const TilePos tb = split_tile(sp, stretch_start(sp, vwg));
    const TilePos te = split_tile(sp, stretch_start(sp, vwg + 1));
    const int64_t x_begin = (int64_t)tb.unit * S + tb.tile * kTileKeys;
    const int64_t x_end = (int64_t)te.unit * S + te.tile * kTileKeys;
    if (x_begin >= x_end) return;  // a stretch in the steps before a unit's first tile
    const int len = (int)(x_end - x_begin);

    // waves 0..3 compute (query half, key half); wave 4 issues every K, V and Q
    // load and waits for them, so no computing wave stalls on a load issue.  Both
    // roles run the same tile walk and the same barriers.
    if (wid >= kComputeWaves)
        tile_loop<true>(a, smem, qslot, mslot, s_ml, wid, lane, T, ctx, S, row0, vwg, len, tb);
    else
        tile_loop<false>(a, smem, qslot, mslot, s_ml, wid, lane, T, ctx, S, row0, vwg, len, tb);

}

// ---------------------------------------------------------------------------
// Merge: one workgroup per (unit, 16 query rows); thread = (row, 8 dims).
// Partials are combined kMergeBatch at a time, their loads issued together.
// Workgroup b: XCD x = b % 8, then the (b / 8)-th (unit, row block) of the units
// XCD x merges; the grid holds 8 * ceil(units / 8) * kRowBlocks workgroups.
// ---------------------------------------------------------------------------
constexpr int kMergeBatch = 8;
constexpr int kRowBlocks = kUnitRows / 16;

// Per merge workgroup, its unit and that unit's first and last stretch (where its
// partials are), computed on the host when the context length is known there: the
// word is read by workgroup index alone, together with the other launch arguments,
// so the kernel starts its loads without the split arithmetic (about 0.9 us at its
// start).  Entry: bit 31 set = unit in use, bits 16..23 unit, 8..15 first stretch,
// 0..7 last stretch.  Up to kPlanWgs merge workgroups (64 units).
constexpr int kPlanWgs = 256;
struct MergePlan {
    int n_wg;                       // workgroups covered (0: computed in the kernel)
    uint32_t e[kPlanWgs];
};
static_assert(kGridWG <= 256, "stretch indices fit 8 bits");

template <bool kHostLen>
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(AttnArgs a, int grid_wg, MergePlan plan) {
    const int tid = threadIdx.x;
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    int unit, vf, vl;
    if (kHostLen && plan.n_wg > 0) {
        const uint32_t e = plan.e[blockIdx.x];
        if (!(e >> 31)) return;
        unit = (int)((e >> 16) & 0xFFu);
        vf = (int)((e >> 8) & 0xFFu);
        vl = (int)(e & 0xFFu);
    } else {
        const int units = a.Hkv * a.RG;
        unit = merge_unit_first(xcd, units) + j / kRowBlocks;
        if (unit >= merge_unit_first(xcd + 1, units)) return;
        const int S = (kHostLen ? a.ctx_h : a.ctx_len[0]) + a.T;
        const Split sp = make_split(S, units, grid_wg);
        const uint32_t p0 = (uint32_t)unit * sp.W + kSegCost4;  // cost step of the unit's first tile
        vf = stretch_of(sp, p0);
        vl = stretch_of(sp, p0 + 4u * (uint32_t)(sp.nt - 1));
    }
    if (vf == vl) return;  // written directly by the main kernel
    const int g = unit / a.RG, rg = unit - g * a.RG;
    const int row = (j % kRowBlocks) * 16 + (tid >> 4);
    const int d0 = (tid & 15) * 8;
    const int rp = rg * kUnitRows + row;
    if (rp >= a.G * a.T) return;
    float M = -INFINITY, L = 0.0f;
    float acc[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] = 0.0f;
    // up to kMergeBatch partials per round, all requested together: slots past the
    // last re-read the last one (same addresses) and get zero weight
    for (int v0 = vf; v0 <= vl; v0 += kMergeBatch) {
        float mv[kMergeBatch], lv[kMergeBatch];
        f16x8 ov[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            const int64_t slot = (int64_t)unit + (v0 + j <= vl ? v0 + j : vl);
            mv[j] = a.part_ml[slot * 128 + row];
            lv[j] = a.part_ml[slot * 128 + 64 + row];
            ov[j] = *(const f16x8*)(a.part_o + slot * (kUnitRows * kD) + (int64_t)row * kD + d0);
        }
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j)
            if (v0 + j > vl) {
                mv[j] = -INFINITY;
                lv[j] = 0.0f;
            }
        float Mn = M;
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) Mn = fmaxf(Mn, mv[j]);
        const float Mu = (Mn == -INFINITY) ? 0.0f : Mn;
        const float sc = __builtin_amdgcn_exp2f(M - Mu);
        L *= sc;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] *= sc;
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            const float w = __builtin_amdgcn_exp2f(mv[j] - Mu) * lv[j];
            L += w;
#pragma unroll
            for (int x = 0; x < 8; ++x) acc[x] += (float)ov[j][x] * w;
        }
        M = Mn;
    }
    int i, hq;
    query_row(a, g, rp, i, hq);
    const float inv = 1.0f / L;
    bf16x8 out;
#pragma unroll
    for (int x = 0; x < 8; ++x) out[x] = (__bf16)(acc[x] * inv);
    *(bf16x8*)(a.o + ((int64_t)i * a.Hq + hq) * kD + d0) = out;
    if (d0 == 0 && a.lse) a.lse[(int64_t)i * a.Hq + hq] = (M + log2f(L)) * kLn2;
}

// ---------------------------------------------------------------------------
// FP32 path: one wave per (tree row, query head).
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

// One workgroup of four waves per (tree row, query head).  Keys in blocks of 64,
// dealt to the waves in turn (block j to wave j mod 4), each wave running an online
// softmax over its blocks: lane c scores key k0 + c in full (q broadcast from LDS),
// one wave maximum and sum per block, then P V with lane = head dimension (two per
// lane when D > 64), the block's probabilities taken from their lanes by readlane.
// Invisible keys (tree rows off the row's root path) score -inf.  The four partial
// (max, sum, output) are combined through LDS.
constexpr int kF32Waves = 4;

__global__ __launch_bounds__(kF32Waves * 64) void tree_attn_f32_kernel(AttnF32Args a) {
    __shared__ __attribute__((aligned(16))) float s_q[128];
    __shared__ float s_ml[2][kF32Waves];
    __shared__ float s_o[kF32Waves][128];
    const int i = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
    const int wid = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int g = hq / a.G;
    const int ctx = a.ctx_len[b], S = ctx + a.T, D = a.D;
    const uint64_t mword = a.mask[(int64_t)b * a.T + i];
    const float* qrow = a.q + (((int64_t)b * a.T + i) * a.Hq + hq) * D;
    if (threadIdx.x < D) s_q[threadIdx.x] = qrow[threadIdx.x] * a.scale;
    __syncthreads();
    const int64_t base = ((int64_t)g * a.kv_rows_total + a.kv_row_off[b]) * D;
    float m = -INFINITY, l = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int k0 = wid * kWave; k0 < S; k0 += kF32Waves * kWave) {
        const int c = k0 + lane;
        const bool vis = c < S && (c < ctx || ((mword >> (c - ctx)) & 1ull));
        float s = -INFINITY;
        if (vis) {
            const float* kr = a.k + base + (int64_t)c * D;
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if ((D & 3) == 0) {  // rows are 16-byte aligned: vector loads, eight in flight
                for (int d0 = 0; d0 < D; d0 += 32) {
                    float4 kv[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        kv[u] = d0 + 4 * u < D ? *reinterpret_cast<const float4*>(kr + d0 + 4 * u)
                                               : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        if (d0 + 4 * u < D) {
                            const float4 qv = *reinterpret_cast<const float4*>(s_q + d0 + 4 * u);
                            acc[0] += qv.x * kv[u].x;
                            acc[1] += qv.y * kv[u].y;
                            acc[2] += qv.z * kv[u].z;
                            acc[3] += qv.w * kv[u].w;
                        }
                    }
                }
            } else {
                for (int d = 0; d < D; ++d) acc[d & 3] += s_q[d] * kr[d];
            }
            s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        }
        const float bmax = wave_max_f32(s);
        if (bmax == -INFINITY) continue;  // nothing visible in this block
        const float m_new = fmaxf(m, bmax);
        const float alpha = expf(m - m_new);  // 0 on the wave's first visible block (m = -inf)
        const float p = vis ? expf(s - m_new) : 0.0f;
        l = l * alpha + wave_sum_f32(p);
        o0 *= alpha;
        o1 *= alpha;
        m = m_new;
        // P V: the V rows of 16 keys requested together; invisible keys have p = 0
        const int nk = S - k0 < kWave ? S - k0 : kWave;
        const float* vb = a.v + base + (int64_t)k0 * D;
        for (int j0 = 0; j0 < nk; j0 += 16) {
            float v0[16], v1[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const bool ok = j0 + u < nk;
                v0[u] = ok && lane < D ? vb[(int64_t)(j0 + u) * D + lane] : 0.0f;
                v1[u] = ok && lane + kWave < D ? vb[(int64_t)(j0 + u) * D + lane + kWave] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), j0 + u));
                o0 += pj * v0[u];
                o1 += pj * v1[u];
            }
        }
    }
    // combine the waves' partials: a wave that saw no visible key has (-inf, 0, 0)
    if (lane == 0) {
        s_ml[0][wid] = m;
        s_ml[1][wid] = l;
    }
    if (lane < D) s_o[wid][lane] = o0;
    if (lane + kWave < D) s_o[wid][lane + kWave] = o1;
    __syncthreads();
    if (wid != 0) return;
    float M = s_ml[0][0];
#pragma unroll
    for (int w = 1; w < kF32Waves; ++w) M = fmaxf(M, s_ml[0][w]);
    float L = 0.0f, r0 = 0.0f, r1 = 0.0f;
#pragma unroll
    for (int w = 0; w < kF32Waves; ++w) {
        const float sc = s_ml[1][w] > 0.0f ? expf(s_ml[0][w] - M) : 0.0f;
        L += s_ml[1][w] * sc;
        if (lane < D) r0 += s_o[w][lane] * sc;
        if (lane + kWave < D) r1 += s_o[w][lane + kWave] * sc;
    }
    float* orow = a.o + (((int64_t)b * a.T + i) * a.Hq + hq) * D;
    if (lane < D) orow[lane] = r0 / L;
    if (lane + kWave < D) orow[lane + kWave] = r1 / L;
    if (lane == 0 && a.lse) a.lse[((int64_t)b * a.T + i) * a.Hq + hq] = M + logf(L);
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

bool attention_split_fits(const eagle_attn_desc& d) {
    if (d.dtype != EAGLE_BF16) return true;
    const int64_t G = d.n_q_heads / d.n_kv_heads;
    const int64_t units = (int64_t)d.n_kv_heads * ((G * d.T + kUnitRows - 1) / kUnitRows);
    const int64_t tiles = (d.kv_rows_total + kTileKeys - 1) / kTileKeys;  // bounds ctx + T of any sequence
    return units * (4 * tiles + kSegCost4) < ((int64_t)1 << 31);
}

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
        tree_attn_f32_kernel<<<dim3(d.T, d.n_q_heads, d.batch), kF32Waves * 64, 0, stream>>>(a);
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
        a.ctx_h = d.ctx_len_host ? d.ctx_len_host[b] : -1;
        a.row0_h = d.kv_row_off_host ? d.kv_row_off_host[b] : 0;
        if (a.ctx_h >= 0)  // 4 computing waves + 4 loaders per workgroup
            tree_attn_bf16_kernel<true><<<kGridWG, kThreads, 0, stream>>>(a);
        else
            tree_attn_bf16_kernel<false><<<kGridWG, kThreads, 0, stream>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int units = d.n_kv_heads * RG;
        const int merge_wg = 8 * ((units + 7) / 8) * kRowBlocks;
        MergePlan plan;
        plan.n_wg = 0;
        if (a.ctx_h >= 0 && merge_wg <= kPlanWgs) {
            // the same split the main kernel makes, and the same workgroup -> unit map
            // the merge kernel would compute, evaluated here once
            const Split sp = make_split(a.ctx_h + d.T, units, kGridWG);
            for (int wg = 0; wg < merge_wg; ++wg) {
                const int xcd = wg & 7, j = wg >> 3;
                const int u = merge_unit_first(xcd, units) + j / kRowBlocks;
                uint32_t e = 0;
                if (u < merge_unit_first(xcd + 1, units)) {
                    const uint32_t p0 = (uint32_t)u * sp.W + kSegCost4;
                    const uint32_t vf = (uint32_t)stretch_of(sp, p0);
                    const uint32_t vl = (uint32_t)stretch_of(sp, p0 + 4u * (uint32_t)(sp.nt - 1));
                    e = (1u << 31) | ((uint32_t)u << 16) | (vf << 8) | vl;
                }
                plan.e[wg] = e;
            }
            plan.n_wg = merge_wg;
        }
        if (a.ctx_h >= 0)
            tree_attn_merge_kernel<true><<<merge_wg, 256, 0, stream>>>(a, kGridWG, plan);
        else
            tree_attn_merge_kernel<false><<<merge_wg, 256, 0, stream>>>(a, kGridWG, plan);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int attention_max_batch() { return 1024; }

}  // namespace eagle
