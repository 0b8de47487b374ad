// Tree attention for gfx950 (MI355X).
//
// Page: EAGLE-2 page (news write-up of "EAGLE-2: Faster Inference of Language
// Models with Dynamic Draft Trees"), the passage after the two stages: every
// flattened draft token attends to the whole context and, inside the tree, to its
// own ancestors only (the It / is / a / has example), so one target pass verifies
// every branch at once.
//
// BF16 path (head_dim 128): a main kernel and a merge kernel per launch of up to
// 256 sequences (the work plan is in attn_plan.hpp).
//  * Work unit = (sequence, KV head, group of 64 packed query rows); the packed
//    rows of a KV head are its G = Hq/Hkv query heads x T tree rows.  The 64-key
//    tiles of all units of all the launch's sequences (ctx_b + T keys each) form
//    one list, split over 256 workgroups, one per CU, on tile boundaries and
//    weighted so that a workgroup spanning two units (two segments to merge and
//    write) takes fewer tiles; a workgroup walks from one sequence's units into the
//    next, so short sequences share the GPU instead of each filling it alone.
//    Workgroup index -> list position is XCD-aware (blockIdx % 8 picks the XCD):
//    each XCD takes one contiguous run of stretches, so the units that share K/V
//    rows (GQA) read them through one L2, and most partials of a unit come from
//    one XCD.
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
//    stretches hold the middle of it (measured faster than a merge indexed by
//    unit alone, although the partials are mostly read from beyond L2, where the
//    main kernel's end wrote them back).
#include "attn_plan.hpp"
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
constexpr int kTileKeys = plan::kTileKeys;
constexpr int kUnitRows = plan::kUnitRows;
constexpr int kComputeWaves = 4;                     // 2 query halves x 2 key halves
constexpr int kLoaders = 4;                          // waves that issue the loads
constexpr int kThreads = (kComputeWaves + kLoaders) * 64;
constexpr int kStages = 4;
constexpr int kGridWG = 256;                         // one per CU, multiple of the 8 XCDs
static_assert(kGridWG % 8 == 0, "workgroups are dealt to the 8 XCDs in turn");

using plan::xcd_first;
using plan::xcd_of;
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

using plan::Pos;
using plan::Split;
using plan::Tile;
using plan::Walker;

// One launch: up to plan::kMaxSeqs sequences.  Pointers are offset to the
// launch's first sequence.
constexpr int kArgSeqs = 32;  // up to this batch, a host-computed plan rides in the arguments

// The per-sequence table computed on the host when it knows the context lengths
// (read by the kernel with scalar loads of its arguments; for one sequence it is a
// single cache line, loaded with the other arguments), so the kernel starts with
// no scan and no dependent memory read.
struct HostPlan {
    int32_t S[kArgSeqs];
    int64_t row0[kArgSeqs];
    uint32_t cost0[kArgSeqs + 1];
    int64_t key0[kArgSeqs + 1];
    plan::Recip rW[kArgSeqs];  // division by the sequence's unit cost
};

struct AttnArgs {
    const __bf16* q;           // [B][T][Hq][D]
    const __bf16* k;           // cache base [Hkv][kv_rows_total][D]; sequence b's rows start at its row0
    const __bf16* v;
    const uint64_t* mask;      // [B][T]
    __bf16* o;                 // [B][T][Hq][D]
    float* lse;                // [B][T][Hq] or null
    const int32_t* ctx_len;    // [B], read when there is no host plan
    const int64_t* kv_row_off; // [B]
    _Float16* part_o;          // [2 * grid][64][128]: normalised partial rows of split units
    uint64_t* part_ml;         // [2 * grid][64]: per row (reference max (base 2), row sum) as two fp32
    int64_t kv_rows_total;
    int B, T, Hq, Hkv, G, RG;
    float scale_log2;
    int32_t one_S;             // kOne: the one sequence's keys (ctx + T) and first row
    int64_t one_row0;
    plan::Recip one_rW;        // kOne: division by the sequence's unit cost
    plan::Split sp_h;          // kOne, kHostTab: the work split, with the reciprocal of its stretch count
    plan::Recip rRG, rT;       // division by RG and by T
    const int32_t* rope_pos;   // kRope: tree rows' positions [B][T]
    double rope_turns[kD / 2]; // kRope: base^(-2d/D) / (2 pi), turns per position
    HostPlan hp;               // kHostTab only
};

// The per-sequence table, as the plan functions read it: from the launch
// arguments (host plan) or from LDS (built by the kernel).
struct ArgTab {
    const HostPlan* hp;
    __host__ __device__ int S(int b) const { return hp->S[b]; }
    __host__ __device__ int64_t row0(int b) const { return hp->row0[b]; }
    __host__ __device__ uint32_t cost0(int b) const { return hp->cost0[b]; }
    __host__ __device__ int64_t key0(int b) const { return hp->key0[b]; }
    __host__ __device__ uint32_t unit_of(int b, uint32_t c) const { return plan::div_by(c, hp->rW[b]); }
};
// One sequence whose length the host knows: every entry from two scalar arguments.
struct OneTab {
    int32_t S0;
    int64_t r0;
    int UPS;
    plan::Recip rW;
    __device__ int S(int) const { return S0; }
    __device__ int64_t row0(int) const { return r0; }
    __device__ uint32_t cost0(int b) const { return b == 0 ? 0u : (uint32_t)UPS * plan::unit_cost(S0); }
    __device__ int64_t key0(int b) const { return b == 0 ? 0 : (int64_t)UPS * S0; }
    __device__ uint32_t unit_of(int, uint32_t c) const { return plan::div_by(c, rW); }
};
struct LdsTab {
    const int32_t* s;
    const int64_t* r;
    const uint32_t* c;
    const int64_t* k;
    __device__ int S(int b) const { return s[b]; }
    __device__ int64_t row0(int b) const { return r[b]; }
    __device__ uint32_t cost0(int b) const { return c[b]; }
    __device__ int64_t key0(int b) const { return k[b]; }
    __device__ uint32_t unit_of(int b, uint32_t c) const { return c / plan::unit_cost(s[b]); }
};

// Packed query row -> (tree row, query head); rows past G*T map to row 0.
__device__ __forceinline__ void query_row(const AttnArgs& a, int g, int rp, int& i, int& hq) {
    if (rp >= a.G * a.T) rp = 0;
    const int gi = (int)plan::div_by((uint32_t)rp, a.rT);
    i = rp - gi * a.T;
    hq = g * a.G + gi;
}
// Element offset of (sequence b, tree row i, query head hq) in q / o.
__device__ __forceinline__ int64_t qo_row(const AttnArgs& a, int b, int i, int hq) {
    return (((int64_t)b * a.T + i) * a.Hq + hq) * kD;
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
    const int64_t elt0 = ((int64_t)t.g * a.kv_rows_total + row0 + t.key0) * kD;
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
__device__ __forceinline__ void load_q(const AttnArgs& a, const Tile& t, unsigned char* qslot, uint32_t* mslot,
                                       int li, int lane) {
    vm_wait<63 - kQLoads>();  // at most 63 loads in flight
    const __bf16* qb = a.q + qo_row(a, t.b, 0, 0);
#pragma unroll
    for (int bi = 0; bi < 16 / kLoaders; ++bi) {
        const int blk = bi * kLoaders + li;
        const int rho = blk * 4 + (lane >> 4);
        int i, hq;
        query_row(a, t.g, t.rg * kUnitRows + rho, i, hq);
        const uint32_t off = (uint32_t)((((int64_t)i * a.Hq + hq) * kD) * 2 + (((lane & 15) ^ swz(rho)) << 4));
        dma_b128(qb, off, lds_u32(qslot + blk * 1024));
    }
    if (li == 0) {
        int i, hq;
        query_row(a, t.g, t.rg * kUnitRows + lane, i, hq);
        const uint32_t* mw = (const uint32_t*)(a.mask + (int64_t)t.b * a.T + i);
        dma_b32(mw, lds_u32(mslot));
        dma_b32(mw + 1, lds_u32(mslot + kWave));
    }
}

// Rotary inside the attention kernel (kRope).  A tree's rows sit at a few
// positions (the context length plus the row's depth), so each workgroup keeps in
// LDS the fp32 (cos, sin) of every pair d < 64 at kRopeTab consecutive positions
// lo .. lo + kRopeTab - 1 (a window).  At a rotation (a unit's 64 q rows at a
// segment start, the tree rows' K when their tile lands) the rows are taken window
// by window: lo = the smallest position of the sequence, then the smallest
// position at or past lo + kRopeTab, and so on; one window covers any tree of
// depth below kRopeTab.  All rotation happens in LDS, by all eight waves, one
// (row, 16-byte chunk pair) per thread: the q rows in the Q slot, or in a copy the
// computing waves write when they loaded them directly.
constexpr int kRopeTab = 8;
struct RopeLds {
    float2* cs;     // [kRopeTab][64] (cos, sin) at lo + j, pair d
    int32_t* pos;   // [4][64] positions of the tree rows, sequence b in ring slot b & 3
    double* f;      // [64] turns per position of pair d
    int32_t* info;  // [2] the first sequence's smallest position, and whether one window misses a row
};
// Rotation of the pair (x[e], y[e]) by (c, sn), rounded to bf16.
__device__ __forceinline__ void rope_pair(bf16x8& x, bf16x8& y, int e, float c, float sn) {
    const float xf = (float)x[e], yf = (float)y[e];
    x[e] = (__bf16)(xf * c - yf * sn);
    y[e] = (__bf16)(yf * c + xf * sn);
}
// One LDS row (q or K, 128 bf16 in 16-byte chunks at positions chunk ^ sw) at
// table row j: logical chunk c < 8 and its partner chunk c + 8.
__device__ __forceinline__ void rope_k_lds(const RopeLds& r, int j, unsigned char* row, int c, int sw) {
    bf16x8* px = (bf16x8*)(row + ((c ^ sw) << 4));
    bf16x8* py = (bf16x8*)(row + (((c + 8) ^ sw) << 4));
    bf16x8 vx = *px, vy = *py;
    const float4* t = reinterpret_cast<const float4*>(r.cs) + j * (kD / 4) + 4 * c;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const float4 v = t[x];
        rope_pair(vx, vy, 2 * x, v.x, v.y);
        rope_pair(vx, vy, 2 * x + 1, v.z, v.w);
    }
    *px = vx;
    *py = vy;
}
// Loader wave li == 0: the T positions of sequence b into LDS (lane l reads row
// min(l, T - 1)).
__device__ __forceinline__ void load_pos(const AttnArgs& a, int b, int32_t* dst, int li, int lane) {
    if (li != 0) return;
    vm_wait<62>();
    const int i = lane < a.T ? lane : a.T - 1;
    dma_b32(a.rope_pos + (int64_t)b * a.T + i, lds_u32(dst));
}
// Minimum over the wave, in every lane: row (16-lane) prefix minima by DPP row
// shifts (a lane with no source keeps its own value), then the rows' last lanes
// broadcast into the rows after them; lane 63 ends with the minimum.
__device__ __forceinline__ int wave_min(int x) {
    x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x111, 0xf, 0xf, false));  // row_shr:1
    x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x112, 0xf, 0xf, false));  // row_shr:2
    x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x114, 0xf, 0xf, false));  // row_shr:4
    x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x118, 0xf, 0xf, false));  // row_shr:8
    x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x142, 0xa, 0xf, false));  // row_bcast:15 into rows 1, 3
    x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x143, 0xc, 0xf, false));  // row_bcast:31 into rows 2, 3
    return __builtin_amdgcn_readlane(x, 63);
}

// The tile walk of one workgroup, for the loader wave (kLoader) or a computing
// wave.  Both instantiations share every branch that reaches a barrier, so the
// five waves always meet the same barriers in the same order.
template <bool kLoader, bool kRope, class Tab>
__device__ __forceinline__ void tile_loop(const AttnArgs& a, const Tab& tab, unsigned char* smem,
                                          unsigned char* qslot, uint32_t* mslot, float (*s_ml)[2][2][kWave],
                                          const RopeLds& rl, int wid, int lane, int vwg, int len, Pos tb) {
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

    const int T = a.T;
    const int B = a.B, UPS = a.Hkv * a.RG;
    Walker w0 = plan::walker_at(tab, a.RG, a.rRG, tb);

    // ---- first segment's Q and mask word, straight into registers ----
    const int qrow = 32 * rb + l32;  // this lane's packed query row inside the unit
    bf16x8 qcur[8];
    uint64_t mword_n;
    // Rotary (kRope): the (cos, sin) table holds the window at rt_lo of sequence
    // rt_b.  For sequence rs_b the smallest position rs_min, and rs_multi: whether
    // a row lies past the first window.  Positions of the sequences after the
    // first ride into LDS with the loads (pos_b: the last sequence whose positions
    // were requested).
    constexpr int64_t kNoWindow = INT64_MIN;
    int64_t rt_lo = kNoWindow;
    int rt_b = tb.b, rs_b = tb.b, rs_min = 0, pos_b = tb.b;
    bool rs_multi = false;
    auto build_window = [&](int64_t lo, double f) {  // computing waves; a barrier follows
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int j = wid + 4 * h;
            const int64_t pj = lo + j;
            float c, sn;
            rope_cs_turns(pj > INT_MAX ? INT_MAX : (int)pj, f, c, sn);
            rl.cs[j * (kD / 2) + lane] = make_float2(c, sn);
        }
    };
    // One rotation, run by every wave (the same barriers): the q rows of tile t's
    // unit in q_buf (64 packed rows laid out as in the Q slot) and the tree rows of
    // tile t's K in stage k_st, either may be null; a barrier ends it.  The caller
    // has made q_buf's contents visible to every wave.
    auto rope_event = [&](const Tile& t, unsigned char* q_buf, unsigned char* k_st) {
        const int32_t* sp = rl.pos + (t.b & 3) * kWave;
        if (t.b != rs_b) {  // another sequence (its positions are in LDS)
            const int p = lane < T ? sp[lane] : INT_MAX;
            rs_min = wave_min(p);
            rs_multi = __any(lane < T && (int64_t)p >= (int64_t)rs_min + kRopeTab);
            rs_b = t.b;
        }
        const int task = wid * kWave + lane;  // (row r, chunk pair c) of 64 x 8
        const int r = task >> 3, c = task & 7;
        int qpos = 0, kpos = 0;
        if (q_buf) {
            int i, hq;
            query_row(a, t.g, t.rg * kUnitRows + r, i, hq);
            qpos = sp[i];
        }
        const int ki = t.key0 + r - (t.S - T);  // tree row of K row r
        const bool k_act = k_st && r < t.nkeys && ki >= 0;
        if (k_act) kpos = sp[ki];
        int64_t lo = rs_min;
        for (;;) {
            if (lo != rt_lo || t.b != rt_b) {
                if (!loader) build_window(lo, rl.f[lane]);
                rt_lo = lo;
                rt_b = t.b;
                barrier_lds();
            }
#pragma nounroll
            for (int h = 0; h < 2; ++h) {
                unsigned char* row = (h == 0 ? q_buf : k_st) + r * kRowBytes;
                const int64_t j = (int64_t)(h == 0 ? qpos : kpos) - lo;
                if ((h == 0 ? q_buf != nullptr : k_act) && j >= 0 && j < kRopeTab)
                    rope_k_lds(rl, (int)j, row, c, swz(r));
            }
            if (!rs_multi) break;
            // the next window: the smallest position at or past lo + kRopeTab
            const int p = lane < T ? sp[lane] : 0;
            const bool later = lane < T && p >= lo + kRopeTab;
            if (!__any(later)) break;
            lo = wave_min(later ? p : INT_MAX);
            barrier_lds();  // every wave is done with this window before it is replaced
        }
        barrier_lds();
    };
    // computing waves of key half 0: this lane's q row into buf (the Q slot's layout)
    auto write_q_rows = [&](unsigned char* buf) {
        if (ks != 0) return;
        const int qr = opaque(qrow), hh = opaque(h2);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int c = (2 * kk + hh) ^ swz(qr);
            *(bf16x8*)(buf + qr * kRowBytes + c * 16) = qcur[kk];
        }
    };
    auto read_q_rows = [&](const unsigned char* buf) {
        const int qr = opaque(qrow), hh = opaque(h2);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int c = (2 * kk + hh) ^ swz(qr);
            qcur[kk] = *(const bf16x8*)(buf + qr * kRowBytes + c * 16);
        }
    };
    auto load_q_direct = [&](const Tile& t) {
        int i, hq;
        query_row(a, t.g, t.rg * kUnitRows + qrow, i, hq);
        const __bf16* qp = a.q + qo_row(a, t.b, i, hq);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qcur[kk] = *(const bf16x8*)(qp + 16 * kk + 8 * h2);
        mword_n = a.mask[(int64_t)t.b * T + i];
        wait_direct_loads();
    };

    // this lane's Q row and mask word from the Q slot
    auto read_q_slot = [&]() {
        read_q_rows(qslot);
        const int qr = opaque(qrow);
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
    if (!loader) {
        if (kRope) {
            const int p0 = lane < T ? a.rope_pos[(int64_t)tb.b * T + lane] : 0;
            const double f0 = a.rope_turns[lane];
            load_q_direct(plan::peek(w0, len));
            rs_min = wave_min(lane < T ? p0 : INT_MAX);
            rs_multi = __any(lane < T && (int64_t)p0 >= (int64_t)rs_min + kRopeTab);
            if (wid == 0) {
                rl.pos[(tb.b & 3) * kWave + lane] = p0;
                rl.f[lane] = f0;
                if (lane == 0) {
                    rl.info[0] = rs_min;
                    rl.info[1] = rs_multi ? 1 : 0;
                }
            }
            build_window(rs_min, f0);
            rt_lo = rs_min;
            write_q_rows(smem + 3 * kStageBytes);  // stage 3 is first filled in the loop
        } else {
            load_q_direct(plan::peek(w0, len));
        }
    }
    auto fetch = [&]() {
        const Tile t = plan::peek(wf, len);
        if (loader)
            load_tile(a, t, t.row0, smem + (nl % kStages) * kStageBytes, off4, wid - kComputeWaves, lane);
        if (t.seg_start && nl > 0 && q_slot_tile < 0) {
            if (loader) load_q(a, t, qslot, mslot, wid - kComputeWaves, lane);
            q_slot_tile = nl;
        }
        plan::advance(wf, t.nkeys, tab, B, a.RG, UPS);
        ++nl;
        // the next sequence's positions ride with the last tile before it
        if (kRope && wf.x < len && wf.b != pos_b) {
            pos_b = wf.b;
            if (loader) load_pos(a, wf.b, rl.pos + (wf.b & 3) * kWave, wid - kComputeWaves, lane);
        }
    };
    fetch();
    if (wf.x < len) fetch();
    if (kRope) {
        barrier_lds();  // the first sequence's positions and first window are in LDS
        if (loader) {
            rs_min = uni(rl.info[0]);
            rs_multi = uni(rl.info[1]) != 0;
            rt_lo = rs_min;
        }
        rope_event(plan::peek(w0, len), smem + 3 * kStageBytes, nullptr);
        if (!loader) read_q_rows(smem + 3 * kStageBytes);
    }
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
    Tile tc = plan::peek(wn, len);
    plan::advance(wn, tc.nkeys, tab, B, a.RG, UPS);
    if (kRope && tc.key0 + tc.nkeys > tc.S - T)  // tree rows in tile 0 (its K has landed)
        rope_event(tc, nullptr, smem);
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

    bool q_copied = false;  // kRope: this iteration's q rows were rotated in this tile's K area
    // Software pipeline: iteration it computes the scores of tile it+1 (MFMA)
    // next to the softmax of tile it (VALU), then PV of tile it.
    for (int it = 0;; ++it) {
        const bool has_next = wn.x < len;
        q_copied = false;
        Tile tn;
        bool from0_n = from0_c;
        if (has_next) {
            // tile it+1 has landed; tile it-1's stage is free
            if (loader) loader_wait(nl - it - 2);
            barrier_lds();
            if (wf.x < len) fetch();
            tn = plan::peek(wn, len);
            // kRope: the q rows at a segment start are rotated in the Q slot, or in a copy
            // in this tile's K area (dead since its scores), with the tree rows of the
            // tile just landed (a new sequence's positions landed with an earlier tile)
            unsigned char* q_rot = nullptr;
            unsigned char* const q_copy = smem + (it % kStages) * kStageBytes;
            if (tn.seg_start) {
                if (q_slot_tile == it + 1) {
                    if (kRope) q_rot = qslot;
                    else if (!loader) read_q_slot();
                    q_slot_tile = -1;  // free once every wave has passed the next barrier
                } else {
                    if (!loader) load_q_direct(tn);  // rare (short segments)
                    if (kRope) {
                        if (!loader) write_q_rows(q_copy);
                        q_rot = q_copy;
                        barrier_lds();
                    }
                }
                from0_n = tn.key0 == 0;
            }
            const bool k_tree = kRope && tn.key0 + tn.nkeys > tn.S - T;
            if (kRope && (q_rot || k_tree)) {
                rope_event(tn, q_rot, k_tree ? smem + ((it + 1) % kStages) * kStageBytes : nullptr);
                if (!loader && q_rot) {
                    if (q_rot == qslot) read_q_slot();
                    else read_q_rows(q_copy);
                }
                q_copied = q_rot == q_copy;
            }
        }

        f32x16 snext;
        if (!loader) {
        const unsigned char* sV = smem + (it % kStages) * kStageBytes + kTileBytes;

        // ---- online softmax (base 2): lane = one query row, 16 of its keys ----
        // Raw scores; the scale (> 0) is applied inside the exponent.
        const int ctx = tc.S - T;
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
            if (!has_next || q_copied) barrier_lds();  // q_copied: the q copy there was just read
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
            const int g = tc.g, rg = tc.rg;
            const bool whole = from0_c && tc.key0 + tc.nkeys == tc.S;
            const int slot = plan::part_slot(vwg, from0_c);
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
                const float c0 = a0 * inv, c1 = w1 * inv;  // weights of this half's and the other's values
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
                            w[x] = __builtin_fmaf((float)o1[db & 1][qd][x], c1, acc[4 * qd + x] * c0);
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
                            a.lse[((int64_t)tc.b * T + i) * a.Hq + hq] = (M + log2f(ltot)) * kLn2;
                        }
                    } else {
                        a.part_ml[(int64_t)slot * kUnitRows + qrow] =
                            ((uint64_t)__float_as_uint(ltot) << 32) | __float_as_uint(M);
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
                            *reinterpret_cast<u32x4*>(a.o + qo_row(a, tc.b, i, hq) + 8 * (ln & 15)) = val[r4];
                        }
                    }
                } else {
                    _Float16* const po = a.part_o + (int64_t)slot * (kUnitRows * kD);
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int row = 16 * wid + 4 * r4 + (ln >> 4);
                        if (rg * kUnitRows + row < a.G * T)
                            *reinterpret_cast<u32x4*>(po + row * kD + 8 * (ln & 15)) = val[r4];
                    }
                }
            }
            // the next segment starts from an empty state
            if (has_next) {
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
                m_run = -INFINITY;
                l_run = 0.0f;
            }
        }
        if (!has_next) break;
        if (!loader) sacc = snext;  // the loader waves never compute scores
        tc = tn;
        plan::advance(wn, tn.nkeys, tab, B, a.RG, UPS);
        mword_c = mword_n;
        from0_c = from0_n;
    }
}

// The per-sequence table of a launch built in LDS by wave 0 from the sequences'
// lengths and first rows: S = ctx + T, cost and key prefixes (wave scans).
__device__ __forceinline__ void build_table(const int32_t* ctx_len, const int64_t* kv_row_off, int B, int T,
                                            int UPS, int32_t* s_S, int64_t* s_row0, uint32_t* s_cost0,
                                            int64_t* s_key0, int lane) {
    uint32_t cost_run = 0;
    int64_t key_run = 0;
    for (int base = 0; base < B; base += kWave) {
        const int b = base + lane;
        int S = 0;
        if (b < B) {
            S = ctx_len[b] + T;
            s_S[b] = S;
            s_row0[b] = kv_row_off[b];
        }
        uint32_t ci = b < B ? (uint32_t)UPS * plan::unit_cost(S) : 0u;
        int64_t ki = b < B ? (int64_t)UPS * S : 0;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const uint32_t cu = __shfl_up(ci, off, kWave);
            const uint32_t klo = __shfl_up((uint32_t)ki, off, kWave);
            const uint32_t khi = __shfl_up((uint32_t)((uint64_t)ki >> 32), off, kWave);
            if (lane >= off) {
                ci += cu;
                ki += (int64_t)(((uint64_t)khi << 32) | klo);
            }
        }
        if (b < B) {
            s_cost0[b + 1] = cost_run + ci;
            s_key0[b + 1] = key_run + ki;
        }
        cost_run += __shfl(ci, kWave - 1, kWave);
        key_run += (int64_t)(((uint64_t)__shfl((uint32_t)((uint64_t)ki >> 32), kWave - 1, kWave) << 32) |
                             __shfl((uint32_t)ki, kWave - 1, kWave));
    }
    if (lane == 0) {
        s_cost0[0] = 0;
        s_key0[0] = 0;
    }
}

// One launch covers B <= plan::kMaxSeqs sequences.  The per-sequence table comes
// from the host (kHostTab: up to kArgSeqs sequences, in the launch arguments;
// kOne: one sequence, two scalar arguments) or is built by the kernel from the
// device arrays of lengths and first rows.
constexpr int kDevTab = 0, kHostTab = 1, kOne = 2;
template <int kMode, bool kRope>
__global__ __launch_bounds__(kThreads, 1) void tree_attn_bf16_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStageBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char qslot[kQBytes];
    __shared__ uint32_t mslot[2 * kWave];
    __shared__ float s_ml[2][2][2][kWave];  // [key half][query half][max, sum][lane]
    __shared__ __attribute__((aligned(16))) float2 s_rcs[kRope ? kRopeTab * kD / 2 : 2];
    __shared__ int32_t s_rpos[kRope ? 4 * kWave : 1];
    __shared__ double s_rf[kRope ? kD / 2 : 1];
    __shared__ int32_t s_rinfo[2];
    const RopeLds rl{s_rcs, s_rpos, s_rf, s_rinfo};

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int B = a.B;
    const int UPS = a.Hkv * a.RG;
    const int xcd = blockIdx.x & 7;
    // waves 0..3 compute (query half, key half); waves 4..7 issue every K, V and Q
    // load and wait for them, so no computing wave stalls on a load issue.  Both
    // roles run the same tile walk and the same barriers.
    auto walk = [&](const auto& tab, int vwg, int len, const Pos& tb) {
        if (wid >= kComputeWaves)
            tile_loop<true, kRope>(a, tab, smem, qslot, mslot, s_ml, rl, wid, lane, vwg, len, tb);
        else
            tile_loop<false, kRope>(a, tab, smem, qslot, mslot, s_ml, rl, wid, lane, vwg, len, tb);
    };
    if constexpr (kMode == kOne) {
        const OneTab tab{a.one_S, a.one_row0, UPS, a.one_rW};
        const Split sp = a.sp_h;  // make_split(cost0(1), gridDim.x, UPS), from the host
        const int vwg = xcd_first(xcd, sp.nwg) + (blockIdx.x >> 3);
        if (vwg >= xcd_first(xcd + 1, sp.nwg)) return;  // nwg <= gridDim.x: every stretch has a workgroup
        const Pos tb = plan::split_tile(tab, 1, UPS, plan::stretch_start(sp, vwg));
        const Pos te = plan::split_tile(tab, 1, UPS, plan::stretch_start(sp, vwg + 1));
        const int64_t x_begin = plan::key_index(tab, 1, tb), x_end = plan::key_index(tab, 1, te);
        if (x_begin >= x_end) return;  // a stretch in the steps before a unit's first tile
        walk(tab, vwg, (int)(x_end - x_begin), tb);
    } else if constexpr (kMode == kHostTab) {
        const ArgTab tab{&a.hp};
        const Split sp = a.sp_h;  // make_split(cost0[B], gridDim.x, B * UPS), from the host
        const int vwg = xcd_first(xcd, sp.nwg) + (blockIdx.x >> 3);
        if (vwg >= xcd_first(xcd + 1, sp.nwg)) return;  // nwg <= gridDim.x: every stretch has a workgroup
        const Pos tb = plan::split_tile(tab, B, UPS, plan::stretch_start(sp, vwg));
        const Pos te = plan::split_tile(tab, B, UPS, plan::stretch_start(sp, vwg + 1));
        const int64_t x_begin = plan::key_index(tab, B, tb), x_end = plan::key_index(tab, B, te);
        if (x_begin >= x_end) return;  // a stretch in the steps before a unit's first tile
        walk(tab, vwg, (int)(x_end - x_begin), tb);
    } else {
        __shared__ int32_t s_S[plan::kMaxSeqs];
        __shared__ int64_t s_row0[plan::kMaxSeqs];
        __shared__ uint32_t s_cost0[plan::kMaxSeqs + 1];
        __shared__ int64_t s_key0[plan::kMaxSeqs + 1];
        if (wid == 0) build_table(a.ctx_len, a.kv_row_off, B, a.T, UPS, s_S, s_row0, s_cost0, s_key0, lane);
        __syncthreads();
        const LdsTab tab{s_S, s_row0, s_cost0, s_key0};
        const Split sp = plan::make_split(s_cost0[B], (int)gridDim.x, B * UPS);
        const int vwg = xcd_first(xcd, sp.nwg) + (blockIdx.x >> 3);
        if (vwg >= xcd_first(xcd + 1, sp.nwg)) return;
        const Pos tb = plan::split_tile(tab, B, UPS, plan::stretch_start(sp, vwg));
        const Pos te = plan::split_tile(tab, B, UPS, plan::stretch_start(sp, vwg + 1));
        const int64_t x_begin = plan::key_index(tab, B, tb), x_end = plan::key_index(tab, B, te);
        if (x_begin >= x_end) return;
        walk(tab, vwg, (int)(x_end - x_begin), tb);
    }
}

// ---------------------------------------------------------------------------
// Merge: one workgroup per (split unit, 16 query rows); thread = (row, 8 dims).
// The partials of the unit's pieces are combined kMergeBatch at a time, their
// loads issued together.  With a host plan, workgroup blk runs on XCD blk % 8
// and merges rows of a unit whose middle piece that XCD computed; without one,
// workgroup (v, row block) merges the split unit whose first stretch is v, if any.
// ---------------------------------------------------------------------------
constexpr int kMergeBatch = 8;
constexpr int kRowBlocks = plan::kMergeRowBlocks;
// One entry per merge workgroup (attn_plan.hpp: merge_plan, merge_unpack).
struct MergePlan {
    uint64_t e[plan::kPlanWgs];
};
struct MergeArgs {
    __bf16* o;
    float* lse;
    const _Float16* part_o;
    const uint64_t* part_ml;
    const int32_t* ctx_len;
    const int64_t* kv_row_off;
    int B, T, Hq, Hkv, G, RG;
    plan::Recip rRG, rT;         // division by RG and by T
    int n_merge;                 // workgroups of the merge proper; kRope: the rest rotate the cache
    // kRope: the tree rows' K in the cache, rotated in place as the rotary call does
    uint16_t* k;
    int64_t kv_rows_total;
    const int32_t* rope_pos;     // [B][T]
    double rope_f[kD / 2];       // base^(-2d/D)
    int64_t krow_h[kArgSeqs];    // with a host plan: sequence b's first tree row
    MergePlan mp;                // kHostPlan only
};

// kRope: the K of the tree rows in the cache rotated in place, with the rotary
// call's arithmetic (fp64 angle, cosine, sine and rotation; fp32, then bf16), so
// the cache ends as that call leaves it.  One workgroup per (tree row, sequence,
// 16 KV heads); thread = (coordinate pair d < 64, every fourth head).  The main
// kernel has read these rows unrotated (it rotates its own copies in LDS); this
// kernel runs after it.
template <bool kHostPlan>
__device__ __forceinline__ void rope_cache_rows(const MergeArgs& m, int x) {
    const int slices = (m.Hkv + 15) / 16;
    const int rest = (int)plan::div_by((uint32_t)x, m.rT), i = x - rest * m.T;
    const int slice = rest % slices, b = rest / slices;
    const int d = threadIdx.x & 63, grp = threadIdx.x >> 6;
    const int64_t krow = kHostPlan ? m.krow_h[b] + i : m.kv_row_off[b] + (int64_t)m.ctx_len[b] + i;
    if (krow < 0 || krow >= m.kv_rows_total) return;  // outside the cache: not rotated
    const int pos = m.rope_pos[(int64_t)b * m.T + i];
    uint16_t* rows[4];
    double xv[4], yv[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        const int h = slice * 16 + grp + 4 * s4;
        rows[s4] = h < m.Hkv ? m.k + ((int64_t)h * m.kv_rows_total + krow) * kD : nullptr;
        if (rows[s4]) {
            xv[s4] = (double)__uint_as_float((uint32_t)rows[s4][d] << 16);
            yv[s4] = (double)__uint_as_float((uint32_t)rows[s4][d + 64] << 16);
        }
    }
    double sn, cs;
    sincos((double)pos * m.rope_f[d], &sn, &cs);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        if (rows[s4]) {
            float xr, yr;
            rope_rotate_f64(xv[s4], yv[s4], cs, sn, xr, yr);
            rows[s4][d] = bf16_bits_rne(xr);
            rows[s4][d + 64] = bf16_bits_rne(yr);
        }
    }
}

template <bool kHostPlan, bool kRope>
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(MergeArgs m) {
    const int tid = threadIdx.x;
    if (kRope && (int)blockIdx.x >= m.n_merge) {
        rope_cache_rows<kHostPlan>(m, (int)blockIdx.x - m.n_merge);
        return;
    }
    int b, uis, vf, vl, rb;
    if constexpr (kHostPlan) {
        plan::MergeEntry me;
        if (!plan::merge_unpack(m.mp.e[blockIdx.x], me)) return;
        b = me.b;
        uis = me.uis;
        vf = me.vf;
        vl = me.vl;
        rb = me.rb;
    } else {
        __shared__ int32_t s_S[plan::kMaxSeqs];
        __shared__ int64_t s_row0[plan::kMaxSeqs];
        __shared__ uint32_t s_cost0[plan::kMaxSeqs + 1];
        __shared__ int64_t s_key0[plan::kMaxSeqs + 1];
        const int UPS = m.Hkv * m.RG;
        if (tid < kWave) build_table(m.ctx_len, m.kv_row_off, m.B, m.T, UPS, s_S, s_row0, s_cost0, s_key0, tid);
        __syncthreads();
        const LdsTab tab{s_S, s_row0, s_cost0, s_key0};
        const Split sp = plan::make_split(s_cost0[m.B], kGridWG, m.B * UPS);
        const int v = blockIdx.x / kRowBlocks;
        rb = blockIdx.x % kRowBlocks;
        if (v >= sp.nwg) return;
        const Pos te = plan::split_tile(tab, m.B, UPS, plan::stretch_start(sp, v + 1));
        if (!plan::split_unit_from(tab, sp, m.B, UPS, v, te, b, uis, vl)) return;
        vf = v;
    }
    const int g = (int)plan::div_by((uint32_t)uis, m.rRG), rg = uis - g * m.RG;
    const int row = rb * 16 + (tid >> 4);
    const int d0 = (tid & 15) * 8;
    const int rp = rg * kUnitRows + row;
    if (rp >= m.G * m.T) return;
    float M = -INFINITY, L = 0.0f;
    float acc[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] = 0.0f;
    for (int v0 = vf; v0 <= vl; v0 += kMergeBatch) {
        uint64_t ml[kMergeBatch];
        f16x8 ov[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            // pieces past the last re-read the last one and get zero weight
            const int v = v0 + j <= vl ? v0 + j : vl;
            const int64_t slot = plan::part_slot(v, v == vf);
            ml[j] = m.part_ml[slot * kUnitRows + row];
            ov[j] = *(const f16x8*)(m.part_o + slot * (kUnitRows * kD) + (int64_t)row * kD + d0);
        }
        float mv[kMergeBatch], lv[kMergeBatch];
        float Mn = M;
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            const bool live = v0 + j <= vl;
            mv[j] = live ? __uint_as_float((uint32_t)ml[j]) : -INFINITY;
            lv[j] = live ? __uint_as_float((uint32_t)(ml[j] >> 32)) : 0.0f;
            Mn = fmaxf(Mn, mv[j]);
        }
        const float Mu = (Mn == -INFINITY) ? 0.0f : Mn;
        const float sc = __builtin_amdgcn_exp2f(M - Mu);
        L *= sc;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] *= sc;
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            // a piece that saw none of a row's keys has (max -inf, sum 0): weight 0
            const float w = __builtin_amdgcn_exp2f(mv[j] - Mu) * lv[j];
            L += w;
#pragma unroll
            for (int x = 0; x < 8; ++x) acc[x] += (float)ov[j][x] * w;
        }
        M = Mn;
    }
    const int gi = (int)plan::div_by((uint32_t)rp, m.rT), i = rp - gi * m.T, hq = g * m.G + gi;
    const float inv = 1.0f / L;
    bf16x8 out;
#pragma unroll
    for (int x = 0; x < 8; ++x) out[x] = (__bf16)(acc[x] * inv);
    *(bf16x8*)(m.o + (((int64_t)b * m.T + i) * m.Hq + hq) * kD + d0) = out;
    if (d0 == 0 && m.lse) m.lse[((int64_t)b * m.T + i) * m.Hq + hq] = (M + log2f(L)) * kLn2;
}

// ---------------------------------------------------------------------------
// FP32 path: one wave per (tree row, query head).
// ---------------------------------------------------------------------------
template <class E>
struct AttnF32Args {
    const E* q;
    const E* k;
    const E* v;
    const uint64_t* mask;
    E* o;
    float* lse;
    const int32_t* ctx_len;
    const int64_t* kv_row_off;
    int64_t kv_rows_total;
    int T, Hq, G, D;
    float scale;
};

// Four consecutive elements (16-byte aligned for fp32, 8-byte for bf16) widened to fp32.
__device__ __forceinline__ float4 load4_f32(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4_f32(const __bf16* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                       __uint_as_float(u.y & 0xFFFF0000u));
}

// Any head_dim up to 128, fp32 or bf16 storage (fp32 arithmetic; a bf16 output is
// rounded once, to nearest even).  One workgroup of eight waves per (tree row, query
// head).  Keys in blocks of 64, dealt to the waves in turn (block j to wave j mod 8),
// each wave running an online softmax over its blocks: lane c scores key k0 + c in
// full (q broadcast from LDS), one wave maximum and sum per block, then P V with lane
// = head dimension (two per lane when D > 64), the block's probabilities taken from
// their lanes by readlane.  Invisible keys (tree rows off the row's root path) score
// -inf.  The eight partial (max, sum, output) are combined through LDS.  (Eight waves
// rather than four: a context of a few hundred keys is then one block per wave, so
// the call's latency is one block's chain of loads: 21.3 -> 19.4 us on a 272-key,
// 64-row call.)
constexpr int kF32Waves = 8;

template <class E>
__global__ __launch_bounds__(kF32Waves * 64) void tree_attn_f32_kernel(AttnF32Args<E> a) {
    __shared__ __attribute__((aligned(16))) float s_q[128];
    __shared__ float s_ml[2][kF32Waves];
    __shared__ float s_o[kF32Waves][128];
    const int i = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
    const int wid = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int g = hq / a.G;
    const int ctx = a.ctx_len[b], S = ctx + a.T, D = a.D;
    const uint64_t mword = a.mask[(int64_t)b * a.T + i];
    const E* qrow = a.q + (((int64_t)b * a.T + i) * a.Hq + hq) * D;
    if ((int)threadIdx.x < D) s_q[threadIdx.x] = (float)qrow[threadIdx.x] * a.scale;
    __syncthreads();
    const int64_t base = ((int64_t)g * a.kv_rows_total + a.kv_row_off[b]) * D;
    float m = -INFINITY, l = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int k0 = wid * kWave; k0 < S; k0 += kF32Waves * kWave) {
        const int c = k0 + lane;
        const bool vis = c < S && (c < ctx || ((mword >> (c - ctx)) & 1ull));
        float s = -INFINITY;
        if (vis) {
            const E* kr = a.k + base + (int64_t)c * D;
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if ((D & 3) == 0) {  // rows aligned for 4-element loads: vector loads, eight in flight
                for (int d0 = 0; d0 < D; d0 += 32) {
                    float4 kv[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        kv[u] = d0 + 4 * u < D ? load4_f32(kr + d0 + 4 * u) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
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
                for (int d = 0; d < D; ++d) acc[d & 3] += s_q[d] * (float)kr[d];
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
        const E* vb = a.v + base + (int64_t)k0 * D;
        for (int j0 = 0; j0 < nk; j0 += 16) {
            float v0[16], v1[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const bool ok = j0 + u < nk;
                v0[u] = ok && lane < D ? (float)vb[(int64_t)(j0 + u) * D + lane] : 0.0f;
                v1[u] = ok && lane + kWave < D ? (float)vb[(int64_t)(j0 + u) * D + lane + kWave] : 0.0f;
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
    E* orow = a.o + (((int64_t)b * a.T + i) * a.Hq + hq) * D;
    if (lane < D) orow[lane] = (E)(r0 / L);
    if (lane + kWave < D) orow[lane + kWave] = (E)(r1 / L);
    if (lane == 0 && a.lse) a.lse[((int64_t)b * a.T + i) * a.Hq + hq] = M + logf(L);
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
    size_t part_o, part_ml, total;
};

// Partial slots of one launch (reused, in stream order, by the next launch).
WsLayout ws_layout(const eagle_attn_desc& d) {
    WsLayout w{0, 0, 0};
    if (d.dtype != EAGLE_BF16 || d.head_dim != kD) return w;
    const size_t slots = 2 * (size_t)kGridWG;
    w.part_o = 0;
    w.part_ml = align_up(slots * kUnitRows * kD * sizeof(_Float16));
    w.total = w.part_ml + align_up(slots * kUnitRows * sizeof(uint64_t));
    return w;
}

// The per-sequence table of up to kArgSeqs sequences, and the merge plan: the
// split units (found as the merge kernel would find them), each of its row blocks
// on the XCD that computed the unit's middle piece.  Returns the merge workgroups
// to launch, or -1 when the plan does not fit kPlanWgs (the merge kernel then
// finds the split units itself).
int host_plan(HostPlan& hp, MergePlan& mp, Split& sp, const int32_t* ctx, const int64_t* row0, int B, int T,
              int UPS) {
    hp.cost0[0] = 0;
    hp.key0[0] = 0;
    for (int b = 0; b < B; ++b) {
        hp.S[b] = ctx[b] + T;
        hp.row0[b] = row0[b];
        hp.rW[b] = plan::recip_of(plan::unit_cost(hp.S[b]));
        hp.cost0[b + 1] = hp.cost0[b] + (uint32_t)UPS * plan::unit_cost(hp.S[b]);
        hp.key0[b + 1] = hp.key0[b] + (int64_t)UPS * hp.S[b];
    }
    const ArgTab tab{&hp};
    sp = plan::make_split_recip(hp.cost0[B], kGridWG, B * UPS);
    return plan::merge_plan(tab, sp, B, UPS, mp.e);
}

}  // namespace

size_t attention_workspace_bytes(const eagle_attn_desc& d) { return ws_layout(d).total; }

bool attention_split_fits(const eagle_attn_desc& d) {
    if (d.dtype != EAGLE_BF16 || d.head_dim != kD) return true;
    // the cost line of one launch, bounded through sum_b ceil(S_b / 64) <=
    // ceil(kv_rows_total / 64) + B (the sequences' rows lie inside the cache)
    const int64_t G = d.n_q_heads / d.n_kv_heads;
    const int64_t ups = (int64_t)d.n_kv_heads * ((G * d.T + kUnitRows - 1) / kUnitRows);
    const int64_t B = d.batch < plan::kMaxSeqs ? d.batch : plan::kMaxSeqs;
    const int64_t tiles = (d.kv_rows_total + kTileKeys - 1) / kTileKeys + B;
    return ups * (4 * tiles + (int64_t)plan::kSegCost * B) < ((int64_t)1 << 31);
}

hipError_t launch_attention(const eagle_attn_desc& d, const void* q, const void* k, const void* v,
                            const uint64_t* mask, void* o, float* lse, void* workspace, hipStream_t stream,
                            const int32_t* rope_position, double rope_base) {
    const bool rope = rope_position != nullptr;
    const float scale = d.scale != 0.0f ? d.scale : 1.0f / sqrtf((float)d.head_dim);
    const int G = d.n_q_heads / d.n_kv_heads;
    if (d.dtype == EAGLE_F32 || d.head_dim != kD) {  // any head_dim <= 128: the row-per-workgroup kernel
        auto run = [&](auto tag) {
            using E = decltype(tag);
            AttnF32Args<E> a;
            a.q = (const E*)q; a.k = (const E*)k; a.v = (const E*)v;
            a.mask = mask; a.o = (E*)o; a.lse = lse;
            a.ctx_len = d.ctx_len; a.kv_row_off = d.kv_row_off; a.kv_rows_total = d.kv_rows_total;
            a.T = d.T; a.Hq = d.n_q_heads; a.G = G; a.D = d.head_dim; a.scale = scale;
            tree_attn_f32_kernel<E><<<dim3(d.T, d.n_q_heads, d.batch), kF32Waves * 64, 0, stream>>>(a);
        };
        if (d.dtype == EAGLE_F32) run(float{});
        else run(__bf16{});
        return hipGetLastError();
    }
    const WsLayout w = ws_layout(d);
    unsigned char* ws = (unsigned char*)workspace;
    const size_t seq_q = (size_t)d.T * d.n_q_heads * kD;
    const int RG = (G * d.T + kUnitRows - 1) / kUnitRows;
    const int UPS = d.n_kv_heads * RG;
    // One main launch per plan::kMaxSeqs sequences: the split covers every
    // sequence of the launch, so workgroups walk from one sequence's units into
    // the next; then one merge launch for the units split between workgroups.
    for (int b0 = 0; b0 < d.batch; b0 += plan::kMaxSeqs) {
        const int nb = d.batch - b0 < plan::kMaxSeqs ? d.batch - b0 : plan::kMaxSeqs;
        AttnArgs a;
        a.q = (const __bf16*)q + b0 * seq_q;
        a.k = (const __bf16*)k;
        a.v = (const __bf16*)v;
        a.mask = mask + (size_t)b0 * d.T;
        a.o = (__bf16*)o + b0 * seq_q;
        a.lse = lse ? lse + (size_t)b0 * d.T * d.n_q_heads : nullptr;
        a.ctx_len = d.ctx_len + b0;
        a.kv_row_off = d.kv_row_off + b0;
        a.part_o = (_Float16*)(ws + w.part_o);
        a.part_ml = (uint64_t*)(ws + w.part_ml);
        a.kv_rows_total = d.kv_rows_total;
        a.B = nb; a.T = d.T; a.Hq = d.n_q_heads; a.Hkv = d.n_kv_heads; a.G = G; a.RG = RG;
        a.rRG = plan::recip_of((uint32_t)RG);
        a.rT = plan::recip_of((uint32_t)d.T);
        a.scale_log2 = scale * kLog2e;
        a.rope_pos = rope ? rope_position + (size_t)b0 * d.T : nullptr;
        MergeArgs m;
        m.o = a.o;
        m.lse = a.lse;
        m.part_o = a.part_o;
        m.part_ml = a.part_ml;
        m.ctx_len = a.ctx_len;
        m.kv_row_off = a.kv_row_off;
        m.B = nb; m.T = d.T; m.Hq = d.n_q_heads; m.Hkv = d.n_kv_heads; m.G = G; m.RG = RG;
        m.rRG = a.rRG;
        m.rT = a.rT;
        m.k = (uint16_t*)k;
        m.kv_rows_total = d.kv_rows_total;
        m.rope_pos = a.rope_pos;
        if (rope) {
            for (int j = 0; j < kD / 2; ++j) {
                // the rotary call's frequencies, and the same in turns for the fp32 form
                m.rope_f[j] = pow(rope_base, -2.0 * j / kD);
                a.rope_turns[j] = m.rope_f[j] / (2.0 * M_PI);
            }
        }
        // rotary write-back workgroups: (tree row, sequence, 16 KV heads)
        const int rope_wg = rope ? d.T * nb * ((d.n_kv_heads + 15) / 16) : 0;
        // the merge plan packs (sequence, unit) in 16 + 24 bits
        const bool host = d.ctx_len_host && nb <= kArgSeqs && UPS < (1 << 24);
        hipError_t e;
        if (host) {
            const int merge_wg =
                host_plan(a.hp, m.mp, a.sp_h, d.ctx_len_host + b0, d.kv_row_off_host + b0, nb, d.T, UPS);
            a.one_S = a.hp.S[0];
            a.one_row0 = a.hp.row0[0];
            a.one_rW = a.hp.rW[0];
            for (int b = 0; b < nb; ++b) m.krow_h[b] = a.hp.row0[b] + (a.hp.S[b] - d.T);
            // 4 computing waves + 4 loaders per workgroup
            if (nb == 1 && rope)
                tree_attn_bf16_kernel<kOne, true><<<kGridWG, kThreads, 0, stream>>>(a);
            else if (nb == 1)
                tree_attn_bf16_kernel<kOne, false><<<kGridWG, kThreads, 0, stream>>>(a);
            else if (rope)
                tree_attn_bf16_kernel<kHostTab, true><<<kGridWG, kThreads, 0, stream>>>(a);
            else
                tree_attn_bf16_kernel<kHostTab, false><<<kGridWG, kThreads, 0, stream>>>(a);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if (merge_wg >= 0) {
                m.n_merge = merge_wg;
                if (rope)
                    tree_attn_merge_kernel<true, true><<<merge_wg + rope_wg, 256, 0, stream>>>(m);
                else if (merge_wg > 0)
                    tree_attn_merge_kernel<true, false><<<merge_wg, 256, 0, stream>>>(m);
            } else {
                m.n_merge = kRowBlocks * kGridWG;
                if (rope)
                    tree_attn_merge_kernel<false, true><<<m.n_merge + rope_wg, 256, 0, stream>>>(m);
                else
                    tree_attn_merge_kernel<false, false><<<m.n_merge, 256, 0, stream>>>(m);
            }
        } else {
            if (rope)
                tree_attn_bf16_kernel<kDevTab, true><<<kGridWG, kThreads, 0, stream>>>(a);
            else
                tree_attn_bf16_kernel<kDevTab, false><<<kGridWG, kThreads, 0, stream>>>(a);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            m.n_merge = kRowBlocks * kGridWG;
            if (rope)
                tree_attn_merge_kernel<false, true><<<m.n_merge + rope_wg, 256, 0, stream>>>(m);
            else
                tree_attn_merge_kernel<false, false><<<m.n_merge, 256, 0, stream>>>(m);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

int attention_max_batch() { return 1024; }

}  // namespace eagle
