// Work plan of the bf16 tree-attention kernel, as plain integer arithmetic that
// the kernel and a host-side checker share.
//
// Units.  Sequence b of a launch owns UPS = n_kv_heads * RG units (KV head g, row
// group rg of 64 packed query rows; unit index inside the sequence uis = g * RG +
// rg).  Unit (b, uis) covers the S_b = ctx_b + T keys of sequence b: nt_b =
// ceil(S_b / 64) tiles of 64 keys.
//
// Cost line.  The units of all sequences, sequence after sequence, are laid on one
// line; a unit of sequence b costs W_b = 4 * nt_b + kSegCost steps: kSegCost steps
// standing for the fixed work of a segment (its key-half merge and its output),
// then 4 steps per tile.  cost0[b] = steps before sequence b's first unit;
// cost0[B] = Wt, the whole line.  The line is cut into nwg equal stretches
// (stretch v = [floor(Wt v / nwg), floor(Wt (v + 1) / nwg))), nwg <= Wt / 4 so every
// stretch is at least one tile long, and nwg <= kMaxPieces per unit so that few
// units are not cut into more pieces than one workgroup can merge quickly;
// workgroup v takes the tiles that start in its stretch.  A stretch that falls
// wholly in the kSegCost steps before a unit's first tile holds no tile and its
// workgroup exits.
//
// Segments and pieces.  The tiles a workgroup takes from one unit form a segment.
// A unit whose tiles all lie in one stretch is whole: that workgroup writes its
// output.  Otherwise each stretch holding some of its tiles computes a piece
// (stretches vf .. vl, all non-empty) and writes a partial to slot 2 v + from0
// (from0: the piece starts at the unit's first key, i.e. v == vf); a second kernel
// merges them.  A stretch holds at most one from0 piece of a split unit (its last
// segment) and at most one other piece (its first segment), so slots are unique in
// [0, 2 nwg); a split unit is found from its first stretch vf, whose last tile it
// holds while the next stretch starts inside it.
//
// Tables.  The functions take the per-sequence table as an object with
// S(b) (keys), row0(b) (first cache row), cost0(b) and key0(b) (prefixes, b <= B),
// and unit_of(b, c) = c / unit_cost(S(b)) (a table built from host lengths holds
// each sequence's reciprocal of that cost).
#pragma once

#include <stdint.h>

#ifndef EAGLE_HD
#define EAGLE_HD __host__ __device__
#endif

namespace eagle {
namespace plan {

constexpr int kTileKeys = 64;
constexpr int kUnitRows = 64;
constexpr uint32_t kSegCost = 16;
constexpr int kMaxSeqs = 256;  // sequences per launch (the per-sequence table lives in LDS)
constexpr int kMaxPieces = 32;  // stretches per unit on average, at most

// Division by a divisor fixed for a launch, as a multiply and a shift: with
// l = ceil(log2 d) and m = ceil(2^(31 + l) / d), floor(n / d) = floor(n m / 2^(31 + l))
// for every 0 <= n < 2^31 (Granlund and Montgomery, "Division by invariant integers
// using multiplication", 1994: m d = 2^(31+l) + e with 0 <= e < d <= 2^l, so the
// product overshoots n / d by n e / (d 2^(31+l)) < 1 / d, which never reaches the
// next integer).  The host computes (m, 31 + l); m <= 2^32, so n m < 2^63.
struct Recip {
    uint64_t m;
    uint32_t sh;
};
inline Recip recip_of(uint32_t d) {  // 1 <= d < 2^31
    uint32_t l = 0;
    while ((1u << l) < d) ++l;
    const uint64_t p = 1ull << (31 + l);
    return Recip{(p + d - 1) / d, 31 + l};
}
EAGLE_HD inline uint32_t div_by(uint32_t n, const Recip& r) { return (uint32_t)(((uint64_t)n * r.m) >> r.sh); }

EAGLE_HD inline int tiles_of(int S) { return (S + kTileKeys - 1) / kTileKeys; }
EAGLE_HD inline uint32_t unit_cost(int S) { return 4u * (uint32_t)tiles_of(S) + kSegCost; }

struct Split {
    uint32_t Wt;    // cost steps in all
    uint32_t q, r;  // Wt = q * nwg + r
    int nwg;        // stretches (workgroups that take part)
    Recip rn;       // division by nwg; m == 0: not computed (plain division)
};
EAGLE_HD inline Split make_split(uint32_t Wt, int grid, int units) {
    Split sp;
    sp.Wt = Wt;
    if ((int64_t)units * kMaxPieces < (int64_t)grid) grid = units * kMaxPieces;
    const uint32_t most = Wt / 4;
    sp.nwg = most < (uint32_t)grid ? (most > 0 ? (int)most : 1) : grid;
    sp.q = Wt / (uint32_t)sp.nwg;
    sp.r = Wt - sp.q * (uint32_t)sp.nwg;
    sp.rn = Recip{0, 0};
    return sp;
}
// The same with the reciprocal of nwg (host side).
inline Split make_split_recip(uint32_t Wt, int grid, int units) {
    Split sp = make_split(Wt, grid, units);
    sp.rn = recip_of((uint32_t)sp.nwg);
    return sp;
}
// First cost step of stretch v (v = nwg gives Wt): floor(Wt * v / nwg).
EAGLE_HD inline uint32_t stretch_start(const Split& sp, int v) {
    const uint32_t rv = sp.r * (uint32_t)v;  // < nwg * (nwg + 1)
    return sp.q * (uint32_t)v + (sp.rn.m ? div_by(rv, sp.rn) : rv / (uint32_t)sp.nwg);
}
// The stretch holding cost step p < Wt.
EAGLE_HD inline int stretch_of(const Split& sp, uint32_t p) {
    int v = (int)((uint64_t)p * (uint64_t)sp.nwg / (uint64_t)sp.Wt);
    if (v > sp.nwg - 1) v = sp.nwg - 1;
    while (v + 1 < sp.nwg && stretch_start(sp, v + 1) <= p) ++v;
    while (v > 0 && stretch_start(sp, v) > p) --v;
    return v;
}

// Largest b < B with cost0(b) <= p.
template <class Tab>
EAGLE_HD inline int seq_of_tab(const Tab& tab, int B, uint32_t p) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tab.cost0(mid) <= p) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// A tile: sequence b, unit uis inside it, tile index.  b == B: past the last unit.
struct Pos {
    int b, uis, tile;
};
// The first tile starting at or after cost step p.
template <class Tab>
EAGLE_HD inline Pos split_tile(const Tab& tab, int B, int UPS, uint32_t p) {
    Pos t;
    if (p >= tab.cost0(B)) {
        t.b = B;
        t.uis = 0;
        t.tile = 0;
        return t;
    }
    t.b = seq_of_tab(tab, B, p);
    const int S = tab.S(t.b);
    const uint32_t W = unit_cost(S);
    const uint32_t local = p - tab.cost0(t.b);
    t.uis = (int)tab.unit_of(t.b, local);
    const uint32_t r = local - (uint32_t)t.uis * W;
    t.tile = r <= kSegCost ? 0 : (int)((r - kSegCost + 3) / 4);
    if (t.tile >= tiles_of(S)) {
        t.tile = 0;
        if (++t.uis == UPS) {
            t.uis = 0;
            ++t.b;
        }
    }
    return t;
}
// Cost step of unit (b, uis)'s first tile.
template <class Tab>
EAGLE_HD inline uint32_t first_tile_step(const Tab& tab, int b, int uis) {
    return tab.cost0(b) + (uint32_t)uis * unit_cost(tab.S(b)) + kSegCost;
}
// Keys before tile position t on the line of all units' keys (key0(b) = keys of
// the units of sequences before b; key0(B) = all keys).
template <class Tab>
EAGLE_HD inline int64_t key_index(const Tab& tab, int B, const Pos& t) {
    if (t.b >= B) return tab.key0(B);
    return tab.key0(t.b) + (int64_t)t.uis * tab.S(t.b) + (int64_t)t.tile * kTileKeys;
}

// Walk of one workgroup over the keys of its stretch.  It carries the current
// sequence's keys and first row, so the table is read only where the walk enters
// the next sequence.
struct Walker {
    int x;                // keys walked since the stretch start
    int b, uis, g, rg;    // current unit: sequence, unit in it, KV head, row group
    int key0;             // first key of the next tile inside the unit
    int S;                // keys of the current unit
    int64_t row0;         // first cache row of the current sequence
};
struct Tile {
    int b, uis, g, rg;
    int key0, nkeys, S;
    int64_t row0;
    bool seg_start, seg_end;
};
// rRG: division by RG (the host computes it for every launch).
template <class Tab>
EAGLE_HD inline Walker walker_at(const Tab& tab, int RG, const Recip& rRG, const Pos& t) {
    Walker w;
    w.x = 0;
    w.b = t.b;
    w.uis = t.uis;
    w.g = (int)div_by((uint32_t)t.uis, rRG);
    w.rg = t.uis - w.g * RG;
    w.key0 = t.tile * kTileKeys;
    w.S = tab.S(t.b);
    w.row0 = tab.row0(t.b);
    return w;
}
// `len` = keys in the stretch.
EAGLE_HD inline Tile peek(const Walker& w, int len) {
    Tile t;
    t.b = w.b;
    t.uis = w.uis;
    t.g = w.g;
    t.rg = w.rg;
    t.key0 = w.key0;
    t.S = w.S;
    t.row0 = w.row0;
    int n = kTileKeys;
    if (w.S - w.key0 < n) n = w.S - w.key0;
    if (len - w.x < n) n = len - w.x;
    t.nkeys = n;
    t.seg_start = (w.x == 0) || (w.key0 == 0);
    t.seg_end = (w.x + n == len) || (w.key0 + n == w.S);
    return t;
}
// Past `nkeys` keys; on leaving a unit, on to the next one (next row group, next KV
// head, next sequence).  The table is read only when the sequence changes, and only
// while it is one of the B sequences.
template <class Tab>
EAGLE_HD inline void advance(Walker& w, int nkeys, const Tab& tab, int B, int RG, int UPS) {
    w.x += nkeys;
    w.key0 += nkeys;
    if (w.key0 == w.S) {
        w.key0 = 0;
        if (++w.rg == RG) {
            w.rg = 0;
            ++w.g;
        }
        if (++w.uis == UPS) {
            w.uis = 0;
            w.g = 0;
            w.rg = 0;
            if (++w.b < B) {
                w.S = tab.S(w.b);
                w.row0 = tab.row0(w.b);
            }
        }
    }
}

// Workgroup blk of a launch runs on XCD blk % 8 (the dispatcher deals workgroups
// to the XCDs in turn).  Of n stretches, XCD x takes [xcd_first(x, n),
// xcd_first(x + 1, n)): one contiguous run each, sizes differing by at most one;
// workgroup blk takes stretch xcd_first(blk % 8, n) + blk / 8 when that lies in
// its XCD's run.
EAGLE_HD inline int xcd_first(int x, int n) { return (x * n + 7) >> 3; }
// The XCD whose run holds stretch v.
EAGLE_HD inline int xcd_of(int v, int n) {
    int x = 0;
    while (x < 7 && xcd_first(x + 1, n) <= v) ++x;
    return x;
}

// Partial slot of a piece (see above).
EAGLE_HD inline int part_slot(int v, bool from0) { return 2 * v + (from0 ? 1 : 0); }

// The split unit whose first stretch is v, if any: stretch v's last tile lies in a
// unit that the next stretch continues, and that unit's first tile lies in v.
// Returns false when there is none; otherwise the unit and its stretches vf = v ..
// vl.  te = split_tile at stretch_start(v + 1).
template <class Tab>
EAGLE_HD inline bool split_unit_from(const Tab& tab, const Split& sp, int B, int /*UPS*/, int v, const Pos& te,
                                     int& b, int& uis, int& vl) {
    if (te.b >= B || te.tile == 0) return false;  // stretch v ends on a unit boundary (or the line's end)
    b = te.b;
    uis = te.uis;
    const uint32_t p0 = first_tile_step(tab, b, uis);
    if (stretch_of(sp, p0) != v) return false;  // the unit started before v: not its first stretch
    vl = stretch_of(sp, p0 + 4u * (uint32_t)(tiles_of(tab.S(b)) - 1));
    return true;
}

// Merge plan, built on the host when it has the context lengths: one 64-bit entry
// per merge workgroup, read by workgroup index alone.  Bit 63 set = in use, then
// sequence b (bits 0..15), unit uis (16..39), first and last stretch vf (40..47)
// and vl (48..55), row block (56..57; a workgroup merges 16 of the unit's 64
// rows).  Each split unit's row blocks go to the XCD whose run holds the unit's
// middle stretch; workgroup 8 j + x runs on XCD x and takes that XCD's j-th entry.
constexpr int kMergeRowBlocks = kUnitRows / 16;
constexpr int kPlanWgs = 256;  // merge workgroups a plan covers (64 split units)
struct MergeEntry {
    int b, uis, vf, vl, rb;
};
EAGLE_HD inline uint64_t merge_pack(int b, int uis, int vf, int vl, int rb) {
    return (1ull << 63) | (uint64_t)(uint32_t)b | ((uint64_t)(uint32_t)uis << 16) | ((uint64_t)(uint32_t)vf << 40) |
           ((uint64_t)(uint32_t)vl << 48) | ((uint64_t)(uint32_t)rb << 56);
}
// False for an unused entry.
EAGLE_HD inline bool merge_unpack(uint64_t e, MergeEntry& m) {
    if (!(e >> 63)) return false;
    m.b = (int)(e & 0xFFFFu);
    m.uis = (int)((e >> 16) & 0xFFFFFFu);
    m.vf = (int)((e >> 40) & 0xFFu);
    m.vl = (int)((e >> 48) & 0xFFu);
    m.rb = (int)((e >> 56) & 3u);
    return true;
}
// Fills e[0 .. kPlanWgs) (unused entries 0) and returns the merge workgroups to
// launch (8 x the most entries any XCD has), or -1 when an XCD would need more
// than kPlanWgs / 8 entries or a field would not fit (B <= 2^16, UPS <= 2^24 and
// nwg <= 256 always fit).  Host side.
template <class Tab>
inline int merge_plan(const Tab& tab, const Split& sp, int B, int UPS, uint64_t* e) {
    if (B > (1 << 16) || UPS > (1 << 24) || sp.nwg > 256) return -1;
    uint64_t by_xcd[8][kPlanWgs / 8];
    int n_xcd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int v = 0; v < sp.nwg; ++v) {
        int b, uis, vl;
        const Pos te = split_tile(tab, B, UPS, stretch_start(sp, v + 1));
        if (!split_unit_from(tab, sp, B, UPS, v, te, b, uis, vl)) continue;
        const int x = xcd_of((v + vl) / 2, sp.nwg);
        for (int rb = 0; rb < kMergeRowBlocks; ++rb) {
            if (n_xcd[x] == kPlanWgs / 8) return -1;
            by_xcd[x][n_xcd[x]++] = merge_pack(b, uis, v, vl, rb);
        }
    }
    int most = 0;
    for (int x = 0; x < 8; ++x) most = n_xcd[x] > most ? n_xcd[x] : most;
    for (int k = 0; k < kPlanWgs; ++k) e[k] = 0;
    for (int j = 0; j < most; ++j)
        for (int x = 0; x < 8; ++x) e[8 * j + x] = j < n_xcd[x] ? by_xcd[x][j] : 0;
    return 8 * most;
}

}  // namespace plan
}  // namespace eagle
