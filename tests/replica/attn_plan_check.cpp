// Host-side check of the bf16 tree-attention work plan (attn_plan.hpp, compiled
// here unchanged): for one launch descriptor, every workgroup's stretch is walked
// exactly as the kernel walks it, and the run fails (assert, or an address
// sanitizer / undefined-behaviour report under -fsanitize) unless
//   * every tile of every unit is taken by exactly one workgroup, and a unit's
//     segments cover its keys 0 .. S-1 in order;
//   * every K/V row a tile loads (full tiles, and the clamped rows of a short one)
//     lies inside its sequence's rows and inside the cache;
//   * every Q row and mask word read, every output row written, lies inside the
//     batch;
//   * partial slots are unique and inside [0, 2 * grid); a split unit's pieces are
//     exactly stretches vf .. vl, its from0 piece is stretch vf, and the merge finds
//     every split unit exactly once, from stretch vf, with the same vl
//     (split_unit_from);
//   * stretch_of maps each tile's cost step to the workgroup that takes it;
//   * a stretch holds at most two pieces: its first segment (not from0) and its
//     last (from0);
//   * the workgroup -> stretch map (XCD runs) gives each stretch one workgroup;
//   * every division the kernel takes from a host reciprocal (by the stretch count,
//     by a sequence's unit cost, by RG and by T) equals the plain division;
//   * xcd_of names the XCD run of every stretch, as the merge plan uses it;
//   * the host's merge plan (merge_plan): every split unit's four row blocks exactly
//     once, with its sequence, unit, vf and vl, each on the XCD whose run holds the
//     unit's middle stretch (entry k runs on XCD k % 8), the unused entries empty,
//     and -1 exactly when an XCD would need more than kPlanWgs / 8 entries.
// Input (stdin): grid T Hq Hkv rows_total B, then B pairs (ctx, row0).
#define EAGLE_HD
#include "../../draft_tree_verification_eagle_amd/csrc/attn_plan.hpp"

#include <cassert>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <vector>

using namespace eagle::plan;

#define CHECK(c)                                                                         \
    do {                                                                                 \
        if (!(c)) {                                                                      \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);         \
            std::abort();                                                                \
        }                                                                                \
    } while (0)

// The table the kernel reads from its launch arguments: unit_of by the host
// reciprocal of each sequence's unit cost, checked against the division.
struct HostTab {
    const int32_t* S_;
    const int64_t* row0_;
    const uint32_t* cost0_;
    const int64_t* key0_;
    const Recip* rW_;
    int S(int b) const { return S_[b]; }
    int64_t row0(int b) const { return row0_[b]; }
    uint32_t cost0(int b) const { return cost0_[b]; }
    int64_t key0(int b) const { return key0_[b]; }
    uint32_t unit_of(int b, uint32_t c) const {
        const uint32_t q = div_by(c, rW_[b]);
        CHECK(q == c / unit_cost(S_[b]));
        return q;
    }
};

int main() {
    int grid, T, Hq, Hkv, B;
    long long rows_total;
    if (std::scanf("%d %d %d %d %lld %d", &grid, &T, &Hq, &Hkv, &rows_total, &B) != 6) return 2;
    CHECK(B >= 1 && B <= kMaxSeqs && T >= 1 && T <= 64 && Hkv >= 1 && Hq % Hkv == 0);
    std::vector<int32_t> S(B);
    std::vector<int64_t> row0(B);
    for (int b = 0; b < B; ++b) {
        int c;
        long long r;
        if (std::scanf("%d %lld", &c, &r) != 2) return 2;
        CHECK(c >= 0 && r >= 0 && r + c + T <= rows_total);
        S[b] = c + T;
        row0[b] = r;
    }
    const int G = Hq / Hkv;
    const int RG = (G * T + kUnitRows - 1) / kUnitRows;
    const int UPS = Hkv * RG;
    // the table the kernel builds (prefix sums as in its wave scan)
    std::vector<uint32_t> cost0(B + 1, 0);
    std::vector<int64_t> key0(B + 1, 0);
    std::vector<Recip> rW(B);
    uint64_t wide = 0;
    for (int b = 0; b < B; ++b) {
        rW[b] = recip_of(unit_cost(S[b]));
        wide += (uint64_t)UPS * unit_cost(S[b]);
        CHECK(wide < (1ull << 31));
        cost0[b + 1] = cost0[b] + (uint32_t)UPS * unit_cost(S[b]);
        key0[b + 1] = key0[b] + (int64_t)UPS * S[b];
    }
    const HostTab tab{S.data(), row0.data(), cost0.data(), key0.data(), rW.data()};
    const Split sp = make_split_recip(cost0[B], grid, B * UPS);
    CHECK(sp.nwg >= 1 && sp.nwg <= grid);
    {
        Split plain = sp;
        plain.rn = Recip{0, 0};
        for (int v = 0; v <= sp.nwg; ++v) CHECK(stretch_start(sp, v) == stretch_start(plain, v));
    }
    const Recip rRG = recip_of((uint32_t)RG), rT = recip_of((uint32_t)T);
    for (int rp = 0; rp < G * T + kUnitRows; ++rp) CHECK(div_by((uint32_t)rp, rT) == (uint32_t)(rp / T));
    for (int u = 0; u < UPS + RG; ++u) CHECK(div_by((uint32_t)u, rRG) == (uint32_t)(u / RG));
    // workgroup -> stretch
    std::vector<int> owner(sp.nwg, -1);
    for (int blk = 0; blk < grid; ++blk) {
        const int xcd = blk & 7;
        const int v = xcd_first(xcd, sp.nwg) + (blk >> 3);
        if (v >= xcd_first(xcd + 1, sp.nwg)) continue;
        CHECK(v >= 0 && v < sp.nwg && owner[v] < 0);
        owner[v] = blk;
    }
    for (int v = 0; v < sp.nwg; ++v) CHECK(owner[v] >= 0);

    // coverage per (b, uis): next key expected
    std::vector<std::vector<int>> next_key(B, std::vector<int>(UPS, 0));
    std::vector<std::vector<int>> pieces(B, std::vector<int>(UPS, 0));
    std::set<int> slots;
    std::map<std::pair<int, int>, std::pair<int, int>> unit_range;  // (b, uis) -> (vf, vl)
    const long long kD = 128;
    for (int v = 0; v < sp.nwg; ++v) {
        const Pos tb = split_tile(tab, B, UPS, stretch_start(sp, v));
        const Pos te = split_tile(tab, B, UPS, stretch_start(sp, v + 1));
        const int64_t xb = key_index(tab, B, tb);
        const int64_t xe = key_index(tab, B, te);
        CHECK(xb <= xe);
        if (xb == xe) continue;
        CHECK(xe - xb < (1ll << 31));
        const int len = (int)(xe - xb);
        CHECK(tb.b < B);
        Walker w = walker_at(tab, RG, rRG, tb);
        bool from0 = false;
        int n_pieces = 0, n_segments = 0;
        while (w.x < len) {
            const Tile t = peek(w, len);
            CHECK(t.b >= 0 && t.b < B && t.uis >= 0 && t.uis < UPS && t.g == t.uis / RG && t.rg == t.uis % RG);
            CHECK(t.S == S[t.b] && t.row0 == row0[t.b] && t.nkeys >= 1 && t.nkeys <= kTileKeys &&
                  t.key0 % kTileKeys == 0);
            CHECK(t.key0 == next_key[t.b][t.uis]);
            next_key[t.b][t.uis] += t.nkeys;
            // the tile's cost step lies in this stretch
            const uint32_t p = first_tile_step(tab, t.b, t.uis) + 4u * (uint32_t)(t.key0 / kTileKeys);
            CHECK(p >= stretch_start(sp, v) && p < stretch_start(sp, v + 1) && stretch_of(sp, p) == v);
            // K / V rows read: key0 .. key0 + 63, rows past nkeys re-read row nkeys - 1
            for (int lrow = 0; lrow < kTileKeys; ++lrow) {
                const int grow = lrow < t.nkeys ? lrow : t.nkeys - 1;
                const long long r = row0[t.b] + t.key0 + grow;
                CHECK(r >= row0[t.b] && r < row0[t.b] + S[t.b] && r < rows_total);
                const long long elt = ((long long)t.g * rows_total + r) * kD;
                CHECK(elt >= 0 && elt + kD <= (long long)Hkv * rows_total * kD);
            }
            if (t.seg_start) {
                from0 = t.key0 == 0;
                // Q rows and mask words of the unit's 64 packed rows (padding rows read row 0)
                for (int rho = 0; rho < kUnitRows; ++rho) {
                    int rp = t.rg * kUnitRows + rho;
                    if (rp >= G * T) rp = 0;
                    const int gi = rp / T, i = rp - gi * T, hq = t.g * G + gi;
                    CHECK(i >= 0 && i < T && hq >= 0 && hq < Hq);
                    const long long qe = (((long long)t.b * T + i) * Hq + hq) * kD;
                    CHECK(qe >= 0 && qe + kD <= (long long)B * T * Hq * kD);
                }
            }
            if (t.seg_end) {
                const bool whole = from0 && t.key0 + t.nkeys == t.S;
                ++n_segments;
                if (!whole) {
                    // a piece is the stretch's first segment (not from0) or its last (from0)
                    ++n_pieces;
                    CHECK(n_pieces <= 2);
                    CHECK(from0 ? (w.x + t.nkeys == len) : (n_segments == 1));
                    const int slot = part_slot(v, from0);
                    CHECK(slot >= 0 && slot < 2 * grid && !slots.count(slot));
                    slots.insert(slot);
                    const uint32_t p0 = first_tile_step(tab, t.b, t.uis);
                    const int vf = stretch_of(sp, p0);
                    const int vl = stretch_of(sp, p0 + 4u * (uint32_t)(tiles_of(t.S) - 1));
                    CHECK(vf < vl && vf >= 0 && vl < sp.nwg && v >= vf && v <= vl);
                    CHECK(from0 == (v == vf));
                    auto key = std::make_pair(t.b, t.uis);
                    auto ur = unit_range.find(key);
                    if (ur == unit_range.end()) unit_range[key] = std::make_pair(vf, vl);
                    else CHECK(ur->second == std::make_pair(vf, vl));
                    ++pieces[t.b][t.uis];
                }
            }
            advance(w, t.nkeys, tab, B, RG, UPS);
        }
    }
    // the merge's discovery of split units: from each stretch, by its end
    std::map<std::pair<int, int>, std::pair<int, int>> found;
    for (int v = 0; v < sp.nwg; ++v) {
        const Pos te = split_tile(tab, B, UPS, stretch_start(sp, v + 1));
        int b, uis, vl;
        if (!split_unit_from(tab, sp, B, UPS, v, te, b, uis, vl)) continue;
        CHECK(b >= 0 && b < B && uis >= 0 && uis < UPS && vl > v && vl < sp.nwg);
        CHECK(!found.count(std::make_pair(b, uis)));
        found[std::make_pair(b, uis)] = std::make_pair(v, vl);
    }
    CHECK(found == unit_range);
    for (int v = 0; v < sp.nwg; ++v) {
        const int x = xcd_of(v, sp.nwg);
        CHECK(x == (owner[v] & 7) && v >= xcd_first(x, sp.nwg) && v < xcd_first(x + 1, sp.nwg));
    }
    // the host's merge plan
    {
        std::vector<uint64_t> e(kPlanWgs, ~0ull);
        const int r = merge_plan(tab, sp, B, UPS, e.data());
        int per_xcd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (const auto& u : found) per_xcd[xcd_of((u.second.first + u.second.second) / 2, sp.nwg)] += kMergeRowBlocks;
        int most = 0;
        for (int x = 0; x < 8; ++x) most = per_xcd[x] > most ? per_xcd[x] : most;
        if (most > kPlanWgs / 8) {
            CHECK(r == -1);
        } else {
            CHECK(r == 8 * most);
            std::map<std::pair<int, int>, int> blocks;  // (b, uis) -> bit mask of row blocks
            for (int k = 0; k < kPlanWgs; ++k) {
                MergeEntry m;
                if (!merge_unpack(e[k], m)) {
                    CHECK(e[k] == 0);
                    continue;
                }
                CHECK(k < r);
                auto it = found.find(std::make_pair(m.b, m.uis));
                CHECK(it != found.end() && it->second == std::make_pair(m.vf, m.vl));
                CHECK(xcd_of((m.vf + m.vl) / 2, sp.nwg) == k % 8);
                CHECK(m.rb >= 0 && m.rb < kMergeRowBlocks);
                int& bits = blocks[std::make_pair(m.b, m.uis)];
                CHECK(!((bits >> m.rb) & 1));
                bits |= 1 << m.rb;
            }
            CHECK(blocks.size() == found.size());
            for (const auto& bl : blocks) CHECK(bl.second == (1 << kMergeRowBlocks) - 1);
        }
    }
    long long split_units = 0;
    for (int b = 0; b < B; ++b)
        for (int u = 0; u < UPS; ++u) {
            CHECK(next_key[b][u] == S[b]);
            auto ur = unit_range.find(std::make_pair(b, u));
            if (ur == unit_range.end()) {
                CHECK(pieces[b][u] == 0);
            } else {
                CHECK(pieces[b][u] == ur->second.second - ur->second.first + 1);
                ++split_units;
            }
        }
    std::printf("ok: %d sequences, %d units each, %d stretches, %lld split units, %zu partial slots\n", B, UPS,
                sp.nwg, split_units, slots.size());
    return 0;
}
