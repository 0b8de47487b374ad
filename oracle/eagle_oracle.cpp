// CPU ORACLE -- TEST INFRASTRUCTURE ONLY.
//
// A plain, slow, single-threaded C++ implementation of one EAGLE-2 draft-tree
// verification step, used to check the HIP library.  Only the test suite, the
// package smoke check and the bench's CPU-baseline leg may load it.  It shares
// no source, header, table or helper with the HIP path.
//
// Pages it follows (cited by title and passage):
//  * EAGLE-2 page: the news write-up of "EAGLE-2: Faster Inference of Language
//    Models with Dynamic Draft Trees" (Japanese body).  Its passage on the two
//    stages (expand / rerank) defines node value, Expand, Rerank and the tie
//    rule; the passage after it defines flattening, the ancestor-only mask (the
//    It / is / a / has example) and the position adjustment; its opening
//    paragraph states that one target forward verifies the draft losslessly.
//  * EAGLE page: abstract of "EAGLE: Speculative Sampling Requires Rethinking
//    Feature Uncertainty" -- output distribution identical to vanilla
//    autoregressive decoding.
//  * CSDN page: blog post "论文解读：eagle/eagle2", section 1.1 (draft stage +
//    parallel verification keeps the distribution) and section 1.2 (lossless
//    under greedy and non-greedy decoding).
//  * Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
//    Easy as 1, 2, 3", SC'11 -- the counter-based generator the sampled
//    acceptance draws its uniforms from.
//
// Readings where the pages are silent are listed in the design notes; the ones
// each function depends on are repeated in its comment.
//
// Pins: every function here is checked by tests against something other than
// itself (brute-force path enumeration, library sorts and softmax, a library
// masked-attention routine, closed-form acceptance laws, Monte-Carlo, and the
// Philox authors' known-answer vectors).
//
// Build: g++ -O2 -std=c++17 -ffp-contract=off -fno-fast-math -shared -fPIC

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// Philox4x32-10 (SC'11 paper): 10 rounds of the 4x32 Philox S-box with the
// paper's two multipliers, the key advanced by the Weyl constants between
// rounds.
// ---------------------------------------------------------------------------
const uint32_t kPhiloxM0 = 0xD2511F53u;
const uint32_t kPhiloxM1 = 0xCD9E8D57u;
const uint32_t kWeyl0 = 0x9E3779B9u;
const uint32_t kWeyl1 = 0xBB67AE85u;

void philox_round(uint32_t c[4], const uint32_t k[2]) {
    uint64_t p0 = (uint64_t)kPhiloxM0 * (uint64_t)c[0];
    uint64_t p1 = (uint64_t)kPhiloxM1 * (uint64_t)c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k[0];
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c[3] ^ k[1];
    uint32_t n3 = lo0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

void philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k[0] += kWeyl0; k[1] += kWeyl1; }
        philox_round(c, k);
    }
    std::memcpy(out, c, sizeof(c));
}

// The uniform for one acceptance decision.  Key = the 64-bit seed split in two
// words; counter = (slot, tree row, sequence, low 32 bits of the step).  The
// top 24 bits of the first output word give u in [0, 1) exactly.
const uint32_t kBonusSlot = 0xFFFFFFFFu;

double uniform_for(uint64_t seed, uint64_t step, uint32_t seq, uint32_t row, uint32_t slot) {
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    uint32_t ctr[4] = {slot, row, seq, (uint32_t)(step & 0xFFFFFFFFu)};
    uint32_t out[4];
    philox4x32_10(ctr, key, out);
    return (double)(out[0] >> 8) * (1.0 / 16777216.0);
}

struct Node {
    int token;
    int parent;
    int depth;
    float value;
};

// True when the fp64 log-normaliser lies within 1e-10 of a point where the
// rounding to fp32 changes; a different fp64 summation order could then round
// to the neighbouring float.
bool lse_rounding_hazard(double lse64, float lse32) {
    float up = std::nextafter(lse32, INFINITY);
    float dn = std::nextafter(lse32, -INFINITY);
    double mid_up = 0.5 * ((double)lse32 + (double)up);
    double mid_dn = 0.5 * ((double)lse32 + (double)dn);
    return std::fabs(lse64 - mid_up) < 1e-10 || std::fabs(lse64 - mid_dn) < 1e-10;
}

}  // namespace

extern "C" {

// ---------------------------------------------------------------------------
// Philox access for the tests (known-answer vectors, uniformity).
// ---------------------------------------------------------------------------
void orc_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
    philox4x32_10(ctr, key, out);
}

double orc_uniform(uint64_t seed, uint64_t step, uint32_t seq, uint32_t row, uint32_t slot) {
    return uniform_for(seed, step, seq, row, slot);
}

// ---------------------------------------------------------------------------
// Tree shape implied by (depth, topk, m): frontier size per layer and the node
// capacity.  Layer 1 expands the root alone; each later layer expands the m
// best nodes of the previous layer (fewer if that layer is smaller).
// ---------------------------------------------------------------------------
int orc_tree_shape(int depth, int topk, int m, int* frontier_sizes, int* capacity) {
    if (depth < 1 || topk < 1 || m < 1) return -1;
    int f = 1, cap = 1;
    for (int l = 0; l < depth; ++l) {
        frontier_sizes[l] = f;
        cap += f * topk;
        f = std::min(m, f * topk);
    }
    *capacity = cap;
    return 0;
}

// ---------------------------------------------------------------------------
// Expand, all layers (EAGLE-2 page, passage on the two stages).
//
// A node's value is the product of the draft confidences on its root path,
// stored as a sum of log-confidences in fp32.  At layer l the frontier is the
// m highest-value nodes of the previous layer (the root at l = 1); each
// frontier node's draft row gives its top-k tokens as children.
//
// Readings used: each expanded node gets top-k children; confidence is the
// softmax of the draft row at temperature 1; top-k ties go to the lower token
// id; frontier order is (value desc, id asc); children are numbered in
// creation order (frontier order, then rank).  The log-normaliser is summed
// in fp64 from the row maximum and rounded to fp32 once; logq and value use
// plain fp32 subtraction and addition.
//
// draft_logits: [R][V] fp32, layer-major, frontier order inside a layer.
// Outputs [cap]: token, parent, depth, value.  row_lse64 / row_hazard: [R].
// Returns 0, or -1 on bad arguments.
// ---------------------------------------------------------------------------
int orc_expand(int V, int depth, int topk, int m, const float* draft_logits, int root_token,
               int* token, int* parent, int* depth_out, float* value, double* row_lse64,
               int* row_hazard, int* n_nodes_out) {
    if (V < 1 || depth < 1 || topk < 1 || topk > V || m < 1) return -1;
    std::vector<Node> nodes;
    nodes.push_back({root_token, -1, 0, 0.0f});
    std::vector<int> frontier = {0};
    std::vector<int> idx(V);
    int row = 0;
    for (int layer = 1; layer <= depth; ++layer) {
        const int layer_begin = (int)nodes.size();
        for (size_t j = 0; j < frontier.size(); ++j, ++row) {
            const int f = frontier[j];
            const float* z = draft_logits + (size_t)row * V;
            float zmax = z[0];
            for (int t = 1; t < V; ++t) if (z[t] > zmax) zmax = z[t];
            double s = 0.0;
            for (int t = 0; t < V; ++t) s += std::exp((double)z[t] - (double)zmax);
            const double lse64 = std::log(s);
            const float lse32 = (float)lse64;
            row_lse64[row] = lse64;
            row_hazard[row] = lse_rounding_hazard(lse64, lse32) ? 1 : 0;
            std::iota(idx.begin(), idx.end(), 0);
            std::partial_sort(idx.begin(), idx.begin() + topk, idx.end(), [z](int a, int b) {
                if (z[a] != z[b]) return z[a] > z[b];
                return a < b;
            });
            for (int r = 0; r < topk; ++r) {
                const int t = idx[r];
                const float shifted = z[t] - zmax;      // fp32
                const float logq = shifted - lse32;     // fp32
                const float val = nodes[f].value + logq;  // fp32
                nodes.push_back({t, f, layer, val});
            }
        }
        if (layer < depth) {
            std::vector<int> layer_ids;
            for (int id = layer_begin; id < (int)nodes.size(); ++id) layer_ids.push_back(id);
            std::stable_sort(layer_ids.begin(), layer_ids.end(), [&](int a, int b) {
                return nodes[a].value > nodes[b].value;  // ids already ascending
            });
            const size_t keep = std::min((size_t)m, layer_ids.size());
            frontier.assign(layer_ids.begin(), layer_ids.begin() + keep);
        }
    }
    for (size_t i = 0; i < nodes.size(); ++i) {
        token[i] = nodes[i].token;
        parent[i] = nodes[i].parent;
        depth_out[i] = nodes[i].depth;
        value[i] = nodes[i].value;
    }
    *n_nodes_out = (int)nodes.size();
    return 0;
}

// ---------------------------------------------------------------------------
// Rerank (EAGLE-2 page, passage on the two stages): sort every non-root node by
// value and keep the first n; equal values keep the shallower node first, then
// the lower id.  The root is always kept and is not counted in n.
// kept: [n] node ids in ascending order.  Returns 0, or -1 when n exceeds the
// number of candidates.
// ---------------------------------------------------------------------------
int orc_rerank(int n_nodes, const float* value, const int* depth, int n, int* kept) {
    if (n < 0 || n > n_nodes - 1) return -1;
    std::vector<int> cand;
    for (int id = 1; id < n_nodes; ++id) cand.push_back(id);
    std::sort(cand.begin(), cand.end(), [&](int a, int b) {
        if (value[a] != value[b]) return value[a] > value[b];
        if (depth[a] != depth[b]) return depth[a] < depth[b];
        return a < b;
    });
    std::vector<int> k(cand.begin(), cand.begin() + n);
    std::sort(k.begin(), k.end());
    for (int i = 0; i < n; ++i) kept[i] = k[i];
    return 0;
}

// ---------------------------------------------------------------------------
// Flatten + mask + positions (EAGLE-2 page, passage after the two stages).
// Flat order: the root, then the kept nodes by ascending id (a topological
// order).  mask[i][j] = 1 iff flat row j lies on the root-to-row-i path, both
// ends included (the It / is / a / has example).  position = ctx_len + depth.
// mask: [T][T] bytes, T = n + 1.  Returns 0, or -2 if a kept node's parent was
// not kept (the kept set is not a connected tree).
// ---------------------------------------------------------------------------
int orc_flatten(int n_nodes, const int* token, const int* parent, const int* depth, const int* kept,
                int n, int ctx_len, int* flat_node, int* flat_token, int* flat_parent,
                int* flat_depth, int* position, unsigned char* mask) {
    const int T = n + 1;
    std::vector<int> where(n_nodes, -1);
    flat_node[0] = 0;
    where[0] = 0;
    for (int i = 0; i < n; ++i) {
        flat_node[i + 1] = kept[i];
        where[kept[i]] = i + 1;
    }
    for (int i = 0; i < T; ++i) {
        const int node = flat_node[i];
        flat_token[i] = token[node];
        flat_depth[i] = depth[node];
        position[i] = ctx_len + depth[node];
        const int p = parent[node];
        if (p < 0) {
            flat_parent[i] = -1;
        } else {
            if (where[p] < 0) return -2;
            flat_parent[i] = where[p];
        }
    }
    std::memset(mask, 0, (size_t)T * T);
    for (int i = 0; i < T; ++i) {
        for (int node = flat_node[i]; node >= 0; node = parent[node]) {
            if (where[node] < 0) return -2;
            mask[(size_t)i * T + where[node]] = 1;
        }
    }
    return 0;
}

// ---------------------------------------------------------------------------
// Tree attention, fp64 dense definition (EAGLE-2 page, mask passage: each tree
// token attends to the whole context and to its own ancestors only).
//
// For tree row i and query head h (KV head g = h / (Hq / Hkv)):
//   keys   = context rows [0, ctx) and tree rows ctx + j with mask[i][j] = 1
//   s_c    = scale * <q_i,h , k_c>
//   o      = sum_c softmax(s)_c v_c ,  lse = log sum_c exp(s_c)
// Inputs are the exact stored values (bf16 widened to fp32 by the caller).
//   q: [T][Hq][D]; k, v: element (g, row, d) at g*head_stride + (row0+row)*D + d.
// sel_i / sel_h: when n_sel >= 0, only those (i, h) pairs are computed and o is
// [n_sel][D], lse [n_sel]; when n_sel < 0 all pairs, o [T][Hq][D], lse [T][Hq].
// ---------------------------------------------------------------------------
int orc_attention(int T, int Hq, int Hkv, int D, int ctx_len, const float* q, const float* k,
                  const float* v, long long head_stride, long long row0, const unsigned char* mask,
                  double scale, int n_sel, const int* sel_i, const int* sel_h, double* o,
                  double* lse) {
    if (Hkv < 1 || Hq % Hkv != 0 || D < 1 || T < 1) return -1;
    const int group = Hq / Hkv;
    const int n_pairs = n_sel >= 0 ? n_sel : T * Hq;
    std::vector<long long> keys;
    std::vector<double> s;
    for (int p = 0; p < n_pairs; ++p) {
        const int i = n_sel >= 0 ? sel_i[p] : p / Hq;
        const int h = n_sel >= 0 ? sel_h[p] : p % Hq;
        if (i < 0 || i >= T || h < 0 || h >= Hq) return -1;
        const int g = h / group;
        keys.clear();
        for (int c = 0; c < ctx_len; ++c) keys.push_back(c);
        for (int j = 0; j < T; ++j)
            if (mask[(size_t)i * T + j]) keys.push_back((long long)ctx_len + j);
        const float* qi = q + ((size_t)i * Hq + h) * D;
        s.assign(keys.size(), 0.0);
        double smax = -INFINITY;
        for (size_t c = 0; c < keys.size(); ++c) {
            const float* kc = k + (size_t)g * head_stride + (size_t)(row0 + keys[c]) * D;
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += (double)qi[d] * (double)kc[d];
            s[c] = scale * dot;
            smax = std::max(smax, s[c]);
        }
        double denom = 0.0;
        for (size_t c = 0; c < keys.size(); ++c) denom += std::exp(s[c] - smax);
        double* out = o + (size_t)p * D;
        for (int d = 0; d < D; ++d) out[d] = 0.0;
        for (size_t c = 0; c < keys.size(); ++c) {
            const double w = std::exp(s[c] - smax) / denom;
            const float* vc = v + (size_t)g * head_stride + (size_t)(row0 + keys[c]) * D;
            for (int d = 0; d < D; ++d) out[d] += w * (double)vc[d];
        }
        lse[p] = smax + std::log(denom);
    }
    return 0;
}

// ---------------------------------------------------------------------------
// Greedy verification (CSDN page 1.2 / EAGLE page: lossless under greedy
// decoding).  Starting at the root row, the target's argmax (lowest id on
// ties) is accepted while the current row has a child carrying that token.
// The last argmax is the bonus token.  Children of a row are the rows whose
// flat parent it is.
// Outputs: accept_len, accept_path [max_depth] (flat rows, -1 padded),
// out_tokens [max_depth + 1] (accepted tokens then the bonus, -1 padded).
// ---------------------------------------------------------------------------
int orc_verify_greedy(int T, int V, const float* target, const int* flat_token,
                      const int* flat_parent, int max_depth, int* accept_len, int* accept_path,
                      int* out_tokens) {
    for (int i = 0; i < max_depth; ++i) accept_path[i] = -1;
    for (int i = 0; i <= max_depth; ++i) out_tokens[i] = -1;
    int cur = 0, len = 0;
    while (true) {
        const float* z = target + (size_t)cur * V;
        int best = 0;
        for (int t = 1; t < V; ++t) if (z[t] > z[best]) best = t;
        int next = -1;
        for (int j = 0; j < T; ++j)
            if (flat_parent[j] == cur && flat_token[j] == best) { next = j; break; }
        if (next < 0 || len >= max_depth) {
            out_tokens[len] = best;
            break;
        }
        accept_path[len] = next;
        out_tokens[len] = flat_token[next];
        ++len;
        cur = next;
    }
    *accept_len = len;
    return 0;
}

// ---------------------------------------------------------------------------
// Sampled verification with several candidates per row (CSDN page 1.1 and
// 1.2, EAGLE page: the output law must equal the target's).
//
// Reading: the children were picked deterministically, so each child proposes
// a point mass on its token.  At row cur, p = softmax(z / temperature) in
// fp64; children are tested in flat order; child c is accepted when
//     u < p(tok c) / sum_{t not removed} p(t)
// with u from Philox (slot = child index); a rejected child's token joins the
// removed set.  A child whose token is already removed (an earlier sibling of
// a caller-given static tree carried the same token) proposes a token of zero
// residual mass, so its ratio is 0 and it is never accepted; it still uses its
// slot.  When no child is accepted (or the row has none) the bonus token is
// drawn from p with removed tokens zeroed: the smallest t whose running sum
// exceeds u * (residual total), u from the bonus slot.
//
// trace [max_trace][4] receives (row, slot, u, ratio) per child test and
// (row, -1, u, margin) for the bonus draw, where margin is the distance of
// u * total to the nearest cumulative boundary, divided by the total.
// ---------------------------------------------------------------------------
int orc_verify_sampled(int T, int V, const float* target, const int* flat_token,
                       const int* flat_parent, int max_depth, float temperature, uint64_t seed,
                       uint64_t step, int seq, int* accept_len, int* accept_path, int* out_tokens,
                       double* trace, int max_trace, int* n_trace) {
    if (!(temperature > 0.0f)) return -1;
    for (int i = 0; i < max_depth; ++i) accept_path[i] = -1;
    for (int i = 0; i <= max_depth; ++i) out_tokens[i] = -1;
    const double temp = (double)temperature;
    std::vector<double> p(V);
    std::vector<char> removed(V);
    int cur = 0, len = 0, nt = 0;
    auto put = [&](double a, double b, double c, double d) {
        if (nt < max_trace) {
            trace[4 * nt + 0] = a; trace[4 * nt + 1] = b;
            trace[4 * nt + 2] = c; trace[4 * nt + 3] = d;
        }
        ++nt;
    };
    while (true) {
        const float* z = target + (size_t)cur * V;
        float zmax = z[0];
        for (int t = 1; t < V; ++t) if (z[t] > zmax) zmax = z[t];
        double total = 0.0;
        for (int t = 0; t < V; ++t) {
            p[t] = std::exp(((double)z[t] - (double)zmax) / temp);
            total += p[t];
        }
        for (int t = 0; t < V; ++t) p[t] /= total;
        std::fill(removed.begin(), removed.end(), 0);
        int accepted = -1, slot = 0;
        if (len < max_depth) {
            for (int j = 0; j < T; ++j) {
                if (flat_parent[j] != cur) continue;
                double rest = 0.0;
                for (int t = 0; t < V; ++t) if (!removed[t]) rest += p[t];
                const int tok = flat_token[j];
                const double ratio = removed[tok] ? 0.0 : p[tok] / rest;
                const double u = uniform_for(seed, step, (uint32_t)seq, (uint32_t)cur, (uint32_t)slot);
                put(cur, slot, u, ratio);
                ++slot;
                if (u < ratio) { accepted = j; break; }
                removed[tok] = 1;
            }
        }
        if (accepted >= 0) {
            accept_path[len] = accepted;
            out_tokens[len] = flat_token[accepted];
            ++len;
            cur = accepted;
            continue;
        }
        double rtotal = 0.0;
        for (int t = 0; t < V; ++t) if (!removed[t]) rtotal += p[t];
        const double u = uniform_for(seed, step, (uint32_t)seq, (uint32_t)cur, kBonusSlot);
        const double target_mass = u * rtotal;
        double run = 0.0, prev = 0.0;
        int pick = -1;
        for (int t = 0; t < V; ++t) {
            if (removed[t]) continue;
            prev = run;
            run += p[t];
            if (run > target_mass) { pick = t; break; }
        }
        if (pick < 0) {  // u * total at the very top after rounding: last live token
            for (int t = V - 1; t >= 0; --t) if (!removed[t] && p[t] > 0.0) { pick = t; break; }
            prev = run;
        }
        const double margin = std::min(target_mass - prev, run - target_mass) / rtotal;
        put(cur, -1, u, margin);
        out_tokens[len] = pick;
        break;
    }
    *accept_len = len;
    *n_trace = nt;
    return 0;
}

// ---------------------------------------------------------------------------
// Flatten a caller-given static tree (EAGLE-2 page, opening paragraphs: EAGLE and
// Medusa use a fixed draft-tree shape; the passage after the two stages: the
// flattened tree's ancestor-only mask and positions).  The tree arrives already
// flattened: parent[0] = -1 and 0 <= parent[i] < i for every other row, so row
// order is topological.  depth(i) = depth(parent(i)) + 1; position = ctx_len +
// depth; mask[i][j] = 1 iff row j lies on the root-to-row-i path (i included).
// Returns 0, or -1 if the parent array is not of that form.
// ---------------------------------------------------------------------------
int orc_flatten_static(int T, const int* parent, int ctx_len, int* flat_depth, int* position,
                       unsigned char* mask) {
    if (T < 1 || parent[0] != -1) return -1;
    for (int i = 1; i < T; ++i)
        if (parent[i] < 0 || parent[i] >= i) return -1;
    for (int i = 0; i < T; ++i) {
        int d = 0;
        for (int r = i; parent[r] >= 0; r = parent[r]) ++d;
        flat_depth[i] = d;
        position[i] = ctx_len + d;
    }
    std::memset(mask, 0, (size_t)T * T);
    for (int i = 0; i < T; ++i)
        for (int r = i; r >= 0; r = parent[r]) mask[(size_t)i * T + r] = 1;
    return 0;
}

// ---------------------------------------------------------------------------
// Rotary position encoding at the tree positions (EAGLE-2 page, passage after
// the two stages: the positions of the flattened tokens are adjusted so that
// each matches the position it would have in autoregressive decoding).  The
// encoding itself is the rotary one of the LLaMA family the workloads are shaped
// after, in its half-split form: for d < D/2, with theta = pos * base^(-2d/D),
// the pair (x[d], x[d + D/2]) is rotated by theta:
//   out[d]       = x[d] cos(theta) - x[d + D/2] sin(theta)
//   out[d + D/2] = x[d + D/2] cos(theta) + x[d] sin(theta)
// computed in fp64.  x: [rows][H][D], pos: [rows]; out: [rows][H][D] fp64.
// Returns 0, or -1 for an odd or non-positive D.
// ---------------------------------------------------------------------------
int orc_rope(int rows, int H, int D, const int* pos, double base, const float* x, double* out) {
    if (D < 2 || D % 2 != 0 || H < 1 || rows < 0) return -1;
    const int half = D / 2;
    for (int i = 0; i < rows; ++i) {
        for (int h = 0; h < H; ++h) {
            const float* xi = x + ((size_t)i * H + h) * D;
            double* oi = out + ((size_t)i * H + h) * D;
            for (int d = 0; d < half; ++d) {
                const double theta = (double)pos[i] * std::pow(base, -2.0 * d / D);
                const double c = std::cos(theta), s = std::sin(theta);
                const double a = xi[d], b = xi[d + half];
                oi[d] = a * c - b * s;
                oi[d + half] = b * c + a * s;
            }
        }
    }
    return 0;
}

// ---------------------------------------------------------------------------
// KV commit of the accepted path (EAGLE-2 page, passage after the two stages:
// the verified tokens must stand exactly as autoregressive decoding would have
// left them; CSDN page 1.1: the accepted draft tokens are emitted as output).
// One sequence, one cache (K or V): rows are row_bytes wide, head g's row r at
// byte offset (g * head_rows + row0 + r) * row_bytes.  The tree rows sit at
// ctx_len .. ctx_len + T - 1 in flattened order, row ctx_len being the root (the
// token emitted last step).  With accepted flattened rows path[0..a-1], the
// committed cache holds, at rows ctx_len + 1 + j, the rows that sat at
// ctx_len + path[j] -- all source rows are read before any is written.  Rows
// outside ctx_len + 1 .. ctx_len + a are left as they were.  The new context
// length (root and accepted rows kept; the bonus token is the next root) is
// returned through new_ctx.  Returns 0, or -1 if the path is not strictly
// increasing inside 1 .. T - 1 (a root path in flattened order always is).
// ---------------------------------------------------------------------------
int orc_kv_commit(int T, int ctx_len, int accept_len, const int* path, int n_heads,
                  long long head_rows, long long row0, long long row_bytes, unsigned char* cache,
                  int* new_ctx) {
    if (accept_len < 0 || accept_len > T - 1) return -1;
    for (int j = 0; j < accept_len; ++j) {
        if (path[j] < 1 || path[j] >= T) return -1;
        if (j > 0 && path[j] <= path[j - 1]) return -1;
    }
    std::vector<unsigned char> rows((size_t)accept_len * row_bytes);
    for (int g = 0; g < n_heads; ++g) {
        unsigned char* head = cache + (size_t)g * head_rows * row_bytes;
        for (int j = 0; j < accept_len; ++j)
            std::memcpy(&rows[(size_t)j * row_bytes],
                        head + (size_t)(row0 + ctx_len + path[j]) * row_bytes, row_bytes);
        for (int j = 0; j < accept_len; ++j)
            std::memcpy(head + (size_t)(row0 + ctx_len + 1 + j) * row_bytes,
                        &rows[(size_t)j * row_bytes], row_bytes);
    }
    *new_ctx = ctx_len + 1 + accept_len;
    return 0;
}

// ---------------------------------------------------------------------------
// Draft-side attention rows (EAGLE-2 page, two-stage passage: the m frontier
// nodes are fed to the draft model; EAGLE page: that model is one decoder layer
// which, like the target, must see each token's own history only).  The query
// of frontier node f attends to the context and to f's root path.  The rows
// used: U = the union of the frontier nodes' root paths, flattened in ascending
// node id (a topological order), padded to T_sub rows.  For row r < |U|:
// sub_node = its node id, sub_parent = its parent's row (-1 for the root),
// position = ctx_len + depth.  Padding rows: node -1, parent -1, position
// ctx_len, and they see only themselves.  mask[r][c] = 1 iff row c lies on the
// root-to-r path (r included).  query_row[j] = the row of frontier[j].
// Returns 0, or -1 if |U| > T_sub or a frontier id is not a node.
// ---------------------------------------------------------------------------
int orc_draft_subtree(int n_nodes, const int* parent, const int* depth, int n_frontier, const int* frontier,
                      int ctx_len, int T_sub, int* sub_node, int* sub_parent, int* position,
                      unsigned char* mask, int* query_row) {
    std::vector<char> in(n_nodes, 0);
    for (int j = 0; j < n_frontier; ++j) {
        if (frontier[j] < 0 || frontier[j] >= n_nodes) return -1;
        for (int x = frontier[j]; x >= 0; x = parent[x]) in[x] = 1;
    }
    std::vector<int> row_of(n_nodes, -1);
    int U = 0;
    for (int x = 0; x < n_nodes; ++x) {
        if (!in[x]) continue;
        if (U >= T_sub) return -1;
        row_of[x] = U;
        sub_node[U] = x;
        ++U;
    }
    std::memset(mask, 0, (size_t)T_sub * T_sub);
    for (int r = 0; r < T_sub; ++r) {
        if (r >= U) {
            sub_node[r] = -1;
            sub_parent[r] = -1;
            position[r] = ctx_len;
            mask[(size_t)r * T_sub + r] = 1;
            continue;
        }
        const int x = sub_node[r];
        sub_parent[r] = parent[x] >= 0 ? row_of[parent[x]] : -1;
        position[r] = ctx_len + depth[x];
        for (int y = x; y >= 0; y = parent[y]) mask[(size_t)r * T_sub + row_of[y]] = 1;
    }
    for (int j = 0; j < n_frontier; ++j) query_row[j] = row_of[frontier[j]];
    return 0;
}

}  // extern "C"
