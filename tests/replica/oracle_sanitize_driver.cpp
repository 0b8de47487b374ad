// Memory and undefined-behaviour check of the CPU oracle: every oracle entry
// point run on seeded small inputs, each buffer allocated at exactly the size the
// entry point's contract gives, compiled with -fsanitize=address,undefined by
// tests/test_oracle_sanitize.py.  A read or write past a buffer, a signed overflow
// or a bad shift aborts the program with the sanitizer's report; return codes are
// checked against the contract (0 for valid arguments, -1 where it says so).
// Prints "ok" and exits 0 otherwise.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../oracle/eagle_oracle.cpp"

namespace {

std::mt19937_64 rng(20240607);

int fail(const char* what, int line) {
    std::fprintf(stderr, "unexpected result: %s (line %d)\n", what, line);
    std::exit(2);
}
#define EXPECT(c) ((c) ? 0 : fail(#c, __LINE__))

float normal(float sigma) {
    std::normal_distribution<float> d(0.0f, sigma);
    return d(rng);
}

// One tree step: expand, rerank, flatten, attention, verify, rope, commit, subtree.
void tree_case(int V, int depth, int topk, int m, int n, int ctx, int Hq, int Hkv, int D, bool ties) {
    std::vector<int> fs(depth);
    int cap = 0;
    EXPECT(orc_tree_shape(depth, topk, m, fs.data(), &cap) == 0);
    int R = 0;
    for (int f : fs) R += f;
    std::vector<float> z((size_t)R * V);
    for (float& x : z) x = ties ? (float)(int)(normal(2.0f) * 2.0f) : normal(2.0f);
    std::vector<int> tok(cap), par(cap), dep(cap), haz(R);
    std::vector<float> val(cap);
    std::vector<double> lse(R);
    int nn = 0;
    EXPECT(orc_expand(V, depth, topk, m, z.data(), 3 % V, tok.data(), par.data(), dep.data(), val.data(),
                      lse.data(), haz.data(), &nn) == 0);
    EXPECT(nn == cap);
    if (n > nn - 1) n = nn - 1;
    std::vector<int> kept(n > 0 ? n : 1);
    EXPECT(orc_rerank(nn, val.data(), dep.data(), n, kept.data()) == 0);
    EXPECT(orc_rerank(nn, val.data(), dep.data(), nn, kept.data()) == -1);  // n past the candidates
    const int T = n + 1;
    std::vector<int> fnode(T), ftok(T), fpar(T), fdep(T), pos(T);
    std::vector<unsigned char> mask((size_t)T * T);
    EXPECT(orc_flatten(nn, tok.data(), par.data(), dep.data(), kept.data(), n, ctx, fnode.data(), ftok.data(),
                       fpar.data(), fdep.data(), pos.data(), mask.data()) == 0);
    // attention: full, and on selected (row, head) pairs
    const long long rows = ctx + T;
    std::vector<float> q((size_t)T * Hq * D), k((size_t)Hkv * rows * D), v((size_t)Hkv * rows * D);
    for (float& x : q) x = normal(1.0f);
    for (float& x : k) x = normal(1.0f);
    for (float& x : v) x = normal(1.0f);
    std::vector<double> o((size_t)T * Hq * D), ol((size_t)T * Hq);
    int si[1] = {0}, sh[1] = {0};
    EXPECT(orc_attention(T, Hq, Hkv, D, ctx, q.data(), k.data(), v.data(), rows * D, 0, mask.data(),
                         0.125, -1, si, sh, o.data(), ol.data()) == 0);
    int seli[3] = {0, T - 1, T / 2}, selh[3] = {0, Hq - 1, Hq / 2};
    std::vector<double> os((size_t)3 * D), osl(3);
    EXPECT(orc_attention(T, Hq, Hkv, D, ctx, q.data(), k.data(), v.data(), rows * D, 0, mask.data(), 0.125, 3,
                         seli, selh, os.data(), osl.data()) == 0);
    // verify over target logits of the flattened rows
    std::vector<float> tgt((size_t)T * V);
    for (float& x : tgt) x = ties ? (float)(int)(normal(2.0f) * 2.0f) : normal(2.0f);
    int al = -1;
    std::vector<int> ap(depth), ot(depth + 1);
    EXPECT(orc_verify_greedy(T, V, tgt.data(), ftok.data(), fpar.data(), depth, &al, ap.data(), ot.data()) == 0);
    const int max_trace = 64;
    std::vector<double> trace((size_t)max_trace * 4);
    int ntr = 0;
    for (int s = 0; s < 4; ++s)
        EXPECT(orc_verify_sampled(T, V, tgt.data(), ftok.data(), fpar.data(), depth, 0.8f, 99, s, 1, &al,
                                  ap.data(), ot.data(), trace.data(), max_trace, &ntr) == 0);
    EXPECT(orc_verify_sampled(T, V, tgt.data(), ftok.data(), fpar.data(), depth, 0.0f, 99, 0, 1, &al, ap.data(),
                              ot.data(), trace.data(), max_trace, &ntr) == -1);
    // rotary of the q rows at the tree positions
    std::vector<double> rot((size_t)T * Hq * D);
    EXPECT(orc_rope(T, Hq, D, pos.data(), 10000.0, q.data(), rot.data()) == 0);
    // KV commit of the greedy path into a byte cache of Hkv heads
    const long long row_bytes = D * 2;
    std::vector<unsigned char> cache((size_t)Hkv * rows * row_bytes);
    for (auto& c : cache) c = (unsigned char)rng();
    int new_ctx = 0;
    std::vector<int> path(al > 0 ? al : 1);
    for (int j = 0; j < al; ++j) path[j] = ap[j];
    EXPECT(orc_kv_commit(T, ctx, al, path.data(), Hkv, rows, 0, row_bytes, cache.data(), &new_ctx) == 0);
    EXPECT(new_ctx == ctx + 1 + al);  // the root row and the accepted rows join the context
    // draft subtree of the deepest layer's first min(m, F) nodes
    std::vector<int> frontier;
    for (int id = 0; id < nn && (int)frontier.size() < m; ++id)
        if (dep[id] == depth) frontier.push_back(id);
    const int nf = (int)frontier.size();
    const int T_sub = 1 + nf * depth;
    std::vector<int> sn(T_sub), sp(T_sub), spos(T_sub), qrow(nf > 0 ? nf : 1);
    std::vector<unsigned char> smask((size_t)T_sub * T_sub);
    EXPECT(orc_draft_subtree(nn, par.data(), dep.data(), nf, frontier.data(), ctx, T_sub, sn.data(), sp.data(),
                             spos.data(), smask.data(), qrow.data()) == 0);
}

void static_case(int T, int V) {
    std::vector<int> par(T), tok(T);
    par[0] = -1;
    for (int i = 1; i < T; ++i) par[i] = (int)(rng() % (unsigned)i);
    for (int i = 0; i < T; ++i) tok[i] = (int)(rng() % (unsigned)V);  // duplicate siblings likely
    std::vector<int> dep(T), pos(T);
    std::vector<unsigned char> mask((size_t)T * T);
    EXPECT(orc_flatten_static(T, par.data(), 7, dep.data(), pos.data(), mask.data()) == 0);
    int depth = 0;
    for (int d : dep) depth = d > depth ? d : depth;
    if (depth < 1) depth = 1;
    std::vector<float> tgt((size_t)T * V);
    for (float& x : tgt) x = normal(2.0f);
    int al = -1;
    std::vector<int> ap(depth), ot(depth + 1);
    EXPECT(orc_verify_greedy(T, V, tgt.data(), tok.data(), par.data(), depth, &al, ap.data(), ot.data()) == 0);
    std::vector<double> trace(4 * 256);
    int ntr = 0;
    EXPECT(orc_verify_sampled(T, V, tgt.data(), tok.data(), par.data(), depth, 1.0f, 5, 2, 0, &al, ap.data(),
                              ot.data(), trace.data(), 256, &ntr) == 0);
    std::vector<int> bad = par;
    if (T > 2) {
        bad[T - 1] = T - 1;  // a row that is its own parent
        EXPECT(orc_flatten_static(T, bad.data(), 7, dep.data(), pos.data(), mask.data()) == -1);
    }
}

}  // namespace

int main() {
    tree_case(300, 4, 4, 4, 25, 37, 8, 2, 16, false);
    tree_case(300, 4, 4, 4, 25, 0, 4, 4, 8, true);      // empty context, many equal logits
    tree_case(2000, 2, 32, 32, 63, 130, 4, 1, 16, false);  // the widest tree (T = 64)
    tree_case(64, 6, 10, 10, 60, 5, 8, 8, 8, true);
    tree_case(17, 1, 1, 1, 1, 3, 2, 1, 4, false);       // the smallest tree
    for (int T : {1, 2, 9, 33, 64}) static_case(T, 12);
    std::printf("ok\n");
    return 0;
}
