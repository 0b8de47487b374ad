"""Pins for the CPU oracle: each check ties it to something other than itself.

Sources of truth used here:
  * the Philox4x32-10 authors' known-answer vectors (tests/golden);
  * numpy / scipy / torch library routines (lexsort, log_softmax, logsumexp,
    argmax, scaled_dot_product_attention) on the same inputs;
  * invariants the EAGLE-2 page states: confidences in [0, 1] so values never
    rise along a path; shallow-first ties keep the kept tree connected; each
    token sees only its ancestors (the It / is / a / has example); positions
    match plain autoregressive decoding;
  * the losslessness claim of the EAGLE page / CSDN page 1.2: the emitted
    tokens follow the target's own autoregressive law, computed here in
    closed form and matched by Monte-Carlo;
  * brute force over every root path on small trees.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Philox4x32-10 and the uniform convention
# ---------------------------------------------------------------------------
def test_philox_known_answer_vectors(orc):
    n = 0
    for line in open(os.path.join(GOLD, "philox4x32_10_kat.txt")):
        if line.startswith("#") or not line.strip():
            continue
        w = [int(x, 16) for x in line.split()]
        assert [int(x) for x in orc.philox4x32_10(w[0:4], w[4:6])] == w[6:10]
        n += 1
    assert n == 3


def test_uniform_counter_layout(orc):
    for seed, step, seq, row, slot in [(0, 0, 0, 0, 0), (2**40 + 17, 5, 3, 9, 2),
                                       (123456789, 2**33 + 4, 15, 60, 0xFFFFFFFF)]:
        w = orc.philox4x32_10([slot, row, seq, step & 0xFFFFFFFF], [seed & 0xFFFFFFFF, seed >> 32])
        assert orc.uniform(seed, step, seq, row, slot) == (int(w[0]) >> 8) / 2.0**24


def test_uniform_is_uniform(orc):
    us = np.array([orc.uniform(99, s, 0, 0, 0) for s in range(20000)])
    assert us.min() >= 0.0 and us.max() < 1.0
    counts, _ = np.histogram(us, bins=20, range=(0.0, 1.0))
    assert scipy.stats.chisquare(counts).pvalue > 1e-3


# ---------------------------------------------------------------------------
# Expand
# ---------------------------------------------------------------------------
def _topk_library(z, k):
    """top-k tokens by (logit desc, id asc) via numpy's lexsort."""
    order = np.lexsort((np.arange(len(z)), -z.astype(np.float64)))
    return order[:k]


def _check_expand(tree, z, depth, k, m, orc):
    """Re-derive the tree from the draft rows with library routines."""
    tok, par, dep, val = tree["token"], tree["parent"], tree["depth"], tree["value"]
    ids = np.arange(tree["n_nodes"])
    logsm = scipy.special.log_softmax(z.astype(np.float64), axis=1)
    fs, cap = orc.tree_shape(depth, k, m)
    assert tree["n_nodes"] == cap
    assert par[0] == -1 and dep[0] == 0 and val[0] == 0.0
    row = 0
    frontier = [0]
    exact = np.zeros(len(ids))  # fp64 path sums of log-confidences
    next_id = 1
    for layer in range(1, depth + 1):
        assert len(frontier) == fs[layer - 1]
        for j, f in enumerate(frontier):
            kids = ids[(par == f)]
            assert list(kids) == list(range(next_id, next_id + k)), "children numbered in creation order"
            next_id += k
            want = _topk_library(z[row], k)
            assert list(tok[kids]) == list(want)
            for c in kids:
                assert dep[c] == layer
                exact[c] = exact[f] + logsm[row, tok[c]]
            row += 1
        layer_ids = ids[dep == layer]
        order = np.lexsort((layer_ids, -val[layer_ids].astype(np.float64)))
        frontier = list(layer_ids[order][:min(m, len(layer_ids))])
    assert row == z.shape[0]
    # values equal the fp64 path sums of log-confidences up to fp32 rounding
    np.testing.assert_allclose(val.astype(np.float64), exact, rtol=4e-6, atol=4e-6 * depth)
    # confidences lie in [0, 1]: a child's value never exceeds its parent's
    for c in ids[1:]:
        assert val[c] <= val[par[c]]


@pytest.mark.parametrize("seed", range(40))
def test_expand_matches_library_rederivation(orc, seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(3, 17))
    depth = int(rng.integers(1, 5))
    k = int(rng.integers(1, min(3, V) + 1))
    m = int(rng.integers(1, 4))
    fs, cap = orc.tree_shape(depth, k, m)
    z = rng.normal(0, 2, (int(fs.sum()), V)).astype(np.float32)
    if seed % 3 == 0:
        z = np.round(z).astype(np.float32)  # many exact logit ties
    tree = orc.expand(z, int(rng.integers(0, V)), depth, k, m)
    _check_expand(tree, z, depth, k, m, orc)


def test_expand_full_vocab_rows(orc):
    rng = np.random.default_rng(5)
    z = rng.normal(0, 3, (51, 32000)).astype(np.float32)
    tree = orc.expand(z, 7, 6, 10, 10)
    _check_expand(tree, z, 6, 10, 10, orc)
    zz = z.astype(np.float64)
    want = scipy.special.logsumexp(zz - zz.max(axis=1, keepdims=True), axis=1)
    np.testing.assert_allclose(tree["row_lse64"], want, rtol=0, atol=1e-12)


def test_expand_single_layer_is_topk_of_one_row(orc):
    rng = np.random.default_rng(11)
    z = rng.normal(0, 3, (1, 1000)).astype(np.float32)
    tree = orc.expand(z, 0, 1, 10, 10)
    got = tree["token"][1:]
    want = torch.topk(torch.from_numpy(z[0]).double(), 10).indices.numpy()
    assert list(got) == list(want)
    kept = orc.rerank(tree["value"], tree["depth"], 10)
    assert list(kept) == list(range(1, 11))


# ---------------------------------------------------------------------------
# Rerank
# ---------------------------------------------------------------------------
def _check_rerank(tree, kept, n):
    val, dep, par = tree["value"], tree["depth"], tree["parent"]
    N = tree["n_nodes"]
    assert len(kept) == n and list(kept) == sorted(set(kept.tolist()))
    assert all(1 <= x < N for x in kept)
    keyf = lambda x: (-float(val[x]), int(dep[x]), int(x))
    dropped = [x for x in range(1, N) if x not in set(kept.tolist())]
    if n and dropped:
        assert max(keyf(x) for x in kept) < min(keyf(x) for x in dropped)
    ks = set(kept.tolist()) | {0}
    for x in kept:
        assert par[x] in ks, "kept tree must stay connected"


@pytest.mark.parametrize("seed", range(40))
def test_rerank_top_n_and_connected(orc, seed):
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(3, 17)); depth = int(rng.integers(1, 5))
    k = int(rng.integers(1, min(3, V) + 1)); m = int(rng.integers(1, 4))
    fs, cap = orc.tree_shape(depth, k, m)
    z = rng.normal(0, 2, (int(fs.sum()), V)).astype(np.float32)
    if seed % 2 == 0:
        z = np.round(z)
    tree = orc.expand(z, 0, depth, k, m)
    for n in sorted({0, 1, (cap - 1) // 2, cap - 1}):
        kept = orc.rerank(tree["value"], tree["depth"], n)
        _check_rerank(tree, kept, n)
    assert list(orc.rerank(tree["value"], tree["depth"], cap - 1)) == list(range(1, cap))
    with pytest.raises(ValueError):
        orc.rerank(tree["value"], tree["depth"], cap)


def test_rerank_equal_values_keep_shallow_node(orc):
    # A dominant logit makes the child's log-confidence vanish in fp32, so the
    # child's value equals its parent's exactly; the shallower node must win.
    V = 50
    z = np.full((2, V), -100.0, dtype=np.float32)
    z[0, 3] = 100.0; z[0, 4] = 0.0
    z[1, 8] = 100.0; z[1, 9] = 0.0
    tree = orc.expand(z, 1, 2, 2, 1)
    a, b = 1, 3  # layer-1 best child and its best child
    assert tree["parent"][b] == a and tree["value"][a] == tree["value"][b]
    kept = orc.rerank(tree["value"], tree["depth"], 1)
    assert list(kept) == [a]


# ---------------------------------------------------------------------------
# Flatten, mask, positions
# ---------------------------------------------------------------------------
def _closure_mask(flat_parent):
    """Reachability by repeated boolean products of the parent relation."""
    T = len(flat_parent)
    A = np.zeros((T, T), dtype=bool)
    for i, p in enumerate(flat_parent):
        if p >= 0:
            A[i, p] = True
    M = np.eye(T, dtype=bool)
    P = np.eye(T, dtype=bool)
    for _ in range(T):
        P = (P.astype(np.int64) @ A.astype(np.int64)) > 0
        M |= P
    return M


@pytest.mark.parametrize("seed", range(20))
def test_flatten_mask_is_ancestor_closure(orc, seed):
    rng = np.random.default_rng(200 + seed)
    V = 12; depth = int(rng.integers(1, 5)); k = int(rng.integers(1, 4)); m = int(rng.integers(1, 4))
    fs, cap = orc.tree_shape(depth, k, m)
    z = rng.normal(0, 2, (int(fs.sum()), V)).astype(np.float32)
    n = int(rng.integers(0, cap))
    ctx = int(rng.integers(0, 50))
    tree, kept, flat = orc.build_tree(z, 3, depth, k, m, n, ctx)
    assert list(flat["flat_node"]) == [0] + list(kept)
    fp = flat["flat_parent"]
    assert fp[0] == -1 and all(0 <= fp[i] < i for i in range(1, n + 1))
    assert (flat["mask"].astype(bool) == _closure_mask(fp)).all()
    np.testing.assert_array_equal(flat["position"], ctx + flat["flat_depth"])
    np.testing.assert_array_equal(flat["flat_token"], tree["token"][flat["flat_node"]])


def test_chain_tree_is_causal_decoding(orc):
    # top-1 expansion of one node per layer = a plain autoregressive draft
    d, V, ctx = 6, 20, 37
    z = np.random.default_rng(1).normal(0, 2, (d, V)).astype(np.float32)
    tree, kept, flat = orc.build_tree(z, 0, d, 1, 1, d, ctx)
    T = d + 1
    assert (flat["mask"].astype(bool) == np.tril(np.ones((T, T), dtype=bool))).all()
    np.testing.assert_array_equal(flat["position"], ctx + np.arange(T))


def test_it_is_a_has_example(orc):
    fx = json.load(open(os.path.join(GOLD, "it_is_a_has.json")))
    vocab = {"It": 0, "is": 1, "a": 2, "has": 3}
    name = {v: k for k, v in vocab.items()}
    # draft rows: root prefers "is" then "has"; "is" prefers "a"
    z = np.full((2, 4), -5.0, dtype=np.float32)
    z[0, vocab["is"]] = 3.0; z[0, vocab["has"]] = 2.0
    z[1, vocab["a"]] = 4.0; z[1, vocab["has"]] = 1.0
    tree, kept, flat = orc.build_tree(z, vocab["It"], 2, 2, 1, 3, 0)
    rows = {name[int(t)]: i for i, t in enumerate(flat["flat_token"])}
    assert set(rows) == set(fx["tree"])
    for child, parent in fx["tree"].items():
        pi = flat["flat_parent"][rows[child]]
        assert (parent is None and pi == -1) or (parent is not None and pi == rows[parent])
    mask = flat["mask"].astype(bool)
    for tok, spec in fx["page_fixes"].items():
        for s in spec["sees"]:
            assert mask[rows[tok], rows[s]]
        for s in spec["never"]:
            assert not mask[rows[tok], rows[s]]
    assert {name[int(flat["flat_token"][j])] for j in np.nonzero(mask[rows["a"]])[0]} == {"It", "is", "a"}


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def _sdpa_reference(q, k, v, mask, ctx):
    """torch's scaled_dot_product_attention in fp64 with the tree key mask."""
    T, Hq, D = q.shape
    Hkv = k.shape[0]
    g = Hq // Hkv
    kk = torch.from_numpy(k.astype(np.float64)).repeat_interleave(g, dim=0)
    vv = torch.from_numpy(v.astype(np.float64)).repeat_interleave(g, dim=0)
    qq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)
    full = np.concatenate([np.ones((T, ctx), dtype=bool), mask.astype(bool)], axis=1)
    am = torch.from_numpy(full)[None].expand(Hq, T, ctx + T)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=am)
    s = (qq @ kk.transpose(1, 2)) / math.sqrt(D)
    s = s.masked_fill(~am, -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


@pytest.mark.parametrize("Hq,Hkv,D,ctx,seed", [(4, 4, 64, 50, 0), (8, 2, 32, 17, 1), (6, 1, 16, 0, 2),
                                               (4, 4, 128, 300, 3)])
def test_attention_matches_library_sdpa(orc, Hq, Hkv, D, ctx, seed):
    rng = np.random.default_rng(300 + seed)
    depth, k, m, n = 3, 3, 2, 9
    fs, cap = orc.tree_shape(depth, k, m)
    z = rng.normal(0, 2, (int(fs.sum()), 40)).astype(np.float32)
    tree, kept, flat = orc.build_tree(z, 0, depth, k, m, n, ctx)
    T = n + 1
    q = rng.normal(size=(T, Hq, D)).astype(np.float32)
    kc = rng.normal(size=(Hkv, ctx + T, D)).astype(np.float32)
    vc = rng.normal(size=(Hkv, ctx + T, D)).astype(np.float32)
    o, lse = orc.attention(q, kc, vc, flat["mask"], ctx)
    ro, rl = _sdpa_reference(q, kc, vc, flat["mask"], ctx)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)
    sel = [(int(i), int(h)) for i, h in zip(rng.integers(0, T, 7), rng.integers(0, Hq, 7))]
    so, sl = orc.attention(q, kc, vc, flat["mask"], ctx, sel=sel)
    for j, (i, h) in enumerate(sel):
        np.testing.assert_array_equal(so[j], o[i, h])
        assert sl[j] == lse[i, h]


def test_attention_row_offset_in_packed_cache(orc):
    rng = np.random.default_rng(9)
    T, Hq, D, ctx, row0 = 4, 2, 16, 10, 23
    mask = np.tril(np.ones((T, T), dtype=np.uint8))
    q = rng.normal(size=(T, Hq, D)).astype(np.float32)
    big_k = rng.normal(size=(Hq, row0 + ctx + T + 5, D)).astype(np.float32)
    big_v = rng.normal(size=(Hq, row0 + ctx + T + 5, D)).astype(np.float32)
    o1, l1 = orc.attention(q, big_k, big_v, mask, ctx, row0=row0)
    o2, l2 = orc.attention(q, big_k[:, row0:row0 + ctx + T].copy(), big_v[:, row0:row0 + ctx + T].copy(),
                           mask, ctx)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_chain_tree_attention_equals_single_query_decodes(orc):
    rng = np.random.default_rng(4)
    T, H, D, ctx = 5, 3, 32, 40
    mask = np.tril(np.ones((T, T), dtype=np.uint8))
    q = rng.normal(size=(T, H, D)).astype(np.float32)
    kc = rng.normal(size=(H, ctx + T, D)).astype(np.float32)
    vc = rng.normal(size=(H, ctx + T, D)).astype(np.float32)
    o, _ = orc.attention(q, kc, vc, mask, ctx)
    for i in range(T):
        for h in range(H):
            s = kc[h, : ctx + i + 1].astype(np.float64) @ q[i, h].astype(np.float64) / math.sqrt(D)
            w = scipy.special.softmax(s)
            np.testing.assert_allclose(o[i, h], w @ vc[h, : ctx + i + 1].astype(np.float64), atol=1e-12)


def test_branch_independence(orc):
    # Perturbing the K/V of a row that is not an ancestor of row i leaves row i
    # bit-identical (each token is unaffected by other branches).
    rng = np.random.default_rng(6)
    depth, k, m, n, ctx = 3, 3, 2, 10, 20
    fs, cap = orc.tree_shape(depth, k, m)
    z = rng.normal(0, 2, (int(fs.sum()), 30)).astype(np.float32)
    tree, kept, flat = orc.build_tree(z, 0, depth, k, m, n, ctx)
    T, H, D = n + 1, 2, 16
    q = rng.normal(size=(T, H, D)).astype(np.float32)
    kc = rng.normal(size=(H, ctx + T, D)).astype(np.float32)
    vc = rng.normal(size=(H, ctx + T, D)).astype(np.float32)
    o, _ = orc.attention(q, kc, vc, flat["mask"], ctx)
    mask = flat["mask"].astype(bool)
    for j in range(T):
        k2, v2 = kc.copy(), vc.copy()
        k2[:, ctx + j] += 3.0; v2[:, ctx + j] -= 2.0
        o2, _ = orc.attention(q, k2, v2, flat["mask"], ctx)
        for i in range(T):
            if not mask[i, j]:
                np.testing.assert_array_equal(o2[i], o[i])
            else:
                assert not np.array_equal(o2[i], o[i])


# ---------------------------------------------------------------------------
# Greedy verification
# ---------------------------------------------------------------------------
def _paths(flat_parent):
    """Every root path as a list of flat rows (root excluded)."""
    T = len(flat_parent)
    out = []
    for i in range(T):
        p, j = [], i
        while j > 0:
            p.append(j); j = flat_parent[j]
        out.append(p[::-1])
    return out


def _greedy_brute(target, flat_token, flat_parent):
    best = []
    for path in _paths(flat_parent):
        ok, prev = True, 0
        for r in path:
            if flat_token[r] != int(np.argmax(target[prev])):
                ok = False; break
            prev = r
        if ok and len(path) > len(best):
            best = path
    last = best[-1] if best else 0
    return best, int(np.argmax(target[last]))


@pytest.mark.parametrize("seed", range(30))
def test_greedy_matches_brute_force(orc, seed):
    rng = np.random.default_rng(400 + seed)
    V = int(rng.integers(3, 9)); depth = int(rng.integers(1, 5))
    k = int(rng.integers(1, min(3, V) + 1)); m = int(rng.integers(1, 4))
    fs, cap = orc.tree_shape(depth, k, m)
    z = rng.normal(0, 2, (int(fs.sum()), V)).astype(np.float32)
    n = int(rng.integers(0, cap))
    tree, kept, flat = orc.build_tree(z, 0, depth, k, m, n, 0)
    T = n + 1
    target = rng.normal(0, 1, (T, V)).astype(np.float32)
    if seed % 2:
        target = np.round(target)  # argmax ties
    # plant some argmax matches so paths are accepted
    for i in range(1, T):
        if rng.random() < 0.6:
            target[flat["flat_parent"][i], flat["flat_token"][i]] = 10.0 + rng.random()
    al, ap, ot = orc.verify_greedy(target, flat["flat_token"], flat["flat_parent"], depth)
    path, bonus = _greedy_brute(target, flat["flat_token"], flat["flat_parent"])
    assert al == len(path)
    assert list(ap[:al]) == path and all(x == -1 for x in ap[al:])
    assert list(ot[:al]) == [int(flat["flat_token"][r]) for r in path]
    assert ot[al] == bonus and all(x == -1 for x in ot[al + 1:])


def test_greedy_planted_chain_length(orc):
    d, V = 6, 30
    z = np.random.default_rng(2).normal(0, 2, (d, V)).astype(np.float32)
    tree, kept, flat = orc.build_tree(z, 0, d, 1, 1, d, 5)
    for j in range(d + 1):
        target = np.zeros((d + 1, V), dtype=np.float32)
        target[:, V - 1] = 1.0  # a token never drafted in this chain, unless it is
        for i in range(j):
            target[i, flat["flat_token"][i + 1]] = 5.0
        if j < d and flat["flat_token"][j + 1] == V - 1:
            target[j, V - 2] = 2.0
        al, ap, ot = orc.verify_greedy(target, flat["flat_token"], flat["flat_parent"], d)
        assert al == j
        assert list(ap[:j]) == list(range(1, j + 1))


# ---------------------------------------------------------------------------
# Sampled verification: the emitted tokens must follow the target's own
# autoregressive law (losslessness), computed here in closed form.
# ---------------------------------------------------------------------------
def _ar_law(target, flat_token, flat_parent, temperature):
    """P(emitted sequence) for autoregressive sampling from the target rows,
    walking the tree while the sampled token is a child and stopping with the
    first token outside it (that token is the bonus)."""
    T, V = target.shape
    P = scipy.special.softmax(target.astype(np.float64) / temperature, axis=1)
    law = {}

    def walk(row, prefix, prob):
        # a token carried by several siblings (possible in a caller-given static
        # tree) leads into the first of them in flattened order
        kids = {}
        for j in range(T):
            if flat_parent[j] == row:
                kids.setdefault(int(flat_token[j]), j)
        for t in range(V):
            pt = prob * P[row, t]
            if pt == 0.0:
                continue
            if t in kids:
                walk(kids[t], prefix + (t,), pt)
            else:
                law[prefix + (t,)] = law.get(prefix + (t,), 0.0) + pt

    walk(0, (), 1.0)
    return law


def _rule_law(target, flat_token, flat_parent, temperature):
    """Exact law of the multi-candidate accept/reject rule, by enumerating its
    branches (accept child i with p(tok)/residual mass, else remove the token),
    used to show the rule reading is lossless independent of any code path."""
    T, V = target.shape
    P = scipy.special.softmax(target.astype(np.float64) / temperature, axis=1)
    law = {}

    def visit(row, prefix, prob):
        p = P[row].copy()
        kids = [j for j in range(T) if flat_parent[j] == row]
        for j in kids:
            tok = int(flat_token[j])
            acc = p[tok] / p.sum() if p[tok] > 0.0 else 0.0
            if acc > 0.0:  # a token already removed at this row has no mass left
                visit(j, prefix + (tok,), prob * acc)
            prob *= (1.0 - acc)
            p[tok] = 0.0
        if p.sum() == 0.0:  # every token was a child and all were tested: no residual
            return
        r = p / p.sum()
        for t in range(V):
            if r[t] > 0:
                law[prefix + (t,)] = law.get(prefix + (t,), 0.0) + prob * r[t]

    visit(0, (), 1.0)
    return law


def _small_tree(orc, seed, V=6, depth=3, k=2, m=2, n=None):
    rng = np.random.default_rng(seed)
    fs, cap = orc.tree_shape(depth, k, m)
    z = rng.normal(0, 2, (int(fs.sum()), V)).astype(np.float32)
    n = cap - 1 if n is None else n
    tree, kept, flat = orc.build_tree(z, 0, depth, k, m, n, 0)
    return rng, flat


@pytest.mark.parametrize("seed,temp", [(0, 1.0), (1, 0.7), (2, 1.0), (3, 2.0)])
def test_acceptance_rule_is_lossless_closed_form(orc, seed, temp):
    rng, flat = _small_tree(orc, 500 + seed)
    T = len(flat["flat_token"])
    target = rng.normal(0, 1.5, (T, 6)).astype(np.float32)
    a = _ar_law(target, flat["flat_token"], flat["flat_parent"], temp)
    b = _rule_law(target, flat["flat_token"], flat["flat_parent"], temp)
    assert set(a) == set(b)
    for key in a:
        assert abs(a[key] - b[key]) < 1e-12


def _mc_counts(orc, target, flat, depth, temp, n, seed):
    counts = {}
    for s in range(n):
        al, ap, ot, _ = orc.verify_sampled(target, flat["flat_token"], flat["flat_parent"], depth, temp,
                                           seed, s, 0)
        key = tuple(int(x) for x in ot[: al + 1])
        counts[key] = counts.get(key, 0) + 1
    return counts


def _chi2_pvalue(counts, law, n):
    keys = sorted(law, key=lambda k: -law[k])
    obs, exp = [], []
    other_o, other_e = 0, 0.0
    for k in keys:
        e = law[k] * n
        if e >= 5:
            obs.append(counts.get(k, 0)); exp.append(e)
        else:
            other_o += counts.get(k, 0); other_e += e
    assert sum(counts.get(k, 0) for k in counts if k not in law) == 0, "emitted an impossible sequence"
    if other_e > 0:
        obs.append(other_o); exp.append(other_e)
    exp = np.array(exp) * (n / sum(exp))
    return scipy.stats.chisquare(np.array(obs), exp).pvalue


@pytest.mark.parametrize("seed,temp", [(0, 1.0), (1, 0.7)])
def test_oracle_sampling_follows_target_law_monte_carlo(orc, seed, temp):
    rng, flat = _small_tree(orc, 600 + seed, V=5, depth=3, k=2, m=2)
    T = len(flat["flat_token"])
    target = rng.normal(0, 1.0, (T, 5)).astype(np.float32)
    for i in range(1, T):  # make acceptances common
        if rng.random() < 0.5:
            target[flat["flat_parent"][i], flat["flat_token"][i]] += 1.5
    law = _ar_law(target, flat["flat_token"], flat["flat_parent"], temp)
    n = 40000
    counts = _mc_counts(orc, target, flat, 3, temp, n, seed=12345 + seed)
    assert _chi2_pvalue(counts, law, n) > 1e-3


def test_oracle_sampling_without_children_is_categorical(orc):
    rng = np.random.default_rng(7)
    target = rng.normal(0, 1.0, (1, 6)).astype(np.float32)
    ft = np.array([3], np.int32); fp = np.array([-1], np.int32)
    n = 30000
    counts = np.zeros(6)
    for s in range(n):
        al, ap, ot, tr = orc.verify_sampled(target, ft, fp, 2, 1.0, 77, s, 0)
        assert al == 0 and len(tr) == 1 and tr[0][1] == -1
        counts[ot[0]] += 1
    p = scipy.special.softmax(target[0].astype(np.float64))
    assert scipy.stats.chisquare(counts, p * n).pvalue > 1e-3


def test_sampled_trace_decisions_are_strict(orc):
    rng, flat = _small_tree(orc, 700, V=6, depth=3, k=2, m=2)
    T = len(flat["flat_token"])
    target = rng.normal(0, 1.0, (T, 6)).astype(np.float32)
    for s in range(200):
        al, ap, ot, tr = orc.verify_sampled(target, flat["flat_token"], flat["flat_parent"], 3, 1.0, 5, s, 0)
        accepted = 0
        for row, slot, u, ratio in tr:
            if slot >= 0:
                assert u == orc.uniform(5, s, 0, int(row), int(slot))
                accepted += int(u < ratio)
        assert accepted == al


# ---------------------------------------------------------------------------
# Sampled verification on caller-given static trees (EAGLE-2 page, opening
# paragraphs: EAGLE and Medusa draft over a fixed tree), where a row may have up
# to T - 1 children and siblings may carry the same token.  The rule must stay
# lossless (EAGLE page abstract; CSDN page 1.2): a token already rejected at a
# row has no residual mass left, so a later sibling carrying it is never
# accepted.
# ---------------------------------------------------------------------------
def _static_trees():
    """(name, flat_parent, flat_token, V, depth) of static trees with wide rows and
    duplicate sibling tokens."""
    out = []
    # duplicate siblings at the root (rows 1, 2) and below row 1 (rows 4, 5); row 2's
    # subtree can never be entered
    out.append(("dup", np.array([-1, 0, 0, 0, 1, 1, 2, 3, 4], np.int32),
                np.array([0, 2, 2, 4, 1, 1, 3, 2, 0], np.int32), 6, 4))
    # a 63-child star with distinct tokens
    out.append(("star63", np.array([-1] + [0] * 63, np.int32),
                np.array([0] + list(range(5, 68)), np.int32), 72, 1))
    # a 63-child star whose children carry only 12 distinct tokens
    rng = np.random.default_rng(31)
    out.append(("star63dup", np.array([-1] + [0] * 63, np.int32),
                np.concatenate([[0], rng.integers(0, 12, 63)]).astype(np.int32), 16, 1))
    # a wide random tree over a small vocabulary (many duplicates at every row)
    par = [-1]
    for i in range(1, 40):
        par.append(0 if rng.random() < 0.4 else int(rng.integers(0, i)))
    out.append(("wide40", np.array(par, np.int32), rng.integers(0, 7, 40).astype(np.int32), 7, 0))
    # depth argument = the tree's own depth, so the walk is never cut short
    res = []
    for name, fp, ft, V, _ in out:
        d = [0] * len(fp)
        for i in range(1, len(fp)):
            d[i] = d[fp[i]] + 1
        res.append((name, fp, ft, V, max(d)))
    return res


def _static_target(flat_token, flat_parent, V, seed, boost=1.5):
    rng = np.random.default_rng(seed)
    T = len(flat_token)
    target = rng.normal(0, 1.0, (T, V)).astype(np.float32)
    for i in range(1, T):  # make acceptances common
        if rng.random() < 0.5:
            target[flat_parent[i], flat_token[i]] += boost
    return target


@pytest.mark.parametrize("idx", [0, 1, 2, 3])
@pytest.mark.parametrize("temp", [1.0, 0.7])
def test_acceptance_rule_is_lossless_on_static_trees_closed_form(idx, temp):
    """Exact enumeration: the accept/reject rule with removed tokens at zero mass
    has the target's autoregressive law on trees with duplicate sibling tokens."""
    name, fp, ft, V, depth = _static_trees()[idx]
    target = _static_target(ft, fp, V, 40 + idx)
    a = _ar_law(target, ft, fp, temp)
    b = _rule_law(target, ft, fp, temp)
    assert set(a) == set(b)
    for key in a:
        assert abs(a[key] - b[key]) < 1e-12


def test_oracle_duplicate_sibling_never_accepted(orc):
    """Every test of a sibling whose token an earlier sibling already carried has
    ratio exactly 0, and such a row is never on an accepted path."""
    for name, fp, ft, V, depth in _static_trees():
        target = _static_target(ft, fp, V, 7)
        T = len(ft)
        dup = np.zeros(T, bool)
        for j in range(1, T):
            dup[j] = any(fp[i] == fp[j] and ft[i] == ft[j] for i in range(1, j))
        assert dup.any() or name == "star63"
        for s in range(300):
            al, ap, ot, tr = orc.verify_sampled(target, ft, fp, depth, 1.0, 9, s, 0)
            assert not any(dup[r] for r in ap[:al])
            for row, slot, u, ratio in tr:
                if slot < 0:
                    continue
                kids = [j for j in range(T) if fp[j] == int(row)]
                j = kids[int(slot)]
                if dup[j]:
                    assert ratio == 0.0
                else:
                    assert ratio > 0.0


def _mc_counts_lean(orc, target, ft, fp, depth, temp, n, seed):
    """Emitted-sequence counts of n oracle draws (steps 0..n-1), calling the
    oracle's C entry with preallocated buffers."""
    import ctypes as C
    L = orc.lib()
    z = np.ascontiguousarray(target, np.float32); T, V = z.shape
    ft = np.ascontiguousarray(ft, np.int32); fp = np.ascontiguousarray(fp, np.int32)
    al = np.zeros(1, np.int32); ap = np.zeros(depth, np.int32); ot = np.zeros(depth + 1, np.int32)
    tr = np.zeros((1, 4)); nt = np.zeros(1, np.int32)
    ptr = lambda a: a.ctypes.data_as(C.c_void_p)
    pz, pft, pfp, pal, pap, pot, ptr_, pnt = map(ptr, (z, ft, fp, al, ap, ot, tr, nt))
    counts = {}
    f = L.orc_verify_sampled
    for s in range(n):
        rc = f(T, V, pz, pft, pfp, depth, float(temp), seed, s, 0, pal, pap, pot, ptr_, 1, pnt)
        assert rc == 0
        key = tuple(int(x) for x in ot[: al[0] + 1])
        counts[key] = counts.get(key, 0) + 1
    return counts


@pytest.mark.slow
@pytest.mark.parametrize("idx,temp", [(0, 1.0), (1, 1.0), (2, 0.7), (3, 1.0)])
def test_oracle_sampling_static_trees_monte_carlo_1e6(orc, idx, temp):
    """10^6 oracle draws on static trees with wide rows and duplicate siblings
    follow the target's autoregressive law (chi-square)."""
    name, fp, ft, V, depth = _static_trees()[idx]
    target = _static_target(ft, fp, V, 70 + idx)
    law = _ar_law(target, ft, fp, temp)
    n = 1_000_000
    counts = _mc_counts_lean(orc, target, ft, fp, depth, temp, n, seed=4242 + idx)
    assert _chi2_pvalue(counts, law, n) > 1e-3


@pytest.mark.slow
@pytest.mark.parametrize("seed,temp", [(0, 1.0), (1, 0.7)])
def test_oracle_sampling_follows_target_law_monte_carlo_1e6(orc, seed, temp):
    """The dynamic-tree Monte-Carlo pin at 10^6 draws."""
    rng, flat = _small_tree(orc, 600 + seed, V=5, depth=3, k=2, m=2)
    T = len(flat["flat_token"])
    target = rng.normal(0, 1.0, (T, 5)).astype(np.float32)
    for i in range(1, T):
        if rng.random() < 0.5:
            target[flat["flat_parent"][i], flat["flat_token"][i]] += 1.5
    law = _ar_law(target, flat["flat_token"], flat["flat_parent"], temp)
    n = 1_000_000
    counts = _mc_counts_lean(orc, target, flat["flat_token"], flat["flat_parent"], 3, temp, n, seed=99 + seed)
    assert _chi2_pvalue(counts, law, n) > 1e-3


def test_oracle_greedy_static_trees_brute_force(orc):
    """Greedy on static trees (wide rows, duplicate siblings): the accepted path is
    the longest root path whose every token is its parent row's argmax, taking the
    first sibling in flattened order where several carry it."""
    for name, fp, ft, V, depth in _static_trees():
        for seed in range(5):
            target = _static_target(ft, fp, V, 300 + seed, boost=4.0)
            T = len(ft)
            # brute force: every root path, its greedy-consistent prefix
            best_path = []
            cur, path = 0, []
            while len(path) < depth:
                am = int(np.argmax(target[cur]))
                kids = [j for j in range(T) if fp[j] == cur and ft[j] == am]
                if not kids:
                    break
                cur = min(kids)
                path.append(cur)
            al, ap, ot = orc.verify_greedy(target, ft, fp, depth)
            assert al == len(path) and list(ap[:al]) == path
            assert ot[al] == int(np.argmax(target[path[-1] if path else 0]))
