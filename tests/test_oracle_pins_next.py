"""Pins for the oracle's static-tree flattening, rotary at tree positions, KV
commit of the accepted path and draft-side attention rows: each check ties them
to something other than themselves.

Sources of truth used here:
  * the dynamic-tree flattening (pinned on its own by ancestor closure, the
    causal chain and the It / is / a / has fixture) on the same trees;
  * reachability by boolean matrix powers of the parent relation;
  * closed forms of a rotation whose angle grows linearly with position: the
    identity at position 0, norm preservation, composition R(a) R(b) = R(a + b),
    the relative-position identity <R(p) q, R(r) k> = <R(p - r) q, k>, the
    angle of the first frequency (the position itself) and of frequency D/4
    (position / sqrt(base)), and the half-split pairing of coordinates;
  * consistency with plain autoregressive decoding (EAGLE-2 page, passage after
    the two stages): a committed cache must equal the cache that decoding the
    accepted tokens one by one would have produced, for a model whose K/V rows
    depend only on the token prefix;
  * for the draft side: the union of the frontier's root paths by parent walks,
    the frontier recomputed from its definition (the m best nodes of the last
    layer by value, then id), and softmax attention over exactly the context and
    a frontier node's root path.
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _closure_mask(parent):
    T = len(parent)
    A = np.zeros((T, T), dtype=np.int64)
    for i, p in enumerate(parent):
        if p >= 0:
            A[i, p] = 1
    M = np.eye(T, dtype=bool)
    P = np.eye(T, dtype=np.int64)
    for _ in range(T):
        P = ((P @ A) > 0).astype(np.int64)
        M |= P > 0
    return M


def _random_parent(rng, T):
    par = np.full(T, -1, np.int32)
    for i in range(1, T):
        par[i] = rng.integers(0, i)
    return par


# ---------------------------------------------------------------------------
# Static tree flattening
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(12))
def test_static_flatten_equals_dynamic_flatten(orc, seed):
    rng = np.random.default_rng(700 + seed)
    V = 14; depth = int(rng.integers(1, 5)); k = int(rng.integers(1, 4)); m = int(rng.integers(1, 4))
    fs, cap = orc.tree_shape(depth, k, m)
    z = rng.normal(0, 2, (int(fs.sum()), V)).astype(np.float32)
    n = int(rng.integers(0, cap))
    ctx = int(rng.integers(0, 40))
    tree, kept, flat = orc.build_tree(z, 1, depth, k, m, n, ctx)
    st = orc.flatten_static(flat["flat_parent"], ctx)
    np.testing.assert_array_equal(st["flat_depth"], flat["flat_depth"])
    np.testing.assert_array_equal(st["position"], flat["position"])
    np.testing.assert_array_equal(st["mask"], flat["mask"])


@pytest.mark.parametrize("seed", range(12))
def test_static_flatten_is_ancestor_closure(orc, seed):
    rng = np.random.default_rng(800 + seed)
    T = int(rng.integers(1, 65))
    par = _random_parent(rng, T)
    st = orc.flatten_static(par, 100)
    assert (st["mask"].astype(bool) == _closure_mask(par)).all()
    # depth = number of proper ancestors = row sum of the mask minus the row itself
    np.testing.assert_array_equal(st["flat_depth"], st["mask"].sum(axis=1) - 1)
    np.testing.assert_array_equal(st["position"], 100 + st["flat_depth"])


def test_static_chain_is_causal_and_it_is_a_has(orc):
    T = 9
    st = orc.flatten_static(np.arange(-1, T - 1), 5)
    assert (st["mask"].astype(bool) == np.tril(np.ones((T, T), dtype=bool))).all()
    np.testing.assert_array_equal(st["position"], 5 + np.arange(T))
    fx = json.load(open(os.path.join(GOLD, "it_is_a_has.json")))
    order = ["It", "is", "has", "a"]
    par = [-1 if fx["tree"][t] is None else order.index(fx["tree"][t]) for t in order]
    mask = orc.flatten_static(par, 0)["mask"].astype(bool)
    for tok, spec in fx["page_fixes"].items():
        for s in spec["sees"]:
            assert mask[order.index(tok), order.index(s)]
        for s in spec["never"]:
            assert not mask[order.index(tok), order.index(s)]


@pytest.mark.parametrize("par", [[0], [-1, 1], [-1, 0, 3, 1], [-1, -1], [-1, 0, 2]])
def test_static_flatten_rejects_non_trees(orc, par):
    with pytest.raises(ValueError):
        orc.flatten_static(par, 0)


# ---------------------------------------------------------------------------
# Rotary at tree positions
# ---------------------------------------------------------------------------
def test_rope_position_zero_is_identity(orc):
    x = np.random.default_rng(0).normal(0, 1, (3, 4, 64)).astype(np.float32)
    out = orc.rope(x, [0, 0, 0])
    np.testing.assert_array_equal(out, x.astype(np.float64))


@pytest.mark.parametrize("D", [8, 64, 128])
def test_rope_is_a_rotation_linear_in_position(orc, D):
    rng = np.random.default_rng(D)
    x = rng.normal(0, 1, (1, 2, D)).astype(np.float32)
    xs = x.astype(np.float64)
    for p in (1, 7, 300, 4157, 16444):
        y = orc.rope(x, [p])
        np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(xs, axis=-1), rtol=1e-12)
        # pairs (d, d + D/2) each keep their own norm
        h = D // 2
        np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:] ** 2, xs[..., :h] ** 2 + xs[..., h:] ** 2,
                                   rtol=1e-10, atol=1e-12)
    # composition: rotating by a then by b equals rotating by a + b
    a, b = 123, 4096
    ya = orc.rope(x, [a]).astype(np.float32)  # re-enters as fp32
    yab = orc.rope(ya, [b])
    np.testing.assert_allclose(yab, orc.rope(x, [a + b]), atol=2e-6)


@pytest.mark.parametrize("p,r", [(5, 2), (4100, 4096), (16440, 3), (10, 10)])
def test_rope_relative_position_identity(orc, p, r):
    rng = np.random.default_rng(p * 31 + r)
    q = rng.normal(0, 1, (1, 1, 128)).astype(np.float32)
    k = rng.normal(0, 1, (1, 1, 128)).astype(np.float32)
    lhs = float(np.sum(orc.rope(q, [p]) * orc.rope(k, [r])))
    rhs = float(np.sum(orc.rope(q, [p - r]) * k.astype(np.float64)))
    assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))


def test_rope_frequencies_and_pairing(orc):
    D, base = 64, 10000.0
    h = D // 2
    for d in range(h):
        e = np.zeros((1, 1, D), np.float32); e[0, 0, d] = 1.0
        y = orc.rope(e, [3])[0, 0]
        support = set(np.nonzero(np.abs(y) > 1e-15)[0]) - {d, d + h}
        assert not support, f"coordinate {d} leaked into {support}"
    # first frequency: the angle is the position itself
    e0 = np.zeros((1, 1, D), np.float32); e0[0, 0, 0] = 1.0
    y = orc.rope(e0, [5])[0, 0]
    assert abs(y[0] - np.cos(5.0)) < 1e-15 and abs(y[h] - np.sin(5.0)) < 1e-15
    # frequency index D/4: base^(-1/2)
    eq = np.zeros((1, 1, D), np.float32); eq[0, 0, D // 4] = 1.0
    y = orc.rope(eq, [700], base=base)[0, 0]
    ang = 700.0 / np.sqrt(base)
    assert abs(y[D // 4] - np.cos(ang)) < 1e-12 and abs(y[D // 4 + h] - np.sin(ang)) < 1e-12


def test_rope_at_tree_positions_matches_decoding(orc):
    """Rows at equal depth share a position (siblings get the same rotation), and a
    chain tree's rows rotate exactly as consecutive decoding positions."""
    rng = np.random.default_rng(3)
    V = 10
    fs, cap = orc.tree_shape(3, 3, 2)
    z = rng.normal(0, 2, (int(fs.sum()), V)).astype(np.float32)
    tree, kept, flat = orc.build_tree(z, 0, 3, 3, 2, cap - 1, 50)
    T = cap
    x = np.repeat(rng.normal(0, 1, (1, 2, 32)).astype(np.float32), T, axis=0)
    y = orc.rope(x, flat["position"])
    for i in range(T):
        ar = orc.rope(x[:1], [50 + int(flat["flat_depth"][i])])
        np.testing.assert_array_equal(y[i], ar[0])


# ---------------------------------------------------------------------------
# KV commit of the accepted path
# ---------------------------------------------------------------------------
def _fake_kv(prefix, D):
    """K/V row of the last token of `prefix`, a function of the token prefix only
    (what causal attention guarantees for a real model)."""
    h = 1469598103934665603
    for t in prefix:
        h = ((h ^ (int(t) + 1)) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return np.random.default_rng(h).normal(0, 1, D).astype(np.float32)


def _tree_cache(flat, ctx_tokens, H, D, extra_rows):
    T = len(flat["flat_token"])
    ctx = len(ctx_tokens)
    rows = ctx + T + extra_rows
    cache = np.zeros((H, rows, D), np.float32)
    for g in range(H):
        for c in range(ctx):
            cache[g, c] = _fake_kv((g,) + tuple(ctx_tokens[:c + 1]), D)
        for i in range(T):
            path = []
            r = i
            while r >= 0:
                path.append(int(flat["flat_token"][r])); r = int(flat["flat_parent"][r])
            cache[g, ctx + i] = _fake_kv((g,) + tuple(ctx_tokens) + tuple(path[::-1]), D)
        cache[g, ctx + T:] = 7.0
    return cache


@pytest.mark.parametrize("seed", range(10))
def test_kv_commit_equals_autoregressive_cache(orc, seed):
    rng = np.random.default_rng(900 + seed)
    V = 8; depth = int(rng.integers(1, 5)); k = int(rng.integers(1, 4)); m = int(rng.integers(1, 4))
    fs, cap = orc.tree_shape(depth, k, m)
    z = rng.normal(0, 2, (int(fs.sum()), V)).astype(np.float32)
    n = int(rng.integers(0, cap))
    ctx_tokens = list(rng.integers(0, V, int(rng.integers(0, 12))))
    tree, kept, flat = orc.build_tree(z, int(rng.integers(0, V)), depth, k, m, n, len(ctx_tokens))
    T = n + 1
    target = rng.normal(0, 1, (T, V)).astype(np.float32)
    for i in range(1, T):
        if rng.random() < 0.7:
            target[flat["flat_parent"][i], flat["flat_token"][i]] = 9.0 + rng.random()
    al, ap, ot = orc.verify_greedy(target, flat["flat_token"], flat["flat_parent"], depth)
    H, D = 3, 16
    cache = _tree_cache(flat, ctx_tokens, H, D, extra_rows=5)
    before = cache.copy()
    ctx = len(ctx_tokens)
    new_ctx = orc.kv_commit(cache, ctx, T, al, ap)
    assert new_ctx == ctx + 1 + al
    # the decoded sequence: context, the root token, then the accepted tokens
    seq = list(ctx_tokens) + [int(flat["flat_token"][0])] + [int(t) for t in ot[:al]]
    for g in range(H):
        for c in range(new_ctx):
            np.testing.assert_array_equal(cache[g, c], _fake_kv((g,) + tuple(seq[:c + 1]), D))
    np.testing.assert_array_equal(cache[:, new_ctx:], before[:, new_ctx:])


def test_kv_commit_noops(orc):
    rng = np.random.default_rng(5)
    cache = rng.normal(0, 1, (2, 30, 8)).astype(np.float32)
    before = cache.copy()
    assert orc.kv_commit(cache, 10, 12, 0, []) == 11
    assert orc.kv_commit(cache, 10, 12, 4, [1, 2, 3, 4]) == 15
    np.testing.assert_array_equal(cache, before)
    # packed cache: another sequence's rows are not touched
    cache2 = before.copy()
    orc.kv_commit(cache2, 3, 6, 2, [2, 5], row0=20)
    np.testing.assert_array_equal(cache2[:, :20], before[:, :20])
    np.testing.assert_array_equal(cache2[:, 24], before[:, 25])
    np.testing.assert_array_equal(cache2[:, 25], before[:, 28])


@pytest.mark.parametrize("al,path", [(2, [3, 3]), (2, [4, 2]), (1, [0]), (1, [6]), (-1, []), (6, [1, 2, 3, 4, 5, 6])])
def test_kv_commit_rejects_non_paths(orc, al, path):
    cache = np.zeros((1, 20, 4), np.float32)
    with pytest.raises(ValueError):
        orc.kv_commit(cache, 4, 6, al, path)


# ---------------------------------------------------------------------------
# Draft-side attention rows: the frontier's root paths as a small flattened tree
# ---------------------------------------------------------------------------
def _frontier_of_layer(tree, layer, m):
    """Frontier consumed by draft layer `layer` (>= 2): the min(m, |layer - 1|) nodes
    of depth layer - 1 with the largest value, ties to the lower id."""
    ids = np.nonzero(tree["depth"] == layer - 1)[0]
    order = np.lexsort((ids, -tree["value"][ids].astype(np.float64)))
    return ids[order][:min(m, len(ids))]


def _root_path(tree, x):
    path = []
    while x >= 0:
        path.append(int(x)); x = int(tree["parent"][x])
    return path


@pytest.mark.parametrize("seed", range(12))
def test_draft_subtree_is_union_of_root_paths(orc, seed):
    rng = np.random.default_rng(1100 + seed)
    V = 16; depth = int(rng.integers(2, 6)); k = int(rng.integers(1, 5)); m = int(rng.integers(1, 5))
    fs, cap = orc.tree_shape(depth, k, m)
    z = rng.normal(0, 2, (int(fs.sum()), V)).astype(np.float32)
    tree = orc.expand(z, 2, depth, k, m)
    ctx = int(rng.integers(0, 30))
    for layer in range(2, depth + 1):
        fr = _frontier_of_layer(tree, layer, m)
        T_sub = 1 + len(fr) * (layer - 1) + int(rng.integers(0, 3))
        st = orc.draft_subtree(tree, fr, ctx, T_sub)
        U = sorted(set(x for f in fr for x in _root_path(tree, f)))
        nU = len(U)
        assert list(st["sub_node"][:nU]) == U and all(x == -1 for x in st["sub_node"][nU:])
        row = {x: r for r, x in enumerate(U)}
        for r, x in enumerate(U):
            assert st["position"][r] == ctx + tree["depth"][x]
            seen = {int(c) for c in np.nonzero(st["mask"][r])[0]}
            assert seen == {row[y] for y in _root_path(tree, x)}
            p = tree["parent"][x]
            assert st["sub_parent"][r] == (row[p] if p >= 0 else -1)
        for r in range(nU, T_sub):
            assert set(np.nonzero(st["mask"][r])[0]) == {r} and st["position"][r] == ctx
        assert [U[q] for q in st["query_row"]] == [int(f) for f in fr]


def test_draft_subtree_attention_is_context_plus_root_path(orc):
    """Attention of a frontier node's row over the flattened rows equals softmax
    attention over exactly the context and that node's root path."""
    rng = np.random.default_rng(77)
    V, depth, k, m = 20, 4, 3, 3
    fs, cap = orc.tree_shape(depth, k, m)
    z = rng.normal(0, 2, (int(fs.sum()), V)).astype(np.float32)
    tree = orc.expand(z, 0, depth, k, m)
    layer, ctx, H, D = 4, 23, 2, 16
    fr = _frontier_of_layer(tree, layer, m)
    T_sub = 1 + len(fr) * (layer - 1)
    st = orc.draft_subtree(tree, fr, ctx, T_sub)
    n_nodes = len(tree["parent"])
    # node-indexed draft K/V and per-node queries
    kc = rng.normal(0, 1, (H, ctx, D)).astype(np.float32); vc = rng.normal(0, 1, (H, ctx, D)).astype(np.float32)
    kn = rng.normal(0, 1, (H, n_nodes, D)).astype(np.float32); vn = rng.normal(0, 1, (H, n_nodes, D)).astype(np.float32)
    qn = rng.normal(0, 1, (n_nodes, H, D)).astype(np.float32)
    nodes = np.where(st["sub_node"] >= 0, st["sub_node"], 0)
    k = np.concatenate([kc, kn[:, nodes]], axis=1); v = np.concatenate([vc, vn[:, nodes]], axis=1)
    q = qn[nodes]
    o, lse = orc.attention(q, k, v, st["mask"], ctx)
    for j, f in enumerate(fr):
        path = _root_path(tree, f)
        keys = np.concatenate([kc, kn[:, path]], axis=1).astype(np.float64)
        vals = np.concatenate([vc, vn[:, path]], axis=1).astype(np.float64)
        for h in range(H):
            sc = keys[h] @ qn[f, h].astype(np.float64) / np.sqrt(D)
            w = np.exp(sc - sc.max()); w /= w.sum()
            np.testing.assert_allclose(o[st["query_row"][j], h], w @ vals[h], rtol=1e-12, atol=1e-12)


def test_draft_subtree_rejects_overflow(orc):
    tree = dict(parent=np.array([-1, 0, 0, 1, 2]), depth=np.array([0, 1, 1, 2, 2]))
    with pytest.raises(ValueError):
        orc.draft_subtree(tree, [3, 4], 0, 4)  # needs 5 rows
    with pytest.raises(ValueError):
        orc.draft_subtree(tree, [9], 0, 8)
    st = orc.draft_subtree(tree, [3, 4], 0, 5)
    assert list(st["sub_node"]) == [0, 1, 2, 3, 4]
