"""Logits holding NaN or +-Inf: the library promises memory-safe calls with
unspecified values (include/eagle_tree.h, conventions).  Every index the kernels
derive from logits comes from a (logit order, token id) key, so tokens stay inside
the vocabulary and node and row ids inside the tree whatever the values are; this
checks that on the GPU, through the C ABI: the calls return EAGLE_OK (the binding
raises otherwise), and the tree, its flattening and the verdicts are structurally
valid (ids, parents, masks, paths and tokens in range).  With such values the kept
set need not be ancestor-closed: a row whose parent was not kept has parent -1."""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from draft_tree_verification_eagle_amd import binding, step, workload
    binding.lib()
    return binding, step, workload


def poison_rows(x, rng):
    """x: [..., V] float32; poisons a spread of rows in place in four ways."""
    rows = x.reshape(-1, x.shape[-1])
    V = rows.shape[1]
    for r in range(rows.shape[0]):
        kind = r % 5
        if kind == 0:    # all NaN
            rows[r] = np.nan
        elif kind == 1:  # a few +Inf (ties among them) and a few NaN
            rows[r, rng.integers(0, V, 7)] = np.inf
            rows[r, rng.integers(0, V, 5)] = np.nan
        elif kind == 2:  # all -Inf but one finite entry
            keep = rng.integers(0, V)
            v = rows[r, keep]
            rows[r] = -np.inf
            rows[r, keep] = v
        elif kind == 3:  # negative NaN (sign bit set) and -Inf mixed in
            rows[r, rng.integers(0, V, 9)] = -np.nan
            rows[r, rng.integers(0, V, 9)] = -np.inf
        # kind 4: left finite


def check_tree(vs, w):
    B, T, V, cap = w.batch, w.T, w.vocab, vs.cap
    st = vs.state
    tok = st.token.cpu().numpy()
    par = st.parent.cpu().numpy()
    dep = st.depth.cpu().numpy()
    n_nodes = st.n_nodes.cpu().numpy()
    for b in range(B):
        assert n_nodes[b] == cap
        assert par[b, 0] == -1 and dep[b, 0] == 0
        ids = np.arange(1, cap)
        assert np.all((tok[b, 1:] >= 0) & (tok[b, 1:] < V))
        assert np.all((par[b, 1:] >= 0) & (par[b, 1:] < ids))
        assert np.all(dep[b, 1:] == dep[b, par[b, 1:]] + 1)
    kept = vs.kept.cpu().numpy()
    for b in range(B):
        k = kept[b, :w.n]
        assert np.all((k >= 1) & (k < cap)) and np.all(np.diff(k) > 0)
    ft = vs.flat_token.cpu().numpy()
    fp = vs.flat_parent.cpu().numpy()
    fd = vs.flat_depth.cpu().numpy()
    pos = vs.position.cpu().numpy()
    mask = vs.mask.cpu().numpy().view(np.uint64)
    for b in range(B):
        assert fp[b, 0] == -1 and fd[b, 0] == 0
        for i in range(T):
            assert 0 <= ft[b, i] < V
            assert -1 <= fp[b, i] < i
            assert pos[b, i] == vs.ctx_lens_np[b] + fd[b, i]
            m = int(mask[b, i])
            want = 1 << i
            if fp[b, i] >= 0:
                want |= int(mask[b, fp[b, i]])
            assert m == want
    return ft, fp


def check_verdict(vs, w, fp, ft):
    B, T, V, d = w.batch, w.T, w.vocab, w.depth
    L = vs.accept_len.cpu().numpy()
    P = vs.accept_path.cpu().numpy()
    O = vs.out_tokens.cpu().numpy()
    for b in range(B):
        assert 0 <= L[b] <= d
        cur = 0
        for k in range(L[b]):
            r = P[b, k]
            assert 1 <= r < T and fp[b, r] == cur
            assert O[b, k] == ft[b, r]
            cur = r
        assert np.all(P[b, L[b]:] == -1)
        assert -1 <= O[b, L[b]] < V
        assert np.all(O[b, L[b] + 1:] == -1)


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["tiny_f32", "llama2_7b_layer"])
def test_nonfinite_logits_are_memory_safe(mods, name):
    binding, step, wl = mods
    w = wl.CONFIGS[name]
    rng = np.random.default_rng(41)
    draft = wl.draft_logits(w).astype(np.float32, copy=True)
    poison_rows(draft, rng)
    print(f"[nonfinite] {name}: tree from poisoned draft logits", flush=True)
    vs = step.VerifyStep(w, device="cuda", draft=draft)
    vs.tree()
    torch.cuda.synchronize()
    ft, fp = check_tree(vs, w)
    vs.attention()
    torch.cuda.synchronize()
    target = wl.target_logits_base(w).astype(np.float32, copy=True)
    poison_rows(target, rng)
    vs.set_target(target)
    for temp, seed in ((0.0, 1), (1.0, 5), (0.7, 9)):
        vs.accept_len.fill_(-7)
        vs.out_tokens.fill_(-7)
        vs.verify(temp, seed, 3)
        torch.cuda.synchronize()
        check_verdict(vs, w, fp, ft)
