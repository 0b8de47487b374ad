"""eagle_tree_attention_noalloc (no caller workspace; the partials live in the
library's per-device array) against eagle_tree_attention on
the same inputs, through the C ABI: two calls in a row, the second on a smaller
input, each bit-identical to the workspace entry point (the same kernels, the same
arithmetic), plus the size limit and the checks of a bad argument.
"""
import ctypes as C
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_tree_verification_eagle_amd import binding, step, workload
    return binding, step, workload


def shape(wl, **kw):
    base = dict(name="noalloc", vocab=500, depth=4, topk=4, m=4, n=25, n_q_heads=32, n_kv_heads=32, head_dim=128,
                layers=1, batch=2, ctx=2048, ctx_range=None, dtype="bf16", draft_sigma=2.0, target_sigma=2.0,
                temperatures=(0.0,), plant_frac=0.5, seed=55)
    base.update(kw)
    return wl.Workload(**base)


def both_ways(eb, vs):
    """(o, lse) of the workspace entry point and of the no-alloc one."""
    a = vs.attn[0]
    o1 = torch.full_like(a["o"], float("nan")); l1 = torch.full_like(a["lse"], float("nan"))
    o2 = torch.full_like(a["o"], float("nan")); l2 = torch.full_like(a["lse"], float("nan"))
    eb.eagle_tree_attention(vs.desc, a["q"], a["k"], a["v"], vs.mask, o1, l1, vs.attn_ws)
    eb.eagle_tree_attention_noalloc(vs.desc, a["q"], a["k"], a["v"], vs.mask, o2, l2)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def test_noalloc_matches_workspace_entry_point_twice(lib, orc):
    eb, stepm, wl = lib
    big = shape(wl, batch=3, ctx_range=(1500, 6000), n_q_heads=40, n_kv_heads=40, n=60, depth=6, topk=10, m=10,
                seed=56)
    small = shape(wl, batch=1, ctx=300, n_q_heads=8, n_kv_heads=2, n=15, seed=57)
    for w in (big, small):  # the second call is on a smaller input
        say(f"[no-alloc attention] batch {w.batch}, heads {w.n_q_heads}/{w.n_kv_heads}, T {w.T}")
        vs = stepm.VerifyStep(w)
        vs.tree()
        o1, l1, o2, l2 = both_ways(eb, vs)
        assert torch.isfinite(o1.float()).all()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        # one output row against the oracle as well
        b = 0
        ctx = int(vs.ctx_lens_np[b]); r0 = int(vs.kv_off_np[b])
        a = vs.attn[0]
        tree, kept, flat = orc.build_tree(vs.draft_np[b], int(vs.root_np[b]), w.depth, w.topk, w.m, w.n, ctx)
        k = a["k"][:, r0:r0 + ctx + w.T].float().cpu().numpy(); v = a["v"][:, r0:r0 + ctx + w.T].float().cpu().numpy()
        oo, _ = orc.attention(a["q"][b].float().cpu().numpy(), k, v, flat["mask"], ctx, sel=[(w.T - 1, 0)])
        assert np.abs(o2[b, w.T - 1, 0].float().cpu().numpy() - oo[0]).max() <= 2e-2


def test_noalloc_size_limit_and_bad_arguments(lib):
    eb, stepm, wl = lib
    L = eb.lib()
    dev = torch.zeros(64, dtype=torch.int64, device="cuda")
    f = dev.data_ptr()
    # the partials of any accepted shape fit the array (1024 sequences x 1024 KV heads)
    d = eb.make_attn_desc(eb.EAGLE_BF16, 1024, 64, 1024, 1024, 128, dev, dev, 1024 * 4096)
    assert 0 < eb.eagle_tree_attention_workspace(d) <= (16 << 20)
    d2 = eb.make_attn_desc(eb.EAGLE_BF16, 1, 16, 8, 8, 128, dev, dev, 4096)
    assert L.eagle_tree_attention_noalloc(C.byref(d2), None, f, f, f, f, None, None) == eb.EAGLE_ERR_INVALID_ARG
    d3 = eb.make_attn_desc(eb.EAGLE_BF16, 1, 16, 8, 8, 130, dev, dev, 4096)  # head_dim > 128: rejected
    assert L.eagle_tree_attention_noalloc(C.byref(d3), f, f, f, f, f, None, None) == eb.EAGLE_ERR_UNSUPPORTED


def test_noalloc_graph_replays_match_eager(lib):
    """The callers this entry point is for include code under HIP graph capture: a
    captured no-alloc call replays to its eager result bit for bit, with eager
    no-alloc calls on other inputs (which overwrite the shared array) in between."""
    eb, stepm, wl = lib
    w = shape(wl, batch=2, ctx_range=(700, 3000), n_q_heads=16, n_kv_heads=4, n=40, depth=5, topk=8, m=8, seed=58)
    other = shape(wl, batch=1, ctx=5000, n_q_heads=40, n_kv_heads=40, n=60, depth=6, topk=10, m=10, seed=59)
    say(f"[no-alloc graph] batch {w.batch}, heads {w.n_q_heads}/{w.n_kv_heads}, T {w.T}")
    vs = stepm.VerifyStep(w)
    vs.tree()
    vo = stepm.VerifyStep(other)
    vo.tree()
    a, ao = vs.attn[0], vo.attn[0]
    o = torch.empty_like(a["o"]); lse = torch.empty_like(a["lse"])
    eb.eagle_tree_attention_noalloc(vs.desc, a["q"], a["k"], a["v"], vs.mask, o, lse)  # eager, also the warm-up
    torch.cuda.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        eb.eagle_tree_attention_noalloc(vs.desc, a["q"], a["k"], a["v"], vs.mask, o, lse)
    torch.cuda.synchronize()
    for rep in range(3):
        eb.eagle_tree_attention_noalloc(vo.desc, ao["q"], ao["k"], ao["v"], vo.mask, ao["o"], ao["lse"])
        o.fill_(7.0); lse.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"replay {rep} differs from the eager call"
