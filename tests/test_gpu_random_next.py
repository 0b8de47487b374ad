"""GPU parity of the calls around the step on seeded random workloads (the
generator of the random attention sweep): the static-tree mask of each tree's
flattened parents (against the dynamic mask and the oracle), the rotary at the
tree positions, the KV commit of the path the GPU's own greedy verification of
planted targets accepts (every layer, bit for bit), and, for some of them, the
draft-side rows of every draft layer as the tree grows."""
import random

import numpy as np
import pytest
import torch

import test_gpu_next as N
import test_gpu_random_sweep as RS
from test_gpu_parity import lib  # noqa: F401  (the library fixture)

pytestmark = pytest.mark.gpu


def draft_rows_every_layer(eb, stepm, orc, w):
    vs = stepm.VerifyStep(w, layers=0)
    trees = [orc.expand(vs.draft_np[b], int(vs.root_np[b]), w.depth, w.topk, w.m) for b in range(w.batch)]
    for layer in range(1, w.depth + 1):
        if layer >= 2:
            eb.eagle_tree_expand(vs.cfg, layer - 1, vs.draft_layers[layer - 2], vs.root, vs.state, vs.expand_ws)
        T_sub = eb.eagle_draft_subtree_rows(vs.cfg, layer)
        buf = N._subtree_buffers(w, T_sub)
        if T_sub > 64:  # more rows than one mask word: documented as unsupported, nothing launched
            with pytest.raises(eb.EagleError) as err:
                eb.eagle_draft_subtree(vs.cfg, layer, vs.state, vs.ctx_len, buf["node"], buf["parent"],
                                       buf["position"], buf["mask"], buf["query_row"])
            assert err.value.status == eb.EAGLE_ERR_UNSUPPORTED
            continue
        eb.eagle_draft_subtree(vs.cfg, layer, vs.state, vs.ctx_len, buf["node"], buf["parent"], buf["position"],
                               buf["mask"], buf["query_row"])
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in buf.items()}
        for b in range(w.batch):
            fr = [0] if layer == 1 else N._frontier_of_layer(trees[b], layer, w.m)
            ref = orc.draft_subtree(trees[b], fr, int(vs.ctx_lens_np[b]), T_sub)
            np.testing.assert_array_equal(got["node"][b], ref["sub_node"])
            np.testing.assert_array_equal(got["parent"][b], ref["sub_parent"])
            np.testing.assert_array_equal(got["position"][b], ref["position"])
            np.testing.assert_array_equal(got["mask"][b].view(np.uint64), N.mask_words(ref["mask"]))
            qr = np.full(w.m, -1, np.int32)
            qr[:len(fr)] = ref["query_row"]
            np.testing.assert_array_equal(got["query_row"][b], qr)


@pytest.mark.parametrize("block", range(2))
def test_random_next_rows(lib, orc, block):
    eb, stepm, wl = lib
    rng = random.Random(8191 + block)
    for i in range(25):
        kw = RS.random_workload(rng)
        kw["ctx"] = min(kw["ctx"], 3000)
        if kw["ctx_range"] is not None:
            kw["ctx_range"] = (kw["ctx_range"][0], min(kw["ctx_range"][1], 3000))
        N.say(f"[random next {block}.{i}] {kw}")
        w = N.small(wl, **kw, layers=2)
        vs = stepm.VerifyStep(w, layers=2)
        vs.tree()
        torch.cuda.synchronize()
        # static-tree mask of the flattened parents
        fp = vs.flat_parent.cpu().numpy()
        dep, pos, msk = N.static_mask(eb, fp, vs.ctx_lens_np)
        np.testing.assert_array_equal(dep, vs.flat_depth.cpu().numpy())
        np.testing.assert_array_equal(pos, vs.position.cpu().numpy())
        np.testing.assert_array_equal(msk, vs.mask.cpu().numpy().view(np.uint64))
        st = orc.flatten_static(fp[0], int(vs.ctx_lens_np[0]))
        np.testing.assert_array_equal(msk[0], N.mask_words(st["mask"]))
        # rotary of layer 0's q and tree rows of K
        N.rope_check(eb, orc, vs, base=500000.0 if w.dtype == "f32" else 10000.0)
        # KV commit of the greedily accepted paths, both layers
        ft, fpar = vs.flat_host()
        vs.set_target(wl.plant(wl.target_logits_base(w), ft, fpar, 0.8, w.seed))
        vs.verify(0.0, 0, 0)
        torch.cuda.synchronize()
        al = vs.accept_len.cpu().numpy()
        ap = vs.accept_path.cpu().numpy()
        dtype = eb.EAGLE_F32 if w.dtype == "f32" else eb.EAGLE_BF16
        N.commit_check(eb, orc, [(a["k"], a["v"]) for a in vs.attn], vs.ctx_lens_np, vs.kv_off_np, w.T, w.depth,
                       al, ap, dtype, w.head_dim, w.n_kv_heads)
        if i < 8:
            draft_rows_every_layer(eb, stepm, orc, w)
