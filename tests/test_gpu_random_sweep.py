"""GPU parity on seeded random workloads: random vocabularies, tree shapes, head
counts and ratios, head sizes, dtypes, batches and (ragged) context lengths within
the library's limits, each through tree build, attention (plain, and with the rotary
inside for bf16 head size 128), host- versus device-held lengths, and greedy and
sampled verification, by the same bars and helpers as the edge-case tests."""
import random

import pytest
import torch

import test_gpu_attention_rope as RP
import test_gpu_parity as P
from test_gpu_parity import lib  # noqa: F401  (the library fixture)

pytestmark = pytest.mark.gpu


def random_workload(rng):
    while True:
        vocab = rng.choice([20, 64, 300, 1000, 5000, 32000, 128000])
        depth = rng.randint(1, 6)
        topk = rng.randint(1, min(16, vocab))
        m = rng.randint(1, topk)
        nodes = 1 + topk + (depth - 1) * m * topk
        if m * topk > 1024 or nodes > 4096:
            continue
        n = rng.randint(0, min(63, nodes - 1))
        hkv = rng.choice([1, 2, 4, 5, 8])
        G = rng.choice([1, 1, 2, 3, 4, 8])
        if hkv * G > 64:
            continue
        r = rng.random()
        if r < 0.8:
            dtype, hd = "bf16", 128
        elif r < 0.9:
            dtype, hd = "bf16", rng.choice([32, 40, 64, 96])
        else:
            dtype, hd = "f32", rng.choice([64, 128])
        batch = rng.choice([1, 1, 1, 2, 3, 6])
        if batch == 1:
            ctx, ctx_range = rng.choice([0, 1, 5, 63, 64, 65, 500, 1500, 3000, 4096, 8000]), None
        else:
            lo = rng.randint(0, 500)
            ctx, ctx_range = 0, (lo, lo + rng.randint(0, 2500))
        return dict(vocab=vocab, depth=depth, topk=topk, m=m, n=n, n_q_heads=hkv * G, n_kv_heads=hkv,
                    head_dim=hd, dtype=dtype, batch=batch, ctx=ctx, ctx_range=ctx_range,
                    seed=rng.randint(1, 10 ** 6))


@pytest.mark.parametrize("block", range(4))
def test_random_workloads(lib, orc, block):
    eb, stepm, wl = lib
    rng = random.Random(4099 + block)
    for i in range(40):
        kw = random_workload(rng)
        P.say(f"[random {block}.{i}] {kw}")
        w = P.small(wl, **kw)
        vs = stepm.VerifyStep(w)
        vs.tree(); vs.attention()
        torch.cuda.synchronize()
        trees = P.oracle_trees(orc, w, vs.draft_np, vs.root_np, vs.ctx_lens_np)
        P.compare_trees(vs, trees)
        dense = w.T * w.n_q_heads * (int(vs.ctx_lens_np.max()) + w.T) * w.batch
        P.attention_check(orc, vs, trees, 0, None if dense < 2e6 else 40,
                          atol=P.ATOL_F32 if w.dtype == "f32" else P.ATOL_BF16)
        P.same_without_host_lengths(eb, vs)
        target, ft, fp = P.planted_target(wl, w, trees)
        P.verify_check(orc, vs, w, target, ft, fp, 0.0, 1, range(1))
        P.verify_check(orc, vs, w, target, ft, fp, 0.8, 7, range(3))
        if w.dtype == "bf16" and w.head_dim == 128:
            RP.fused_check(eb, orc, RP.prepared(stepm, w), n_pairs=None if dense < 2e6 else 40)
