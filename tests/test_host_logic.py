"""Host-side logic that needs no GPU: the step driver's buffer set-up (no
launches happen in its constructor), workload shapes and the plant rule."""
import numpy as np
import pytest
import scipy.special

from draft_tree_verification_eagle_amd import step as stepm
from draft_tree_verification_eagle_amd import workload as wl


@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_step_buffers_on_cpu(name):
    w = wl.CONFIGS[name]
    vs = stepm.VerifyStep(w, device="cpu", layers=0)
    assert vs.cap == w.capacity
    assert [t.shape for t in vs.draft_layers] == [(w.batch, f, w.vocab) for f in w.frontier_sizes()]
    assert vs.kv_rows_total == int((w.ctx_lens().astype(np.int64) + w.T).sum())
    assert vs.attn_ws.numel() >= 1 and vs.verify_ws.numel() >= 1


def test_step_buffers_with_layers_on_cpu():
    w = wl.CONFIGS["tiny_f32"].replace(layers=2)
    vs = stepm.VerifyStep(w, device="cpu")
    assert len(vs.attn) == 2
    q, k = vs.attn[0]["q"], vs.attn[0]["k"]
    assert q.shape == (1, w.T, w.n_q_heads, w.head_dim) and k.shape == (w.n_kv_heads, 256 + w.T, w.head_dim)
    assert not np.array_equal(vs.attn[0]["k"].numpy(), vs.attn[1]["k"].numpy())


def test_ragged_offsets_are_contiguous():
    w = wl.CONFIGS["batched_13b"]
    lens = w.ctx_lens()
    assert lens.min() >= 512 and lens.max() <= 16384 and len(lens) == 16
    off, total = w.kv_row_offsets()
    assert off[0] == 0 and np.all(np.diff(off) == lens[:-1] + w.T) and total == off[-1] + lens[-1] + w.T


def test_plant_rule_sets_the_share_and_skips_planted_parents():
    rng = np.random.default_rng(0)
    T, V = 9, 50
    ft = rng.integers(0, V, (1, T)).astype(np.int32)
    fp = np.array([[-1, 0, 0, 1, 1, 2, 3, 3, 6]], dtype=np.int32)
    base = rng.normal(0, 2, (1, T, V)).astype(np.float32)
    out = wl.plant(base, ft, fp, 1.0, 3)
    planted_parents = set()
    for v in range(1, T):
        p = fp[0, v]
        if p in planted_parents:
            continue
        planted_parents.add(p)
        share = scipy.special.softmax(out[0, p].astype(np.float64))[ft[0, v]]
        assert abs(share - 0.8) < 1e-5 and np.argmax(out[0, p]) == ft[0, v]
    assert np.array_equal(wl.plant(base, ft, fp, 0.0, 3), base)
