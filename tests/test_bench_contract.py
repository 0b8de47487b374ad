"""bench.py pieces that need no GPU: the one-GPU rule on the command line, and the
algorithmic bytes per attention call against the per-call figures the sizes give
by hand (K and V over ctx + T rows per KV head, plus Q and O)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


@pytest.mark.parametrize("name,expect", [
    # 40 KV heads x (4096 + 61) rows x 128 x 2 B x (K, V) + 2 x 61 x 40 x 128 x 2 B
    ("llama2_13b", 2 * 40 * 4157 * 128 * 2 + 2 * 61 * 40 * 128 * 2),
    # 32 heads, ctx 2048
    ("llama2_7b_layer", 2 * 32 * 2109 * 128 * 2 + 2 * 61 * 32 * 128 * 2),
    # 8 KV heads, ctx 8192; Q and O over the 64 query heads
    ("llama2_70b_gqa", 2 * 8 * 8253 * 128 * 2 + 2 * 61 * 64 * 128 * 2),
    # fp32, 4 heads x 64, ctx 256, T = 16
    ("tiny_f32", 2 * 4 * 272 * 64 * 4 + 2 * 16 * 4 * 64 * 4),
])
def test_attention_bytes_per_launch(name, expect):
    sys.path.insert(0, ROOT)
    import bench
    from draft_tree_verification_eagle_amd import workload as wl
    assert bench.attention_bytes_per_launch(wl.CONFIGS[name]) == expect


def test_attention_bytes_13b_matches_the_stated_figure():
    sys.path.insert(0, ROOT)
    import bench
    from draft_tree_verification_eagle_amd import workload as wl
    assert bench.attention_bytes_per_launch(wl.CONFIGS["llama2_13b"]) == 86_384_640


def test_attention_flops_count_context_and_ancestors():
    """4 D flops per (query head, attended key); a chain of T rows attends to ctx + i + 1 keys."""
    sys.path.insert(0, ROOT)
    import bench
    from draft_tree_verification_eagle_amd import workload as wl
    w = wl.CONFIGS["llama2_13b"]
    T = w.T
    chain = [[(1 << (i + 1)) - 1 for i in range(T)]]  # row i sees rows 0..i
    got = bench.attention_flops_per_launch(w, chain, [4096])
    keys = sum(4096 + i + 1 for i in range(T))
    assert got == keys * w.n_q_heads * 4 * w.head_dim
