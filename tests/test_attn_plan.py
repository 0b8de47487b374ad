"""The bf16 tree-attention work plan, checked on the host before any GPU run.

tests/replica/attn_plan_check.cpp compiles the kernel's plan header
(draft_tree_verification_eagle_amd/csrc/attn_plan.hpp) unchanged, with the
address and undefined-behaviour sanitizers, and walks every workgroup of a
launch the way the kernel does: every tile taken once, every K/V, Q and output
row inside its sequence and the buffers, partial slots and arrival counters
unique, piece counts consistent.  Driven here with the launch descriptors of
every workload (the 16-sequence ragged batch and the 1024-sequence batch, which
the launcher splits into launches of 256 sequences), the GPU edge cases, and
random descriptors.
"""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "replica", "attn_plan_check.cpp")
MAX_SEQS = 256
GRID = 256


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("plan") / "attn_plan_check")
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-o", exe, SRC])
    return exe


def launches(T, Hq, Hkv, ctx, row0, rows_total):
    """The launcher's launches: consecutive chunks of at most 256 sequences."""
    out = []
    for b0 in range(0, len(ctx), MAX_SEQS):
        c = ctx[b0:b0 + MAX_SEQS]; r = row0[b0:b0 + MAX_SEQS]
        out.append(f"{GRID} {T} {Hq} {Hkv} {rows_total} {len(c)} " + " ".join(f"{a} {b}" for a, b in zip(c, r)))
    return out


def packed(ctx, T, gap=0):
    ctx = [int(c) for c in ctx]
    row0, r = [], 0
    for c in ctx:
        row0.append(r)
        r += c + T + gap
    return ctx, row0, r


def run(checker, line):
    p = subprocess.run([checker], input=line, capture_output=True, text=True)
    assert p.returncode == 0, f"plan check failed for `{line[:120]}`:\n{p.stderr[-2000:]}"
    return p.stdout


@pytest.mark.parametrize("name", ["llama2_7b_layer", "llama2_13b", "llama2_70b_gqa", "batched_13b"])
def test_plan_of_every_workload(checker, name):
    from draft_tree_verification_eagle_amd import workload as wl
    w = wl.CONFIGS[name]
    ctx, row0, total = packed(w.ctx_lens(), w.T)
    for line in launches(w.T, w.n_q_heads, w.n_kv_heads, ctx, row0, total):
        out = run(checker, line)
        assert out.startswith("ok")


EDGE = [
    dict(T=1, Hq=4, Hkv=4, ctx=[70]), dict(T=9, Hq=4, Hkv=4, ctx=[0]), dict(T=13, Hq=4, Hkv=4, ctx=[1]),
    dict(T=9, Hq=4, Hkv=4, ctx=[63]), dict(T=9, Hq=4, Hkv=4, ctx=[64]), dict(T=16, Hq=4, Hkv=4, ctx=[65]),
    dict(T=16, Hq=4, Hkv=4, ctx=[0, 57, 200, 13, 129]), dict(T=20, Hq=8, Hkv=2, ctx=[150]),
    dict(T=16, Hq=6, Hkv=1, ctx=[33]), dict(T=64, Hq=4, Hkv=4, ctx=[500]),
    dict(T=61, Hq=40, Hkv=40, ctx=[2000, 9000, 5321]), dict(T=64, Hq=4, Hkv=4, ctx=[100, 100]),
    dict(T=64, Hq=1, Hkv=1, ctx=[16384]), dict(T=64, Hq=1, Hkv=1, ctx=[16384, 0]),
    dict(T=61, Hq=64, Hkv=8, ctx=[8192] * 3),
]


@pytest.mark.parametrize("e", EDGE, ids=[str(i) for i in range(len(EDGE))])
@pytest.mark.parametrize("gap", [0, 7])
def test_plan_edge_shapes(checker, e, gap):
    ctx, row0, total = packed(e["ctx"], e["T"], gap)
    for line in launches(e["T"], e["Hq"], e["Hkv"], ctx, row0, total):
        run(checker, line)


def test_plan_batch_1024(checker):
    rng = np.random.default_rng(17)
    ctx, row0, total = packed(rng.integers(0, 61, 1024), 9)
    lines = launches(9, 4, 4, ctx, row0, total)
    assert len(lines) == 4
    for line in lines:
        run(checker, line)


def test_plan_random_descriptors(checker):
    rng = np.random.default_rng(2026)
    for _ in range(60):
        T = int(rng.integers(1, 65)); Hkv = int(rng.choice([1, 2, 4, 8, 40])); G = int(rng.integers(1, 9))
        B = int(rng.choice([1, 2, 3, 16, 100, 300]))
        hi = int(rng.choice([64, 700, 5000, 20000]))
        ctx = rng.integers(0, hi + 1, B)
        gap = int(rng.integers(0, 3))
        c, r, total = packed(ctx, T, gap)
        RG = (G * T + 63) // 64
        if Hkv * RG * (4 * ((total + 63) // 64 + min(B, 256)) + 16 * min(B, 256)) >= 2 ** 31:
            continue  # the host rejects this shape
        for line in launches(T, Hkv * G, Hkv, c, r, total):
            run(checker, line)


def test_host_reciprocals(tmp_path):
    """The multiply-and-shift divisions the kernels take from host reciprocals
    (attn_plan.hpp recip_of / div_by) equal the plain division for every dividend
    below 2^31: all divisors up to 4096, random divisors up to 2^31 - 1, powers of
    two and their neighbours, and two divisors over every dividend."""
    exe = str(tmp_path / "recip_check")
    subprocess.check_call(["g++", "-std=c++17", "-O2", "-o", exe,
                           os.path.join(ROOT, "tests", "replica", "recip_check.cpp")])
    p = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stderr
    assert p.stdout.strip() == "ok"
