"""Seeded synthetic workloads for one draft-tree verification step.

This module is shared by the HIP path's callers (tests, bench) and by the
CPU oracle's callers.  It only draws random numbers and shapes; it holds none
of the method's arithmetic (no softmax, no top-k, no tree logic, no attention).

The five workloads mirror LLaMA2-shaped layers (7B, 13B, 70B-GQA, a tiny fp32
case and a ragged 16-sequence batch of the 13B shape).  "N(0, s)" in the
workload descriptions is read as mean 0, standard deviation s.

Tensor families and their generators:
  * draft logits  -- numpy PCG64, fp32, [B][R][V]; R = draft rows of all
                     layers, layer-major, frontier order inside a layer.
  * target logits -- numpy PCG64, fp32, [B][T][V]; optionally planted (below).
  * Q / K / V     -- torch generator on the requested device, N(0, 1), in the
                     workload's storage dtype.
  * ragged context lengths -- numpy PCG64, uniform integers.

Plant rule (so greedy and sampled acceptance lengths are non-trivial): after
the tree is known, walk the flattened rows in order; a row v (not the root) is
chosen with probability `plant_frac` unless its parent row already carries a
plant; a chosen row's token gets, in its parent's target row, the logit that
gives it 0.8 of the softmax mass at temperature 1 (so it is the argmax).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np

# Sub-stream ids: one independent PCG64 stream per tensor family.
_S_DRAFT, _S_TARGET, _S_PLANT, _S_CTX, _S_ROOT = 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    vocab: int
    depth: int
    topk: int
    m: int
    n: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    layers: int
    batch: int
    ctx: int                       # fixed context length (ignored when ctx_range is set)
    ctx_range: Optional[Tuple[int, int]]  # inclusive uniform range for ragged batches
    dtype: str                     # "f32" or "bf16" storage of Q/K/V/O
    draft_sigma: float
    target_sigma: float
    temperatures: Tuple[float, ...]  # 0.0 means greedy
    plant_frac: float
    seed: int

    # ---- shapes implied by the tree parameters -------------------------
    def frontier_sizes(self) -> list:
        """Number of draft-logit rows consumed at each layer 1..depth."""
        sizes, f = [], 1
        for _ in range(self.depth):
            sizes.append(f)
            f = min(self.m, f * self.topk)
        return sizes

    @property
    def draft_rows(self) -> int:
        return sum(self.frontier_sizes())

    @property
    def capacity(self) -> int:
        """Tree nodes incl. the root after all layers are grown."""
        return 1 + self.topk * sum(self.frontier_sizes())

    @property
    def T(self) -> int:
        """Flattened tree rows: kept nodes plus the root."""
        return self.n + 1

    def ctx_lens(self) -> np.ndarray:
        if self.ctx_range is None:
            return np.full(self.batch, self.ctx, dtype=np.int32)
        rng = _rng(self.seed, _S_CTX)
        lo, hi = self.ctx_range
        return rng.integers(lo, hi + 1, size=self.batch, dtype=np.int64).astype(np.int32)

    def kv_row_offsets(self) -> Tuple[np.ndarray, int]:
        """First cache row of each sequence in the packed [Hkv][rows][D] cache."""
        lens = self.ctx_lens().astype(np.int64) + self.T
        off = np.zeros(self.batch, dtype=np.int64)
        off[1:] = np.cumsum(lens)[:-1]
        return off, int(lens.sum())

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # Tiny fp32 single verify step.
    "tiny_f32": Workload("tiny_f32", vocab=1000, depth=4, topk=4, m=4, n=15,
                         n_q_heads=4, n_kv_heads=4, head_dim=64, layers=1, batch=1,
                         ctx=256, ctx_range=None, dtype="f32", draft_sigma=2.0,
                         target_sigma=2.0, temperatures=(0.0,), plant_frac=0.0, seed=1001),
    # LLaMA2-7B-shaped single layer, greedy, half the nodes planted.
    "llama2_7b_layer": Workload("llama2_7b_layer", vocab=32000, depth=6, topk=10, m=10, n=60,
                                n_q_heads=32, n_kv_heads=32, head_dim=128, layers=1, batch=1,
                                ctx=2048, ctx_range=None, dtype="bf16", draft_sigma=3.0,
                                target_sigma=2.0, temperatures=(0.0,), plant_frac=0.5, seed=1002),
    # LLaMA2-13B-shaped full 40-layer verify step, sampled at temperature 1.
    "llama2_13b": Workload("llama2_13b", vocab=32000, depth=6, topk=10, m=10, n=60,
                           n_q_heads=40, n_kv_heads=40, head_dim=128, layers=40, batch=1,
                           ctx=4096, ctx_range=None, dtype="bf16", draft_sigma=3.0,
                           target_sigma=2.0, temperatures=(1.0,), plant_frac=0.5, seed=1003),
    # LLaMA2-70B-shaped GQA (64 query / 8 KV heads), 80 layers, greedy and T=0.7.
    "llama2_70b_gqa": Workload("llama2_70b_gqa", vocab=32000, depth=6, topk=10, m=10, n=60,
                               n_q_heads=64, n_kv_heads=8, head_dim=128, layers=80, batch=1,
                               ctx=8192, ctx_range=None, dtype="bf16", draft_sigma=3.0,
                               target_sigma=2.0, temperatures=(0.0, 0.7), plant_frac=0.5, seed=1004),
    # 16 ragged 13B-shaped sequences, each with its own tree, T=1.0.
    "batched_13b": Workload("batched_13b", vocab=32000, depth=7, topk=8, m=8, n=60,
                            n_q_heads=40, n_kv_heads=40, head_dim=128, layers=40, batch=16,
                            ctx=0, ctx_range=(512, 16384), dtype="bf16", draft_sigma=3.0,
                            target_sigma=2.0, temperatures=(1.0,), plant_frac=0.5, seed=1005),
    # The largest batch the library takes: 1024 sequences, each a small tree (T = 9) over
    # a short context (0-60 tokens), one layer of 4 heads (four attention launches of
    # 256 sequences).
    "batch1024_small": Workload("batch1024_small", vocab=300, depth=3, topk=3, m=2, n=8,
                                n_q_heads=4, n_kv_heads=4, head_dim=128, layers=1, batch=1024,
                                ctx=0, ctx_range=(0, 60), dtype="bf16", draft_sigma=2.0,
                                target_sigma=2.0, temperatures=(0.0,), plant_frac=0.5, seed=1006),
}
CONFIG_ORDER = ["tiny_f32", "llama2_7b_layer", "llama2_13b", "llama2_70b_gqa", "batched_13b"]


def _rng(seed: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, *extra])))


def draft_logits(w: Workload) -> np.ndarray:
    """fp32 [B][R][V] draft logits, N(0, draft_sigma)."""
    rng = _rng(w.seed, _S_DRAFT)
    x = rng.standard_normal((w.batch, w.draft_rows, w.vocab), dtype=np.float32)
    x *= np.float32(w.draft_sigma)
    return x


def draft_layer_slices(w: Workload) -> list:
    """(row_begin, row_end) of each layer inside the R axis of draft_logits."""
    out, r = [], 0
    for f in w.frontier_sizes():
        out.append((r, r + f))
        r += f
    return out


def root_tokens(w: Workload) -> np.ndarray:
    rng = _rng(w.seed, _S_ROOT)
    return rng.integers(0, w.vocab, size=w.batch, dtype=np.int64).astype(np.int32)


def target_logits_base(w: Workload, T: Optional[int] = None) -> np.ndarray:
    """fp32 [B][T][V] target logits, N(0, target_sigma), before planting."""
    T = w.T if T is None else T
    rng = _rng(w.seed, _S_TARGET)
    x = rng.standard_normal((w.batch, T, w.vocab), dtype=np.float32)
    x *= np.float32(w.target_sigma)
    return x


def plant(target: np.ndarray, flat_token: np.ndarray, flat_parent: np.ndarray,
          frac: float, seed: int, mass: float = 0.8) -> np.ndarray:
    """Return a planted copy of target [B][T][V] (see module docstring).

    flat_token / flat_parent are [B][T] int arrays describing the flattened
    tree (parent -1 for the root row).  Each planted row's token receives the
    logit that makes its softmax share equal to `mass` in its parent's row.
    """
    out = np.array(target, dtype=np.float32, copy=True)
    if frac <= 0.0:
        return out
    B, T, V = out.shape
    rng = _rng(seed, _S_PLANT)
    for b in range(B):
        planted_row = np.zeros(T, dtype=bool)
        draws = rng.random(T)
        for v in range(1, T):
            p = int(flat_parent[b, v])
            if p < 0 or planted_row[p] or draws[v] >= frac:
                continue
            tok = int(flat_token[b, v])
            row = out[b, p].astype(np.float64)
            others = np.delete(row, tok)
            # log-sum of the other tokens' weights, then odds mass/(1-mass)
            logrest = float(np.logaddexp.reduce(others))
            out[b, p, tok] = np.float32(logrest + math.log(mass / (1.0 - mass)))
            planted_row[p] = True
    return out


def attention_inputs(w: Workload, layer: int, device="cpu", ctx_lens: Optional[np.ndarray] = None):
    """Q [B][T][Hq][D], K and V [Hkv][rows][D] for one layer, N(0, 1).

    Returns (q, k, v, kv_row_off [B] int64 numpy, rows_total).  The cache
    holds, for each sequence, ctx_len context rows followed by its T tree rows.
    """
    import torch

    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    lens = w.ctx_lens() if ctx_lens is None else np.asarray(ctx_lens, dtype=np.int32)
    B = len(lens)
    rows = lens.astype(np.int64) + w.T
    off = np.zeros(B, dtype=np.int64)
    off[1:] = np.cumsum(rows)[:-1]
    total = int(rows.sum())
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 100003 + layer * 7 + 11)
    q = torch.randn((B, w.T, w.n_q_heads, w.head_dim), generator=g, device=device, dtype=dt)
    k = torch.randn((w.n_kv_heads, total, w.head_dim), generator=g, device=device, dtype=dt)
    v = torch.randn((w.n_kv_heads, total, w.head_dim), generator=g, device=device, dtype=dt)
    return q, k, v, off, total
