"""One draft-tree verification step driven through the C ABI.

`VerifyStep` owns the device buffers of one workload (synthetic inputs from
`workload`) and enqueues, on the current stream:
    eagle_tree_expand x depth -> eagle_tree_rerank -> eagle_tree_mask
    -> eagle_tree_attention x layers -> eagle_verify
It performs no arithmetic of its own.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import binding as eb
from . import workload as wl


class VerifyStep:
    def __init__(self, w: wl.Workload, device: str = "cuda", layers: Optional[int] = None,
                 draft: Optional[np.ndarray] = None, root: Optional[np.ndarray] = None,
                 ctx_lens: Optional[np.ndarray] = None, with_lse: bool = True, host_lengths: bool = True):
        """host_lengths: also hand the attention call host copies of the context lengths
        and cache row offsets (the library then passes them as launch arguments)."""
        self.w = w
        self.device = device
        B, T, V = w.batch, w.T, w.vocab
        self.cfg = eb.make_cfg(B, V, w.depth, w.topk, w.m, w.n)
        self.cap = eb.eagle_tree_capacity(self.cfg)
        if self.cap != w.capacity:
            raise ValueError("capacity mismatch between library and workload shapes")
        i32 = dict(dtype=torch.int32, device=device)
        self.state = eb.TreeState.allocate(self.cfg, device)
        ews = eb.eagle_tree_expand_workspace(self.cfg)
        self.expand_ws = torch.zeros(max(ews, 1), dtype=torch.uint8, device=device)
        self.kept = torch.zeros((B, max(w.n, 1)), **i32)
        lens = w.ctx_lens() if ctx_lens is None else np.asarray(ctx_lens, dtype=np.int32)
        self.ctx_lens_np = lens
        self.ctx_len = torch.from_numpy(lens.astype(np.int32)).to(device)
        self.flat_token = torch.zeros((B, T), **i32)
        self.flat_parent = torch.zeros((B, T), **i32)
        self.flat_depth = torch.zeros((B, T), **i32)
        self.position = torch.zeros((B, T), **i32)
        self.mask = torch.zeros((B, T), dtype=torch.int64, device=device)
        # draft logits, one contiguous device tensor per layer: [B][F_l][V]
        d = wl.draft_logits(w) if draft is None else draft
        self.draft_np = d
        self.draft_layers = [torch.from_numpy(np.ascontiguousarray(d[:, a:b])).to(device)
                             for a, b in wl.draft_layer_slices(w)]
        r = wl.root_tokens(w) if root is None else root
        self.root_np = np.asarray(r, dtype=np.int32)
        self.root = torch.from_numpy(self.root_np).to(device)
        # attention, one set of buffers per layer
        rows = lens.astype(np.int64) + T
        off = np.zeros(B, dtype=np.int64)
        off[1:] = np.cumsum(rows)[:-1]
        total = int(rows.sum())
        self.n_layers = w.layers if layers is None else layers
        self.attn = []
        for layer in range(self.n_layers):
            q, k, v, off_l, total_l = wl.attention_inputs(w, layer, device=device, ctx_lens=lens)
            assert total_l == total and np.array_equal(off_l, off)
            self.attn.append(dict(q=q, k=k, v=v, o=torch.empty_like(q),
                                  lse=torch.empty((B, T, w.n_q_heads), dtype=torch.float32, device=device)
                                  if with_lse else None))
        self.kv_off_np = off
        self.kv_rows_total = total
        self.kv_row_off = torch.from_numpy(off).to(device)
        dtype = eb.EAGLE_F32 if w.dtype == "f32" else eb.EAGLE_BF16
        self.desc = eb.make_attn_desc(dtype, B, T, w.n_q_heads, w.n_kv_heads, w.head_dim, self.ctx_len,
                                      self.kv_row_off, total,
                                      ctx_len_host=lens if host_lengths else None,
                                      kv_row_off_host=off if host_lengths else None)
        ws = eb.eagle_tree_attention_workspace(self.desc)
        self.attn_ws = torch.zeros(max(ws, 1), dtype=torch.uint8, device=device)
        # verification
        self.target = torch.zeros((B, T, V), dtype=torch.float32, device=device)
        self.accept_len = torch.zeros((B,), **i32)
        self.accept_path = torch.zeros((B, w.depth), **i32)
        self.out_tokens = torch.zeros((B, w.depth + 1), **i32)
        vws = eb.eagle_verify_workspace(self.cfg)
        self.verify_ws = torch.zeros(max(vws, 1), dtype=torch.uint8, device=device)

    # ---- stages -----------------------------------------------------------
    def tree(self, stream=None):
        for layer in range(1, self.w.depth + 1):
            eb.eagle_tree_expand(self.cfg, layer, self.draft_layers[layer - 1], self.root, self.state,
                                 self.expand_ws, stream)
        if self.w.n > 0:
            eb.eagle_tree_rerank(self.cfg, self.state, self.kept, stream)
        eb.eagle_tree_mask(self.cfg, self.state, self.kept, self.ctx_len, self.flat_token, self.flat_parent,
                           self.flat_depth, self.position, self.mask, stream)

    def attention(self, layers: Optional[Sequence[int]] = None, stream=None):
        for layer in (range(self.n_layers) if layers is None else layers):
            a = self.attn[layer]
            eb.eagle_tree_attention(self.desc, a["q"], a["k"], a["v"], self.mask, a["o"], a["lse"],
                                    self.attn_ws, stream)

    def attention_rope(self, layers: Optional[Sequence[int]] = None, base: float = 10000.0, stream=None):
        """Tree attention with the rotary at the tree positions applied inside it (q and
        the K tree rows given unrotated; the cache's tree rows are left rotated)."""
        for layer in (range(self.n_layers) if layers is None else layers):
            a = self.attn[layer]
            eb.eagle_tree_attention_rope(self.desc, self.position, base, a["q"], a["k"], a["v"], self.mask, a["o"],
                                         a["lse"], self.attn_ws, stream)

    def verify(self, temperature: float, seed: int, step: int, stream=None):
        eb.eagle_verify(self.cfg, self.target, self.flat_token, self.flat_parent, temperature, seed, step,
                        self.accept_len, self.accept_path, self.out_tokens, self.verify_ws, stream)

    def rope(self, layers: Optional[Sequence[int]] = None, base: float = 10000.0, stream=None):
        """Rotary at the tree positions, in place on each layer's q and K tree rows."""
        for layer in (range(self.n_layers) if layers is None else layers):
            a = self.attn[layer]
            eb.eagle_tree_rope(self.desc, self.position, base, a["q"], a["k"], stream)

    def commit(self, stream=None):
        """Move the accepted rows' K/V of every layer behind the context
        (accept_len / accept_path from the last verify)."""
        if not hasattr(self, "new_ctx_len"):
            self.new_ctx_len = torch.zeros_like(self.ctx_len)
            dtype = eb.EAGLE_F32 if self.w.dtype == "f32" else eb.EAGLE_BF16
            self.commit_desc = eb.make_commit_desc(dtype, self.w.batch, self.w.T, self.w.depth, self.w.n_kv_heads,
                                                   self.w.head_dim, self.n_layers, self.ctx_len, self.kv_row_off,
                                                   self.kv_rows_total)
        eb.eagle_kv_commit(self.commit_desc, self.accept_len, self.accept_path, [a["k"] for a in self.attn],
                           [a["v"] for a in self.attn], self.new_ctx_len, stream)

    def run(self, temperature: float, seed: int, step: int, stream=None):
        self.tree(stream)
        self.attention(stream=stream)
        self.verify(temperature, seed, step, stream)

    # ---- inputs that depend on the tree -------------------------------------
    def set_target(self, target: np.ndarray):
        self.target.copy_(torch.from_numpy(np.ascontiguousarray(target, dtype=np.float32)))

    def flat_host(self):
        return (self.flat_token.cpu().numpy(), self.flat_parent.cpu().numpy())
