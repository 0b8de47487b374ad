"""Thin ctypes binding over libeagle_tree.so (the C ABI in include/eagle_tree.h).

Argument marshalling only: torch tensors supply device pointers and the current
HIP stream; every step of the verification path runs in the library's kernels.
There is no fallback: if the library is missing, importing raises.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libeagle_tree.so")

EAGLE_OK, EAGLE_ERR_INVALID_ARG, EAGLE_ERR_UNSUPPORTED, EAGLE_ERR_WORKSPACE, EAGLE_ERR_HIP = 0, -1, -2, -3, -4
EAGLE_F32, EAGLE_BF16 = 0, 1
MAX_TREE_ROWS = 64


class EagleError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


class TreeCfg(C.Structure):
    _fields_ = [("batch", C.c_int32), ("vocab", C.c_int32), ("depth", C.c_int32),
                ("topk", C.c_int32), ("m", C.c_int32), ("n", C.c_int32)]


class TreeStateC(C.Structure):
    _fields_ = [("token", C.c_void_p), ("parent", C.c_void_p), ("depth", C.c_void_p),
                ("value", C.c_void_p), ("frontier", C.c_void_p), ("n_nodes", C.c_void_p)]


class AttnDesc(C.Structure):
    _fields_ = [("dtype", C.c_int), ("batch", C.c_int32), ("T", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ctx_len", C.c_void_p),
                ("kv_row_off", C.c_void_p), ("kv_rows_total", C.c_int64), ("scale", C.c_float),
                ("ctx_len_host", C.c_void_p), ("kv_row_off_host", C.c_void_p)]


class CommitDesc(C.Structure):
    _fields_ = [("dtype", C.c_int), ("batch", C.c_int32), ("T", C.c_int32), ("depth", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("n_layers", C.c_int32),
                ("ctx_len", C.c_void_p), ("kv_row_off", C.c_void_p), ("kv_rows_total", C.c_int64)]


def load_library(path: str = _LIB_PATH) -> C.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    L = C.CDLL(path)
    P, i32, u64, sz = C.c_void_p, C.c_int32, C.c_uint64, C.c_size_t
    L.eagle_tree_capacity.argtypes = [P]; L.eagle_tree_capacity.restype = i32
    L.eagle_tree_frontier_rows.argtypes = [P, i32]; L.eagle_tree_frontier_rows.restype = i32
    L.eagle_tree_expand_workspace.argtypes = [P]; L.eagle_tree_expand_workspace.restype = sz
    L.eagle_tree_expand.argtypes = [P, i32, P, P, P, P, sz, P]; L.eagle_tree_expand.restype = C.c_int
    L.eagle_tree_rerank.argtypes = [P, P, P, P]; L.eagle_tree_rerank.restype = C.c_int
    L.eagle_tree_mask.argtypes = [P, P, P, P, P, P, P, P, P, P]; L.eagle_tree_mask.restype = C.c_int
    L.eagle_tree_attention_workspace.argtypes = [P]; L.eagle_tree_attention_workspace.restype = sz
    L.eagle_tree_attention.argtypes = [P, P, P, P, P, P, P, P, sz, P]; L.eagle_tree_attention.restype = C.c_int
    L.eagle_tree_attention_rope.argtypes = [P, P, C.c_double, P, P, P, P, P, P, P, sz, P]
    L.eagle_tree_attention_rope.restype = C.c_int
    L.eagle_tree_attention_noalloc.argtypes = [P, P, P, P, P, P, P, P]
    L.eagle_tree_attention_noalloc.restype = C.c_int
    L.eagle_verify_workspace.argtypes = [P]; L.eagle_verify_workspace.restype = sz
    L.eagle_verify.argtypes = [P, P, P, P, C.c_float, u64, u64, P, P, P, P, sz, P]
    L.eagle_verify.restype = C.c_int
    L.eagle_tree_mask_static.argtypes = [i32, i32, P, P, P, P, P, P]; L.eagle_tree_mask_static.restype = C.c_int
    L.eagle_tree_rope.argtypes = [P, P, C.c_double, P, P, P]; L.eagle_tree_rope.restype = C.c_int
    L.eagle_kv_commit.argtypes = [P, P, P, P, P, P, P]; L.eagle_kv_commit.restype = C.c_int
    L.eagle_draft_subtree_rows.argtypes = [P, i32]; L.eagle_draft_subtree_rows.restype = i32
    L.eagle_draft_subtree.argtypes = [P, i32, P, P, P, P, P, P, P, P]; L.eagle_draft_subtree.restype = C.c_int
    L.eagle_kv_gather.argtypes = [P, P, C.c_int64, C.c_int64, P, P, P, P, P]; L.eagle_kv_gather.restype = C.c_int
    L.eagle_status_string.argtypes = [C.c_int]; L.eagle_status_string.restype = C.c_char_p
    return L


_lib = load_library()


def lib() -> C.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.eagle_status_string(status).decode()


def _check(fn: str, status: int):
    if status != EAGLE_OK:
        raise EagleError(fn, status)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_cfg(batch, vocab, depth, topk, m, n) -> TreeCfg:
    return TreeCfg(batch, vocab, depth, topk, m, n)


@dataclass
class TreeState:
    """Device tree arrays ([batch][capacity] each; frontier [batch][m])."""
    token: object
    parent: object
    depth: object
    value: object
    frontier: object
    n_nodes: object

    @classmethod
    def allocate(cls, cfg: TreeCfg, device="cuda"):
        import torch
        cap = eagle_tree_capacity(cfg)
        if cap < 0:
            raise EagleError("eagle_tree_capacity", EAGLE_ERR_INVALID_ARG)
        i32 = dict(dtype=torch.int32, device=device)
        return cls(torch.zeros((cfg.batch, cap), **i32), torch.zeros((cfg.batch, cap), **i32),
                   torch.zeros((cfg.batch, cap), **i32),
                   torch.zeros((cfg.batch, cap), dtype=torch.float32, device=device),
                   torch.zeros((cfg.batch, cfg.m), **i32), torch.zeros((cfg.batch,), **i32))

    def c_struct(self) -> TreeStateC:
        return TreeStateC(_ptr(self.token), _ptr(self.parent), _ptr(self.depth), _ptr(self.value),
                          _ptr(self.frontier), _ptr(self.n_nodes))


def make_attn_desc(dtype: int, batch: int, T: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                   ctx_len, kv_row_off, kv_rows_total: int, scale: float = 0.0,
                   ctx_len_host=None, kv_row_off_host=None) -> AttnDesc:
    """ctx_len / kv_row_off: device tensors.  ctx_len_host / kv_row_off_host: optional
    host copies (array-likes, converted to contiguous int32 / int64 arrays that the
    descriptor keeps alive)."""
    hc = ho = None
    if (ctx_len_host is None) != (kv_row_off_host is None):
        raise ValueError("give both host copies or neither")
    if ctx_len_host is not None:
        hc = np.ascontiguousarray(ctx_len_host, dtype=np.int32)
        ho = np.ascontiguousarray(kv_row_off_host, dtype=np.int64)
    d = AttnDesc(dtype, batch, T, n_q_heads, n_kv_heads, head_dim, _ptr(ctx_len), _ptr(kv_row_off),
                 int(kv_rows_total), float(scale),
                 hc.ctypes.data if hc is not None else None, ho.ctypes.data if ho is not None else None)
    d._host_copies = (hc, ho)
    return d


# ---------------------------------------------------------------------------
# The five calls of the C ABI, same names.
# ---------------------------------------------------------------------------
def eagle_tree_capacity(cfg: TreeCfg) -> int:
    return _lib.eagle_tree_capacity(C.byref(cfg))


def eagle_tree_frontier_rows(cfg: TreeCfg, layer: int) -> int:
    return _lib.eagle_tree_frontier_rows(C.byref(cfg), layer)


def eagle_tree_expand_workspace(cfg: TreeCfg) -> int:
    return _lib.eagle_tree_expand_workspace(C.byref(cfg))


def eagle_tree_expand(cfg: TreeCfg, layer: int, draft_logits, root_token, state: TreeState, workspace,
                      stream=None):
    st = state.c_struct()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("eagle_tree_expand", _lib.eagle_tree_expand(C.byref(cfg), layer, _ptr(draft_logits),
                                                       _ptr(root_token), C.byref(st), _ptr(workspace),
                                                       nbytes, _stream(stream)))


def eagle_tree_rerank(cfg: TreeCfg, state: TreeState, kept, stream=None):
    st = state.c_struct()
    _check("eagle_tree_rerank", _lib.eagle_tree_rerank(C.byref(cfg), C.byref(st), _ptr(kept), _stream(stream)))


def eagle_tree_mask(cfg: TreeCfg, state: TreeState, kept, ctx_len, flat_token, flat_parent, flat_depth,
                    position, mask, stream=None):
    st = state.c_struct()
    _check("eagle_tree_mask", _lib.eagle_tree_mask(C.byref(cfg), C.byref(st), _ptr(kept), _ptr(ctx_len),
                                                   _ptr(flat_token), _ptr(flat_parent), _ptr(flat_depth),
                                                   _ptr(position), _ptr(mask), _stream(stream)))


def eagle_tree_attention_workspace(desc: AttnDesc) -> int:
    return _lib.eagle_tree_attention_workspace(C.byref(desc))


def eagle_tree_attention(desc: AttnDesc, q, k_cache, v_cache, mask, o, lse, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("eagle_tree_attention", _lib.eagle_tree_attention(
        C.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(mask), _ptr(o), _ptr(lse),
        _ptr(workspace), nbytes, _stream(stream)))


def eagle_tree_attention_rope(desc: AttnDesc, position, base: float, q, k_cache, v_cache, mask, o, lse, workspace,
                              stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("eagle_tree_attention_rope", _lib.eagle_tree_attention_rope(
        C.byref(desc), _ptr(position), float(base), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(mask), _ptr(o),
        _ptr(lse), _ptr(workspace), nbytes, _stream(stream)))


def eagle_tree_attention_noalloc(desc: AttnDesc, q, k_cache, v_cache, mask, o, lse, stream=None):
    _check("eagle_tree_attention_noalloc", _lib.eagle_tree_attention_noalloc(
        C.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(mask), _ptr(o), _ptr(lse), _stream(stream)))


def eagle_verify_workspace(cfg: TreeCfg) -> int:
    return _lib.eagle_verify_workspace(C.byref(cfg))


def eagle_verify(cfg: TreeCfg, target_logits, flat_token, flat_parent, temperature: float, seed: int,
                 step: int, accept_len, accept_path, out_tokens, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("eagle_verify", _lib.eagle_verify(
        C.byref(cfg), _ptr(target_logits), _ptr(flat_token), _ptr(flat_parent), float(temperature),
        int(seed) & 0xFFFFFFFFFFFFFFFF, int(step) & 0xFFFFFFFFFFFFFFFF, _ptr(accept_len), _ptr(accept_path),
        _ptr(out_tokens), _ptr(workspace), nbytes, _stream(stream)))


# ---------------------------------------------------------------------------
# Around the step: static-tree mask, rotary at the tree positions, KV commit.
# ---------------------------------------------------------------------------
def eagle_tree_mask_static(batch: int, T: int, flat_parent, ctx_len, flat_depth, position, mask, stream=None):
    _check("eagle_tree_mask_static", _lib.eagle_tree_mask_static(
        int(batch), int(T), _ptr(flat_parent), _ptr(ctx_len), _ptr(flat_depth), _ptr(position), _ptr(mask),
        _stream(stream)))


def eagle_tree_rope(desc: AttnDesc, position, base: float, q, k_cache, stream=None):
    _check("eagle_tree_rope", _lib.eagle_tree_rope(C.byref(desc), _ptr(position), float(base), _ptr(q),
                                                   _ptr(k_cache), _stream(stream)))


def make_commit_desc(dtype: int, batch: int, T: int, depth: int, n_kv_heads: int, head_dim: int,
                     n_layers: int, ctx_len, kv_row_off, kv_rows_total: int) -> CommitDesc:
    return CommitDesc(dtype, batch, T, depth, n_kv_heads, head_dim, n_layers, _ptr(ctx_len), _ptr(kv_row_off),
                      int(kv_rows_total))


def eagle_kv_commit(desc: CommitDesc, accept_len, accept_path, k_layers, v_layers, new_ctx_len, stream=None):
    """k_layers / v_layers: sequences of device tensors (one cache per layer)."""
    n = len(k_layers)
    KA = (C.c_void_p * max(n, 1))(*[_ptr(t) for t in k_layers])
    VA = (C.c_void_p * max(n, 1))(*[_ptr(t) for t in v_layers])
    _check("eagle_kv_commit", _lib.eagle_kv_commit(C.byref(desc), _ptr(accept_len), _ptr(accept_path), KA, VA,
                                                   _ptr(new_ctx_len), _stream(stream)))


# ---------------------------------------------------------------------------
# Draft-side attention rows and the row gather into the KV cache.
# ---------------------------------------------------------------------------
def eagle_draft_subtree_rows(cfg: TreeCfg, layer: int) -> int:
    return _lib.eagle_draft_subtree_rows(C.byref(cfg), layer)


def eagle_draft_subtree(cfg: TreeCfg, layer: int, state: TreeState, ctx_len, sub_node, sub_parent, position, mask,
                        query_row, stream=None):
    st = state.c_struct()
    _check("eagle_draft_subtree", _lib.eagle_draft_subtree(
        C.byref(cfg), int(layer), C.byref(st), _ptr(ctx_len), _ptr(sub_node), _ptr(sub_parent), _ptr(position),
        _ptr(mask), _ptr(query_row), _stream(stream)))


def eagle_kv_gather(desc: AttnDesc, rows, src_rows_per_seq: int, src_rows_total: int, src_k, src_v, k_cache,
                    v_cache, stream=None):
    _check("eagle_kv_gather", _lib.eagle_kv_gather(
        C.byref(desc), _ptr(rows), int(src_rows_per_seq), int(src_rows_total), _ptr(src_k), _ptr(src_v),
        _ptr(k_cache), _ptr(v_cache), _stream(stream)))
