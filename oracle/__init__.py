"""CPU oracle for one EAGLE-2 draft-tree verification step -- TEST INFRASTRUCTURE.

Only the test suite, the package smoke check and the bench's CPU-baseline leg
may import this package.  The product path (the HIP library and its binding)
never does.  All arithmetic lives in ``eagle_oracle.cpp`` (plain single-threaded
C++); this module only marshals numpy arrays through ctypes and loops over the
sequences of a batch.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "eagle_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
BONUS_SLOT = -1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (single-threaded, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = C.CDLL(_LIB)
        P = C.c_void_p
        i32, u32, u64, f64, f32, i64 = C.c_int, C.c_uint32, C.c_uint64, C.c_double, C.c_float, C.c_longlong
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_uniform.argtypes = [u64, u64, u32, u32, u32]
        L.orc_uniform.restype = f64
        L.orc_tree_shape.argtypes = [i32, i32, i32, P, P]
        L.orc_expand.argtypes = [i32, i32, i32, i32, P, i32, P, P, P, P, P, P, P]
        L.orc_rerank.argtypes = [i32, P, P, i32, P]
        L.orc_flatten.argtypes = [i32, P, P, P, P, i32, i32, P, P, P, P, P, P]
        L.orc_attention.argtypes = [i32, i32, i32, i32, i32, P, P, P, i64, i64, P, f64, i32, P, P, P, P]
        L.orc_verify_greedy.argtypes = [i32, i32, P, P, P, i32, P, P, P]
        L.orc_verify_sampled.argtypes = [i32, i32, P, P, P, i32, f32, u64, u64, i32, P, P, P, P, i32, P]
        L.orc_flatten_static.argtypes = [i32, P, i32, P, P, P]
        L.orc_rope.argtypes = [i32, i32, i32, P, f64, P, P]
        L.orc_kv_commit.argtypes = [i32, i32, i32, P, i32, i64, i64, i64, P, P]
        L.orc_draft_subtree.argtypes = [i32, P, P, i32, P, i32, i32, P, P, P, P, P]
        for f in ("orc_tree_shape", "orc_expand", "orc_rerank", "orc_flatten", "orc_attention",
                  "orc_verify_greedy", "orc_verify_sampled", "orc_flatten_static", "orc_rope",
                  "orc_kv_commit", "orc_draft_subtree"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------
def philox4x32_10(ctr, key):
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def uniform(seed: int, step: int, seq: int, row: int, slot: int) -> float:
    return lib().orc_uniform(seed, step, seq, row, slot & 0xFFFFFFFF)


def tree_shape(depth: int, topk: int, m: int):
    f = np.zeros(depth, dtype=np.int32)
    cap = np.zeros(1, dtype=np.int32)
    rc = lib().orc_tree_shape(depth, topk, m, _p(f), _p(cap))
    if rc:
        raise ValueError("bad tree shape")
    return f, int(cap[0])


def expand(draft_logits, root_token: int, depth: int, topk: int, m: int):
    """One sequence: draft_logits [R][V] fp32.  Returns a dict of numpy arrays."""
    z = _c(draft_logits, np.float32)
    R, V = z.shape
    fs, cap = tree_shape(depth, topk, m)
    if int(fs.sum()) != R:
        raise ValueError(f"draft rows {R} != {int(fs.sum())} implied by the tree shape")
    tok = np.zeros(cap, np.int32); par = np.zeros(cap, np.int32)
    dep = np.zeros(cap, np.int32); val = np.zeros(cap, np.float32)
    lse = np.zeros(R, np.float64); haz = np.zeros(R, np.int32); nn = np.zeros(1, np.int32)
    rc = lib().orc_expand(V, depth, topk, m, _p(z), int(root_token), _p(tok), _p(par), _p(dep),
                          _p(val), _p(lse), _p(haz), _p(nn))
    if rc:
        raise ValueError("orc_expand rejected its arguments")
    n = int(nn[0])
    return dict(token=tok[:n], parent=par[:n], depth=dep[:n], value=val[:n], row_lse64=lse,
                row_hazard=haz, n_nodes=n)


def rerank(value, depth, n: int):
    v = _c(value, np.float32); d = _c(depth, np.int32)
    kept = np.zeros(n, np.int32)
    rc = lib().orc_rerank(len(v), _p(v), _p(d), n, _p(kept))
    if rc:
        raise ValueError("n exceeds the number of candidates")
    return kept


def flatten(tree: dict, kept, ctx_len: int):
    kept = _c(kept, np.int32)
    n = len(kept); T = n + 1
    tok = _c(tree["token"], np.int32); par = _c(tree["parent"], np.int32); dep = _c(tree["depth"], np.int32)
    out = {k: np.zeros(T, np.int32) for k in ("flat_node", "flat_token", "flat_parent", "flat_depth", "position")}
    mask = np.zeros((T, T), np.uint8)
    rc = lib().orc_flatten(len(tok), _p(tok), _p(par), _p(dep), _p(kept), n, int(ctx_len),
                           _p(out["flat_node"]), _p(out["flat_token"]), _p(out["flat_parent"]),
                           _p(out["flat_depth"]), _p(out["position"]), _p(mask))
    if rc:
        raise ValueError("kept set is not connected")
    out["mask"] = mask
    return out


def attention(q, k, v, mask, ctx_len: int, row0: int = 0, scale: float | None = None, sel=None):
    """One sequence.  q [T][Hq][D]; k, v [Hkv][rows][D] (any float dtype, widened
    exactly to fp32); mask [T][T] bool.  sel: optional list of (i, h) pairs.
    Returns (o, lse) in fp64: o [T][Hq][D] / lse [T][Hq], or [n_sel][D] / [n_sel]."""
    q = _c(q, np.float32); k = _c(k, np.float32); v = _c(v, np.float32)
    T, Hq, D = q.shape
    Hkv, rows, _ = k.shape
    mask = _c(mask, np.uint8)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if sel is None:
        n_sel, si, sh = -1, np.zeros(1, np.int32), np.zeros(1, np.int32)
        o = np.zeros((T, Hq, D)); lse = np.zeros((T, Hq))
    else:
        sel = np.asarray(sel, dtype=np.int32).reshape(-1, 2)
        n_sel = len(sel)
        si = _c(sel[:, 0], np.int32); sh = _c(sel[:, 1], np.int32)
        o = np.zeros((n_sel, D)); lse = np.zeros(n_sel)
    rc = lib().orc_attention(T, Hq, Hkv, D, int(ctx_len), _p(q), _p(k), _p(v), rows * D, int(row0),
                             _p(mask), float(scale), n_sel, _p(si), _p(sh), _p(o), _p(lse))
    if rc:
        raise ValueError("orc_attention rejected its arguments")
    return o, lse


def verify_greedy(target, flat_token, flat_parent, max_depth: int):
    z = _c(target, np.float32); T, V = z.shape
    ft = _c(flat_token, np.int32); fp = _c(flat_parent, np.int32)
    al = np.zeros(1, np.int32); ap = np.zeros(max_depth, np.int32); ot = np.zeros(max_depth + 1, np.int32)
    lib().orc_verify_greedy(T, V, _p(z), _p(ft), _p(fp), max_depth, _p(al), _p(ap), _p(ot))
    return int(al[0]), ap, ot


def verify_sampled(target, flat_token, flat_parent, max_depth: int, temperature: float, seed: int,
                   step: int, seq: int, max_trace: int = 4096):
    z = _c(target, np.float32); T, V = z.shape
    ft = _c(flat_token, np.int32); fp = _c(flat_parent, np.int32)
    al = np.zeros(1, np.int32); ap = np.zeros(max_depth, np.int32); ot = np.zeros(max_depth + 1, np.int32)
    tr = np.zeros((max_trace, 4)); nt = np.zeros(1, np.int32)
    rc = lib().orc_verify_sampled(T, V, _p(z), _p(ft), _p(fp), max_depth, float(temperature), seed, step,
                                  seq, _p(al), _p(ap), _p(ot), _p(tr), max_trace, _p(nt))
    if rc:
        raise ValueError("temperature must be > 0")
    return int(al[0]), ap, ot, tr[: min(int(nt[0]), max_trace)]


def flatten_static(parent, ctx_len: int):
    """Caller-given flattened tree: parent [T] (parent[0] = -1, parent[i] < i).
    Returns dict(flat_depth, position, mask [T][T] uint8)."""
    par = _c(parent, np.int32); T = len(par)
    dep = np.zeros(T, np.int32); pos = np.zeros(T, np.int32); mask = np.zeros((T, T), np.uint8)
    if lib().orc_flatten_static(T, _p(par), int(ctx_len), _p(dep), _p(pos), _p(mask)):
        raise ValueError("parent array is not a flattened tree")
    return dict(flat_depth=dep, position=pos, mask=mask)


def rope(x, positions, base: float = 10000.0):
    """Half-split rotary of x [rows][H][D] (widened exactly to fp32) at positions
    [rows]; returns fp64 [rows][H][D]."""
    xf = _c(x, np.float32); rows, H, D = xf.shape
    pos = _c(positions, np.int32)
    out = np.zeros((rows, H, D))
    if lib().orc_rope(rows, H, D, _p(pos), float(base), _p(xf), _p(out)):
        raise ValueError("head_dim must be even")
    return out


def kv_commit(cache, ctx_len: int, T: int, accept_len: int, path, row0: int = 0):
    """One sequence, one cache array [heads][rows][D] of any dtype, updated in place.
    Returns the new context length."""
    assert cache.flags["C_CONTIGUOUS"]
    H, rows = cache.shape[0], cache.shape[1]
    row_bytes = cache.strides[1]
    pa = _c(np.asarray(path)[:max(accept_len, 0)], np.int32)
    if pa.size == 0:
        pa = np.zeros(1, np.int32)
    nc = np.zeros(1, np.int32)
    if lib().orc_kv_commit(int(T), int(ctx_len), int(accept_len), _p(pa), H, rows, int(row0), row_bytes,
                           cache.ctypes.data_as(C.c_void_p), _p(nc)):
        raise ValueError("accepted path is not a strictly increasing run of tree rows")
    return int(nc[0])


def draft_subtree(tree: dict, frontier, ctx_len: int, T_sub: int):
    """Rows of the draft-side attention for one sequence's frontier: dict(sub_node,
    sub_parent, position [T_sub], mask [T_sub][T_sub] uint8, query_row [len(frontier)])."""
    par = _c(tree["parent"], np.int32); dep = _c(tree["depth"], np.int32)
    fr = _c(frontier, np.int32)
    out = {k: np.zeros(T_sub, np.int32) for k in ("sub_node", "sub_parent", "position")}
    mask = np.zeros((T_sub, T_sub), np.uint8)
    qr = np.zeros(max(len(fr), 1), np.int32)
    if lib().orc_draft_subtree(len(par), _p(par), _p(dep), len(fr), _p(fr), int(ctx_len), int(T_sub),
                               _p(out["sub_node"]), _p(out["sub_parent"]), _p(out["position"]), _p(mask), _p(qr)):
        raise ValueError("the frontier's root paths do not fit T_sub rows, or a frontier id is not a node")
    out["mask"] = mask
    out["query_row"] = qr[:len(fr)]
    return out


# ---------------------------------------------------------------------------
# Whole step for one sequence: tree -> rerank -> flatten (no attention).
def build_tree(draft_logits, root_token: int, depth: int, topk: int, m: int, n: int, ctx_len: int):
    tree = expand(draft_logits, root_token, depth, topk, m)
    kept = rerank(tree["value"], tree["depth"], n)
    flat = flatten(tree, kept, ctx_len)
    return tree, kept, flat
