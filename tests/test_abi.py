"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and host-side validation returns the documented status codes
before anything is launched (these calls never reach a kernel)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eagle_tree.h")


@pytest.fixture(scope="module")
def eb():
    from draft_tree_verification_eagle_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\**\s+\**(eagle_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for f in ("eagle_tree_expand", "eagle_tree_rerank", "eagle_tree_mask", "eagle_tree_attention",
              "eagle_verify"):
        assert f in names


def test_library_exports_every_declared_symbol(eb):
    L = eb.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


def test_status_strings(eb):
    assert eb.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert eb.status_string(s) != "unknown status"


@pytest.mark.parametrize("name", ["tiny_f32", "llama2_7b_layer", "llama2_13b", "llama2_70b_gqa", "batched_13b"])
def test_tree_shape_helpers_match_workloads_and_oracle(eb, orc, name):
    from draft_tree_verification_eagle_amd import workload as wl
    w = wl.CONFIGS[name]
    cfg = eb.make_cfg(w.batch, w.vocab, w.depth, w.topk, w.m, w.n)
    assert eb.eagle_tree_capacity(cfg) == w.capacity
    fs, cap = orc.tree_shape(w.depth, w.topk, w.m)
    assert cap == w.capacity
    for layer in range(1, w.depth + 1):
        assert eb.eagle_tree_frontier_rows(cfg, layer) == fs[layer - 1] == w.frontier_sizes()[layer - 1]
    assert eb.eagle_tree_frontier_rows(cfg, 0) == -1
    assert eb.eagle_tree_frontier_rows(cfg, w.depth + 1) == -1


def test_capacities_from_the_tree_parameters(eb):
    # 1 + k + (d-1) m k when m <= k: 53, 511, 393 nodes for the three tree shapes
    assert eb.eagle_tree_capacity(eb.make_cfg(1, 1000, 4, 4, 4, 15)) == 53
    assert eb.eagle_tree_capacity(eb.make_cfg(1, 32000, 6, 10, 10, 60)) == 511
    assert eb.eagle_tree_capacity(eb.make_cfg(16, 32000, 7, 8, 8, 60)) == 393


FAKE = 0x1000  # never dereferenced: validation fails before any launch


def _state(eb):
    return eb.TreeStateC(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)


def test_expand_validation(eb):
    L = eb.lib()
    st = _state(eb)
    good = eb.make_cfg(1, 100, 3, 4, 4, 10)
    need = L.eagle_tree_expand_workspace(C.byref(good))
    assert need > 0
    call = lambda cfg, layer, logits=FAKE, root=FAKE, state=C.byref(st), ws=FAKE, nb=need: \
        L.eagle_tree_expand(C.byref(cfg), layer, logits, root, state, ws, nb, None)
    for bad, code in [
        (eb.make_cfg(1, 100, 0, 4, 4, 10), eb.EAGLE_ERR_INVALID_ARG),    # depth 0
        (eb.make_cfg(1, 100, 3, 0, 4, 10), eb.EAGLE_ERR_INVALID_ARG),    # topk 0
        (eb.make_cfg(1, 3, 3, 4, 4, 10), eb.EAGLE_ERR_INVALID_ARG),      # vocab < topk
        (eb.make_cfg(-1, 100, 3, 4, 4, 10), eb.EAGLE_ERR_INVALID_ARG),   # negative batch
        (eb.make_cfg(1, 100, 3, 4, 4, 64), eb.EAGLE_ERR_UNSUPPORTED),    # T = 65 > 64
        (eb.make_cfg(1, 100, 3, 33, 4, 10), eb.EAGLE_ERR_UNSUPPORTED),   # topk > 32
        (eb.make_cfg(1, 10000, 3, 32, 33, 10), eb.EAGLE_ERR_UNSUPPORTED),  # m*k > 1024
        (eb.make_cfg(1, 262145, 3, 4, 4, 10), eb.EAGLE_ERR_UNSUPPORTED),   # vocab > 262144
        (eb.make_cfg(1, 100, 2, 2, 2, 10), eb.EAGLE_ERR_INVALID_ARG),    # n > 6 candidates
    ]:
        assert call(bad, 1) == code
    assert call(good, 0) == eb.EAGLE_ERR_INVALID_ARG
    assert call(good, 4) == eb.EAGLE_ERR_INVALID_ARG
    assert call(good, 1, root=None) == eb.EAGLE_ERR_INVALID_ARG
    assert call(good, 1, state=None) == eb.EAGLE_ERR_INVALID_ARG
    nul = eb.TreeStateC(FAKE, 0, FAKE, FAKE, FAKE, FAKE)
    assert call(good, 2, state=C.byref(nul)) == eb.EAGLE_ERR_INVALID_ARG
    assert call(good, 1, ws=None) == eb.EAGLE_ERR_WORKSPACE
    assert call(good, 1, nb=need - 1) == eb.EAGLE_ERR_WORKSPACE
    empty = eb.make_cfg(0, 100, 3, 4, 4, 10)
    assert call(empty, 1, logits=None, ws=None, nb=0) == eb.EAGLE_OK


def test_expand_workspace_grows_with_vocab_batch_and_width(eb):
    L = eb.lib()
    ws = lambda *c: L.eagle_tree_expand_workspace(C.byref(eb.make_cfg(*c)))
    a = ws(1, 32000, 6, 10, 10, 60)
    assert a > 0
    assert ws(1, 64000, 6, 10, 10, 60) > a      # more vocabulary chunks
    assert ws(4, 32000, 6, 10, 10, 60) > a      # more sequences
    assert ws(1, 32000, 6, 10, 20, 60) > a      # more draft rows per layer
    assert ws(1, 262145, 6, 10, 10, 60) == 0    # unsupported configuration


def test_rerank_and_mask_validation(eb):
    L = eb.lib()
    st = _state(eb)
    good = eb.make_cfg(2, 100, 3, 4, 4, 10)
    assert L.eagle_tree_rerank(C.byref(good), C.byref(st), None, None) == eb.EAGLE_ERR_INVALID_ARG
    too_many = eb.make_cfg(2, 100, 1, 4, 4, 5)
    assert L.eagle_tree_rerank(C.byref(too_many), C.byref(st), FAKE, None) == eb.EAGLE_ERR_INVALID_ARG
    args = [FAKE] * 7
    for i in range(1, 7):
        a = list(args); a[i] = None
        assert L.eagle_tree_mask(C.byref(good), C.byref(st), *a, None) == eb.EAGLE_ERR_INVALID_ARG
    empty = eb.make_cfg(0, 100, 3, 4, 4, 10)
    assert L.eagle_tree_mask(C.byref(empty), C.byref(st), *args, None) == eb.EAGLE_OK


def _desc(eb, **kw):
    d = dict(dtype=eb.EAGLE_BF16, batch=1, T=61, n_q_heads=40, n_kv_heads=40, head_dim=128)
    d.update(kw)
    return eb.AttnDesc(d["dtype"], d["batch"], d["T"], d["n_q_heads"], d["n_kv_heads"], d["head_dim"],
                       FAKE, FAKE, kw.get("rows", 4157), kw.get("scale", 0.0))


def test_attention_validation(eb):
    L = eb.lib()
    ok = _desc(eb)
    need = L.eagle_tree_attention_workspace(C.byref(ok))
    assert need > 0
    call = lambda d, ws=FAKE, nb=need: L.eagle_tree_attention(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                                              ws, nb, None)
    assert call(_desc(eb, n_kv_heads=3)) == eb.EAGLE_ERR_INVALID_ARG        # 40 % 3 != 0
    assert call(_desc(eb, T=65)) == eb.EAGLE_ERR_UNSUPPORTED
    assert call(_desc(eb, T=0)) == eb.EAGLE_ERR_INVALID_ARG
    assert call(_desc(eb, head_dim=130)) == eb.EAGLE_ERR_UNSUPPORTED        # head_dim <= 128
    # other bf16 head sizes run the row-per-workgroup kernel, which needs no workspace
    assert L.eagle_tree_attention_workspace(C.byref(_desc(eb, head_dim=64))) == 0
    assert L.eagle_tree_attention_workspace(C.byref(_desc(eb, head_dim=96))) == 0
    assert call(_desc(eb, dtype=7)) == eb.EAGLE_ERR_INVALID_ARG
    assert call(_desc(eb, scale=-1.0)) == eb.EAGLE_ERR_INVALID_ARG
    assert call(_desc(eb, scale=float("nan"))) == eb.EAGLE_ERR_INVALID_ARG
    assert call(_desc(eb, rows=60)) == eb.EAGLE_ERR_INVALID_ARG             # rows < batch * T
    assert call(_desc(eb, batch=1025, rows=10 ** 6)) == eb.EAGLE_ERR_UNSUPPORTED
    # bf16 work split: units * (4 * (ceil(rows / 64) + batch) + 16 * batch) must stay
    # below 2^31 (40 units, batch 1: rows up to 64 * (2^31 / 40 - 20) / 4 fit)
    limit_tiles = ((1 << 31) // 40 - 20) // 4
    assert L.eagle_tree_attention_workspace(C.byref(_desc(eb, rows=64 * limit_tiles))) > 0
    assert L.eagle_tree_attention_workspace(C.byref(_desc(eb, rows=64 * limit_tiles + 64))) == 0
    assert call(_desc(eb, rows=64 * limit_tiles + 64)) == eb.EAGLE_ERR_UNSUPPORTED
    assert call(ok, None, need) == eb.EAGLE_ERR_WORKSPACE
    assert call(ok, FAKE, need - 1) == eb.EAGLE_ERR_WORKSPACE
    assert L.eagle_tree_attention(C.byref(ok), None, FAKE, FAKE, FAKE, FAKE, None, FAKE, need, None) == \
        eb.EAGLE_ERR_INVALID_ARG
    f32 = _desc(eb, dtype=eb.EAGLE_F32, head_dim=64)
    assert L.eagle_tree_attention_workspace(C.byref(f32)) == 0
    assert call(_desc(eb, dtype=eb.EAGLE_F32, head_dim=256)) == eb.EAGLE_ERR_UNSUPPORTED
    assert call(_desc(eb, batch=0, rows=0), None, 0) == eb.EAGLE_OK


def test_attention_host_length_checks(eb):
    """Host copies of ctx_len / kv_row_off: both or neither, and every sequence's
    rows inside the cache (checked by the descriptor validation, seen here through
    the workspace query, which returns 0 for a rejected descriptor)."""
    L = eb.lib()
    ws = lambda d: L.eagle_tree_attention_workspace(C.byref(d))
    mk = lambda lens, offs, rows, batch=None: eb.make_attn_desc(
        eb.EAGLE_BF16, len(lens) if batch is None else batch, 61, 40, 40, 128, None, None, rows,
        ctx_len_host=lens, kv_row_off_host=offs)
    assert ws(mk([4096], [0], 4157)) > 0
    assert ws(mk([4096], [0], 4156)) == 0                     # last tree row past the cache
    assert ws(mk([100, 200], [0, 161], 161 + 261)) > 0
    assert ws(mk([100, 200], [0, 162], 161 + 261)) == 0
    assert ws(mk([-1], [0], 4157)) == 0
    assert ws(mk([10], [-1], 4157)) == 0
    one = eb.make_attn_desc(eb.EAGLE_BF16, 1, 61, 40, 40, 128, None, None, 4157)
    keep = mk([4096], [0], 4157)
    one.ctx_len_host = keep.ctx_len_host                      # ctx_len_host without kv_row_off_host
    assert ws(one) == 0
    with pytest.raises(ValueError):
        eb.make_attn_desc(eb.EAGLE_BF16, 1, 61, 40, 40, 128, None, None, 4157, ctx_len_host=[1])


def test_attention_workspace_is_the_same_for_every_bf16_shape(eb):
    # two partial slots per workgroup of a launch, whatever the batch, heads or
    # context (launches of one call reuse them in stream order)
    L = eb.lib()
    a = L.eagle_tree_attention_workspace(C.byref(_desc(eb)))
    b = L.eagle_tree_attention_workspace(C.byref(_desc(eb, batch=16, rows=16 * 20000)))
    g = L.eagle_tree_attention_workspace(C.byref(_desc(eb, n_q_heads=64, n_kv_heads=8)))
    h = L.eagle_tree_attention_workspace(C.byref(_desc(eb, batch=1024, T=64, n_q_heads=64, n_kv_heads=1,
                                                       rows=1024 * 20000)))
    assert a == b == g == h
    assert a == 2 * 256 * 64 * 128 * 2 + 2 * 256 * 64 * 8


def test_verify_validation(eb):
    L = eb.lib()
    cfg = eb.make_cfg(1, 1000, 4, 4, 4, 15)
    need = L.eagle_verify_workspace(C.byref(cfg))
    assert need > 0
    call = lambda temp, ws=FAKE, nb=need: L.eagle_verify(C.byref(cfg), FAKE, FAKE, FAKE, temp, 1, 0,
                                                         FAKE, FAKE, FAKE, ws, nb, None)
    assert call(-0.5) == eb.EAGLE_ERR_INVALID_ARG
    assert call(float("nan")) == eb.EAGLE_ERR_INVALID_ARG
    assert call(float("inf")) == eb.EAGLE_ERR_INVALID_ARG
    assert call(1.0, None) == eb.EAGLE_ERR_WORKSPACE
    assert call(1.0, FAKE, need - 8) == eb.EAGLE_ERR_WORKSPACE
    assert L.eagle_verify(C.byref(cfg), None, FAKE, FAKE, 0.0, 1, 0, FAKE, FAKE, FAKE, FAKE, need, None) == \
        eb.EAGLE_ERR_INVALID_ARG


def test_static_mask_validation(eb):
    L = eb.lib()
    f = FAKE
    assert L.eagle_tree_mask_static(0, 5, f, f, f, f, f, None) == eb.EAGLE_OK  # empty batch: no launch
    assert L.eagle_tree_mask_static(-1, 5, f, f, f, f, f, None) == eb.EAGLE_ERR_INVALID_ARG
    assert L.eagle_tree_mask_static(2, 0, f, f, f, f, f, None) == eb.EAGLE_ERR_INVALID_ARG
    assert L.eagle_tree_mask_static(2, 65, f, f, f, f, f, None) == eb.EAGLE_ERR_UNSUPPORTED
    assert L.eagle_tree_mask_static(2, 5, None, f, f, f, f, None) == eb.EAGLE_ERR_INVALID_ARG
    assert L.eagle_tree_mask_static(2, 5, f, f, f, f, None, None) == eb.EAGLE_ERR_INVALID_ARG


def test_rope_validation(eb):
    L = eb.lib()
    f = FAKE

    def desc(**kw):
        a = dict(dtype=eb.EAGLE_BF16, batch=1, T=61, n_q_heads=40, n_kv_heads=40, head_dim=128, ctx_len=f,
                 kv_row_off=f, kv_rows_total=5000)
        a.update(kw)
        return eb.make_attn_desc(a["dtype"], a["batch"], a["T"], a["n_q_heads"], a["n_kv_heads"], a["head_dim"],
                                 None, None, a["kv_rows_total"])

    def call(d, pos=f, base=10000.0, q=f, k=f, ctx=f, off=f):
        d.ctx_len = ctx; d.kv_row_off = off
        return L.eagle_tree_rope(C.byref(d), pos, base, q, k, None)

    assert call(desc(), q=None, k=None) == eb.EAGLE_OK  # nothing to rotate
    assert call(desc(batch=0)) == eb.EAGLE_OK
    assert call(desc(head_dim=127)) == eb.EAGLE_ERR_INVALID_ARG
    assert call(desc(head_dim=258)) == eb.EAGLE_ERR_UNSUPPORTED
    assert call(desc(T=65)) == eb.EAGLE_ERR_UNSUPPORTED
    assert call(desc(dtype=7)) == eb.EAGLE_ERR_INVALID_ARG
    for base in (0.0, -1.0, float("inf"), float("nan")):
        assert call(desc(), base=base) == eb.EAGLE_ERR_INVALID_ARG
    assert call(desc(), pos=None) == eb.EAGLE_ERR_INVALID_ARG
    assert call(desc(), ctx=None) == eb.EAGLE_ERR_INVALID_ARG  # rotating K needs the cache rows
    assert L.eagle_tree_rope(None, f, 10000.0, f, f, None) == eb.EAGLE_ERR_INVALID_ARG


def test_kv_commit_validation(eb):
    L = eb.lib()
    f = FAKE
    ks = (C.c_void_p * 2)(0x2000, 0x3000)
    vs = (C.c_void_p * 2)(0x4000, 0x5000)

    def call(dtype=eb.EAGLE_BF16, batch=1, T=61, depth=6, hkv=40, D=128, layers=2, ctx=0x6000, off=0x7000,
             rows=5000, al=f, ap=f, k=ks, v=vs, out=f):
        d = eb.CommitDesc(dtype, batch, T, depth, hkv, D, layers, ctx, off, rows)
        return L.eagle_kv_commit(C.byref(d), al, ap, k, v, out, None)

    assert call(batch=0) == eb.EAGLE_OK
    assert call(batch=-1) == eb.EAGLE_ERR_INVALID_ARG
    assert call(T=0) == eb.EAGLE_ERR_INVALID_ARG
    assert call(depth=0) == eb.EAGLE_ERR_INVALID_ARG
    assert call(T=65) == eb.EAGLE_ERR_UNSUPPORTED
    assert call(depth=256) == eb.EAGLE_ERR_UNSUPPORTED
    assert call(D=124) == eb.EAGLE_ERR_UNSUPPORTED  # bf16 rows must be whole 16-byte chunks
    assert call(dtype=eb.EAGLE_F32, D=126) == eb.EAGLE_ERR_UNSUPPORTED  # fp32 rows: head_dim % 4
    assert call(D=264) == eb.EAGLE_ERR_UNSUPPORTED
    assert call(dtype=5) == eb.EAGLE_ERR_INVALID_ARG
    assert call(al=None) == eb.EAGLE_ERR_INVALID_ARG
    assert call(ap=None) == eb.EAGLE_ERR_INVALID_ARG
    assert call(out=None) == eb.EAGLE_ERR_INVALID_ARG
    assert call(out=0x6000) == eb.EAGLE_ERR_INVALID_ARG  # new_ctx_len may not alias ctx_len
    assert call(k=None) == eb.EAGLE_ERR_INVALID_ARG
    bad = (C.c_void_p * 2)(0x2000, 0x3008)  # not 16-byte aligned
    assert call(k=bad) == eb.EAGLE_ERR_INVALID_ARG
    nul = (C.c_void_p * 2)(0x2000, 0)
    assert call(v=nul) == eb.EAGLE_ERR_INVALID_ARG
    assert L.eagle_kv_commit(None, f, f, ks, vs, f, None) == eb.EAGLE_ERR_INVALID_ARG


def test_draft_subtree_rows_and_validation(eb):
    L = eb.lib()
    f = FAKE
    cfg = eb.make_cfg(1, 32000, 6, 10, 10, 60)
    assert [eb.eagle_draft_subtree_rows(cfg, l) for l in range(1, 7)] == [1, 11, 21, 31, 41, 51]
    cfg5 = eb.make_cfg(16, 32000, 7, 8, 8, 60)
    assert eb.eagle_draft_subtree_rows(cfg5, 7) == 49
    assert eb.eagle_draft_subtree_rows(cfg, 0) == -1 and eb.eagle_draft_subtree_rows(cfg, 7) == -1
    st = _state(eb)
    args = [f] * 6
    assert L.eagle_draft_subtree(C.byref(cfg), 0, C.byref(st), *args, None) == eb.EAGLE_ERR_INVALID_ARG
    assert L.eagle_draft_subtree(C.byref(cfg), 7, C.byref(st), *args, None) == eb.EAGLE_ERR_INVALID_ARG
    wide = eb.make_cfg(1, 2000, 3, 32, 32, 60)  # F_3 = 32: 1 + 32 * 2 = 65 rows
    assert eb.eagle_draft_subtree_rows(wide, 3) == 65
    assert L.eagle_draft_subtree(C.byref(wide), 3, C.byref(st), *args, None) == eb.EAGLE_ERR_UNSUPPORTED
    assert L.eagle_draft_subtree(C.byref(cfg), 2, C.byref(st), None, f, f, f, f, f, None) == eb.EAGLE_ERR_INVALID_ARG
    empty = eb.make_cfg(0, 32000, 6, 10, 10, 60)
    assert L.eagle_draft_subtree(C.byref(empty), 2, C.byref(st), *args, None) == eb.EAGLE_OK


def test_kv_gather_validation(eb):
    L = eb.lib()
    f = FAKE

    def call(dtype=eb.EAGLE_BF16, batch=1, T=51, D=128, per=511, total=511, rows=f, sk=0x2000, sv=0x3000,
             k=0x4000, v=0x5000, ctx=f, off=f):
        d = eb.make_attn_desc(dtype, batch, T, 40, 40, D, None, None, 5000)
        d.ctx_len = ctx; d.kv_row_off = off
        return L.eagle_kv_gather(C.byref(d), rows, per, total, sk, sv, k, v, None)

    assert call(batch=0) == eb.EAGLE_OK
    assert call(T=0) == eb.EAGLE_ERR_INVALID_ARG
    assert call(T=65) == eb.EAGLE_ERR_UNSUPPORTED
    assert call(D=120 + 4) == eb.EAGLE_ERR_UNSUPPORTED
    assert call(per=0) == eb.EAGLE_ERR_INVALID_ARG
    assert call(batch=2, total=600) == eb.EAGLE_ERR_INVALID_ARG  # fewer source rows than 2 x 511
    assert call(rows=None) == eb.EAGLE_ERR_INVALID_ARG
    assert call(sv=None) == eb.EAGLE_ERR_INVALID_ARG
    assert call(k=0x4008) == eb.EAGLE_ERR_INVALID_ARG
    assert call(ctx=None) == eb.EAGLE_ERR_INVALID_ARG


def test_noalloc_attention_validation(eb):
    """The no-workspace attention call rejects a shape whose partials exceed its
    array, and bad arguments, before any HIP call."""
    L = eb.lib()

    class Dev:
        def data_ptr(self):
            return 0x1000

    f = 0x1000
    # every accepted shape's partials fit the array (the workspace does not grow
    # with the shape), so the size check never rejects one
    d = eb.make_attn_desc(eb.EAGLE_BF16, 1024, 64, 1024, 1024, 128, Dev(), Dev(), 1024 * 4096)
    assert 0 < eb.eagle_tree_attention_workspace(d) <= (16 << 20)
    d2 = eb.make_attn_desc(eb.EAGLE_BF16, 1, 16, 8, 8, 128, Dev(), Dev(), 4096)
    assert L.eagle_tree_attention_noalloc(C.byref(d2), None, f, f, f, f, None, None) == eb.EAGLE_ERR_INVALID_ARG
    d3 = eb.make_attn_desc(eb.EAGLE_BF16, 1, 16, 8, 8, 130, Dev(), Dev(), 4096)
    assert L.eagle_tree_attention_noalloc(C.byref(d3), f, f, f, f, f, None, None) == eb.EAGLE_ERR_UNSUPPORTED
    d4 = eb.make_attn_desc(eb.EAGLE_BF16, 0, 16, 8, 8, 128, Dev(), Dev(), 4096)
    assert L.eagle_tree_attention_noalloc(C.byref(d4), f, f, f, f, f, None, None) == eb.EAGLE_OK  # empty batch


def test_attention_rope_validation(eb):
    """Tree attention with rotary: bf16 only, a position array and a positive
    finite base, and the checks of the plain attention call, before any HIP call."""
    L = eb.lib()

    class Dev:
        def data_ptr(self):
            return 0x1000

    f = 0x1000

    def call(d, pos=f, base=10000.0, q=f, k=f, v=f, mask=f, o=f, ws=f, nbytes=1 << 30):
        return L.eagle_tree_attention_rope(C.byref(d), pos, base, q, k, v, mask, o, None, ws, nbytes, None)

    d = eb.make_attn_desc(eb.EAGLE_BF16, 1, 61, 40, 40, 128, Dev(), Dev(), 4157)
    assert call(d, pos=None) == eb.EAGLE_ERR_INVALID_ARG
    for base in (0.0, -1.0, float("inf"), float("nan")):
        assert call(d, base=base) == eb.EAGLE_ERR_INVALID_ARG
    for arg in ("q", "k", "v", "mask", "o"):
        assert call(d, **{arg: None}) == eb.EAGLE_ERR_INVALID_ARG
    assert call(d, ws=None) == eb.EAGLE_ERR_WORKSPACE
    assert call(d, nbytes=16) == eb.EAGLE_ERR_WORKSPACE
    d32 = eb.make_attn_desc(eb.EAGLE_F32, 1, 61, 40, 40, 64, Dev(), Dev(), 4157)
    assert call(d32) == eb.EAGLE_ERR_UNSUPPORTED
    d96 = eb.make_attn_desc(eb.EAGLE_BF16, 1, 61, 8, 8, 96, Dev(), Dev(), 4157)
    assert call(d96) == eb.EAGLE_ERR_UNSUPPORTED
    d0 = eb.make_attn_desc(eb.EAGLE_BF16, 0, 61, 40, 40, 128, Dev(), Dev(), 4157)
    assert call(d0) == eb.EAGLE_OK  # empty batch
    assert L.eagle_tree_attention_rope(None, f, 10000.0, f, f, f, f, f, None, f, 1 << 30, None) == \
        eb.EAGLE_ERR_INVALID_ARG
