"""Guard bands around every buffer the library writes, on the GPU, through the C
ABI: each output, workspace and tree array is the middle of a larger allocation
whose 4 KiB on either side hold a canary byte pattern.  After the calls every
canary byte must be unchanged, and every result must equal, bit for bit, the same
call on ordinary (unguarded) buffers.

Covers the step (expand x depth, rerank, mask, attention with and without the
rotary inside it, the no-workspace attention, verify greedy and sampled) on the
13B shape and on the batched ragged shape, and the calls around it (static mask,
rotary, KV commit, draft subtree, KV gather).
"""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

GUARD = 4096      # bytes on each side (a multiple of 256: the interior keeps its alignment)
CANARY = 0xA5


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_tree_verification_eagle_amd import binding, step, workload
    return binding, step, workload


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Guarded:
    """A tensor of `shape` in the middle of a canary-filled allocation."""

    def __init__(self, shape, dtype, fill=None, device="cuda"):
        elt = torch.empty((), dtype=dtype).element_size()
        g = GUARD // elt
        n = int(np.prod(shape)) if len(shape) else 1
        self.raw = torch.empty(2 * g + n, dtype=dtype, device=device)
        self.raw.view(torch.uint8).fill_(CANARY)
        self.t = self.raw[g:g + n].view(shape)
        if fill is not None:
            if torch.is_tensor(fill):
                self.t.copy_(fill)
            else:
                self.t.fill_(fill)

    def intact(self):
        b = self.raw.view(torch.uint8)
        return bool((b[:GUARD] == CANARY).all()) and bool((b[-GUARD:] == CANARY).all())


def guarded_like(t, fill=None):
    return Guarded(tuple(t.shape), t.dtype, t if fill is None else fill)


def bits(t):
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    if t.dtype == torch.float64:
        return t.view(torch.int64)
    return t


def same(a, b):
    return torch.equal(bits(a), bits(b))


def guarded_state(eb, cfg):
    cap = eb.eagle_tree_capacity(cfg)
    i32 = torch.int32
    parts = dict(token=Guarded((cfg.batch, cap), i32, 0), parent=Guarded((cfg.batch, cap), i32, 0),
                 depth=Guarded((cfg.batch, cap), i32, 0), value=Guarded((cfg.batch, cap), torch.float32, 0),
                 frontier=Guarded((cfg.batch, cfg.m), i32, 0), n_nodes=Guarded((cfg.batch,), i32, 0))
    return eb.TreeState(**{k: v.t for k, v in parts.items()}), parts


def check_all(named):
    bad = [name for name, g in named.items() if not g.intact()]
    assert not bad, f"canary bytes changed around: {bad}"


@pytest.mark.parametrize("name", ["llama2_13b", "batched_13b"])
def test_step_guard_bands(lib, name):
    eb, stepm, wl = lib
    w = wl.CONFIGS[name]
    say(f"[guard bands] {name}: expand, rerank, mask, attention (+ rotary, no-workspace), verify")
    vs = stepm.VerifyStep(w, layers=1)           # the reference run on ordinary buffers
    vs.tree()
    B, T = w.batch, w.T
    g = {}
    state, parts = guarded_state(eb, vs.cfg)
    g.update({f"state.{k}": v for k, v in parts.items()})
    g["expand_ws"] = Guarded(tuple(vs.expand_ws.shape), torch.uint8, 0)
    for layer in range(1, w.depth + 1):
        eb.eagle_tree_expand(vs.cfg, layer, vs.draft_layers[layer - 1], vs.root, state, g["expand_ws"].t)
    g["kept"] = Guarded(tuple(vs.kept.shape), torch.int32, -7)
    if w.n > 0:
        eb.eagle_tree_rerank(vs.cfg, state, g["kept"].t)
    for nm in ("flat_token", "flat_parent", "flat_depth", "position"):
        g[nm] = Guarded((B, T), torch.int32, -7)
    g["mask"] = Guarded((B, T), torch.int64, -7)
    eb.eagle_tree_mask(vs.cfg, state, g["kept"].t, vs.ctx_len, g["flat_token"].t, g["flat_parent"].t,
                       g["flat_depth"].t, g["position"].t, g["mask"].t)
    torch.cuda.synchronize()
    for k in ("token", "parent", "depth", "value", "frontier", "n_nodes"):
        assert same(getattr(state, k), getattr(vs.state, k)), f"state.{k} differs"
    assert same(g["kept"].t, vs.kept)
    for nm in ("flat_token", "flat_parent", "flat_depth", "position", "mask"):
        assert same(g[nm].t, getattr(vs, nm)), f"{nm} differs"

    # attention: plain, with the rotary inside, without a workspace
    a = vs.attn[0]
    vs.attention()
    ws_n = vs.attn_ws.numel()
    for tag in ("plain", "rope", "noalloc"):
        g[f"o.{tag}"] = Guarded(tuple(a["o"].shape), a["o"].dtype, float("nan"))
        g[f"lse.{tag}"] = Guarded(tuple(a["lse"].shape), torch.float32, float("nan"))
    g["attn_ws"] = Guarded((ws_n,), torch.uint8, 0)
    eb.eagle_tree_attention(vs.desc, a["q"], a["k"], a["v"], g["mask"].t, g["o.plain"].t, g["lse.plain"].t,
                            g["attn_ws"].t)
    eb.eagle_tree_attention_noalloc(vs.desc, a["q"], a["k"], a["v"], g["mask"].t, g["o.noalloc"].t,
                                    g["lse.noalloc"].t)
    torch.cuda.synchronize()
    assert same(g["o.plain"].t, a["o"]) and same(g["lse.plain"].t, a["lse"])
    assert same(g["o.noalloc"].t, a["o"]) and same(g["lse.noalloc"].t, a["lse"])
    # the fused rotary writes the cache's tree K rows: run it on guarded copies of
    # the cache, against the same call on ordinary copies
    k_ref = a["k"].clone()
    o_ref = torch.empty_like(a["o"]); lse_ref = torch.empty_like(a["lse"])
    eb.eagle_tree_attention_rope(vs.desc, vs.position, 10000.0, a["q"], k_ref, a["v"], vs.mask, o_ref, lse_ref,
                                 vs.attn_ws)
    g["k_cache"] = guarded_like(a["k"])
    eb.eagle_tree_attention_rope(vs.desc, g["position"].t, 10000.0, a["q"], g["k_cache"].t, a["v"], g["mask"].t,
                                 g["o.rope"].t, g["lse.rope"].t, g["attn_ws"].t)
    torch.cuda.synchronize()
    assert same(g["o.rope"].t, o_ref) and same(g["lse.rope"].t, lse_ref) and same(g["k_cache"].t, k_ref)

    # verify, greedy and sampled
    rng = np.random.default_rng(3)
    target = rng.normal(0.0, 2.0, (B, T, w.vocab)).astype(np.float32)
    vs.set_target(target)
    d1 = w.depth + 1
    for temperature in (0.0, 1.0):
        vs.verify(temperature, 11, 5)
        for nm, shape in (("accept_len", (B,)), ("accept_path", (B, w.depth)), ("out_tokens", (B, d1))):
            g[f"{nm}.{temperature}"] = Guarded(shape, torch.int32, -7)
        g[f"verify_ws.{temperature}"] = Guarded((vs.verify_ws.numel(),), torch.uint8, 0)
        eb.eagle_verify(vs.cfg, vs.target, g["flat_token"].t, g["flat_parent"].t, temperature, 11, 5,
                        g[f"accept_len.{temperature}"].t, g[f"accept_path.{temperature}"].t,
                        g[f"out_tokens.{temperature}"].t, g[f"verify_ws.{temperature}"].t)
        torch.cuda.synchronize()
        assert same(g[f"accept_len.{temperature}"].t, vs.accept_len)
        assert same(g[f"accept_path.{temperature}"].t, vs.accept_path)
        assert same(g[f"out_tokens.{temperature}"].t, vs.out_tokens)
    check_all(g)
    say(f"  {len(g)} guarded buffers intact")


def test_calls_around_the_step_guard_bands(lib):
    eb, stepm, wl = lib
    w = wl.CONFIGS["llama2_13b"]
    say("[guard bands] static mask, rotary, KV commit (two layers), draft subtree, KV gather")
    vs = stepm.VerifyStep(w, layers=2)
    vs.tree()
    B, T = w.batch, w.T
    g = {}
    # static mask of the flattened tree
    for nm in ("flat_depth", "position"):
        g[f"static.{nm}"] = Guarded((B, T), torch.int32, -7)
    g["static.mask"] = Guarded((B, T), torch.int64, -7)
    eb.eagle_tree_mask_static(B, T, vs.flat_parent, vs.ctx_len, g["static.flat_depth"].t, g["static.position"].t,
                              g["static.mask"].t)
    torch.cuda.synchronize()
    assert same(g["static.flat_depth"].t, vs.flat_depth) and same(g["static.position"].t, vs.position)
    assert same(g["static.mask"].t, vs.mask)
    # rotary on guarded copies of q and K
    a = vs.attn[0]
    q_ref, k_ref = a["q"].clone(), a["k"].clone()
    eb.eagle_tree_rope(vs.desc, vs.position, 10000.0, q_ref, k_ref)
    g["rope.q"], g["rope.k"] = guarded_like(a["q"]), guarded_like(a["k"])
    eb.eagle_tree_rope(vs.desc, vs.position, 10000.0, g["rope.q"].t, g["rope.k"].t)
    torch.cuda.synchronize()
    assert same(g["rope.q"].t, q_ref) and same(g["rope.k"].t, k_ref)
    # KV commit of the deepest root path, two layers
    fp = vs.flat_parent.cpu().numpy()
    al = np.zeros(B, np.int32)
    ap = np.full((B, w.depth), -1, np.int32)
    for b in range(B):
        path, r = [], T - 1
        while r > 0:
            path.append(r); r = int(fp[b, r])
        path = path[::-1]
        al[b] = len(path); ap[b, :len(path)] = path
    vs.accept_len.copy_(torch.from_numpy(al)); vs.accept_path.copy_(torch.from_numpy(ap))
    ks = [guarded_like(x["k"]) for x in vs.attn]
    vv = [guarded_like(x["v"]) for x in vs.attn]
    g["commit.new_ctx"] = Guarded((B,), torch.int32, -7)
    vs.commit()
    cd = eb.make_commit_desc(eb.EAGLE_BF16, B, T, w.depth, w.n_kv_heads, w.head_dim, 2, vs.ctx_len, vs.kv_row_off,
                             vs.kv_rows_total)
    eb.eagle_kv_commit(cd, vs.accept_len, vs.accept_path, [x.t for x in ks], [x.t for x in vv],
                       g["commit.new_ctx"].t)
    torch.cuda.synchronize()
    for layer in range(2):
        assert same(ks[layer].t, vs.attn[layer]["k"]) and same(vv[layer].t, vs.attn[layer]["v"])
        g[f"commit.k{layer}"], g[f"commit.v{layer}"] = ks[layer], vv[layer]
    assert same(g["commit.new_ctx"].t, vs.new_ctx_len)
    # draft subtree at the last layer
    layer = w.depth
    Ts = eb.eagle_draft_subtree_rows(vs.cfg, layer)
    outs = {}
    for tag in ("ref", "guarded"):
        mk = (lambda shape, dt: Guarded(shape, dt, -7)) if tag == "guarded" else \
             (lambda shape, dt: type("P", (), {"t": torch.full(shape, -7, dtype=dt, device="cuda")})())
        o = dict(node=mk((B, Ts), torch.int32), par=mk((B, Ts), torch.int32), pos=mk((B, Ts), torch.int32),
                 msk=mk((B, Ts), torch.int64), qrow=mk((B, w.m), torch.int32))
        eb.eagle_draft_subtree(vs.cfg, layer, vs.state, vs.ctx_len, o["node"].t, o["par"].t, o["pos"].t,
                               o["msk"].t, o["qrow"].t)
        outs[tag] = o
    torch.cuda.synchronize()
    for k in outs["ref"]:
        assert same(outs["guarded"][k].t, outs["ref"][k].t), f"draft subtree {k} differs"
        g[f"subtree.{k}"] = outs["guarded"][k]
    # KV gather of the subtree rows' node K/V behind the context
    node = outs["ref"]["node"].t
    gen = torch.Generator(device="cuda").manual_seed(5)
    src_k = torch.randn((w.n_kv_heads, B * vs.cap, w.head_dim), generator=gen, device="cuda").to(torch.bfloat16)
    src_v = torch.randn((w.n_kv_heads, B * vs.cap, w.head_dim), generator=gen, device="cuda").to(torch.bfloat16)
    lens = vs.ctx_lens_np.astype(np.int64)
    off = np.zeros(B, np.int64); off[1:] = np.cumsum(lens + Ts)[:-1]
    total = int((lens + Ts).sum())
    off_t = torch.from_numpy(off).cuda()
    desc = eb.make_attn_desc(eb.EAGLE_BF16, B, Ts, w.n_q_heads, w.n_kv_heads, w.head_dim, vs.ctx_len, off_t, total)
    k_ref = torch.zeros((w.n_kv_heads, total, w.head_dim), dtype=torch.bfloat16, device="cuda")
    v_ref = torch.zeros_like(k_ref)
    eb.eagle_kv_gather(desc, node, vs.cap, B * vs.cap, src_k, src_v, k_ref, v_ref)
    g["gather.k"], g["gather.v"] = Guarded(tuple(k_ref.shape), torch.bfloat16, 0), Guarded(tuple(k_ref.shape),
                                                                                         torch.bfloat16, 0)
    eb.eagle_kv_gather(desc, node, vs.cap, B * vs.cap, src_k, src_v, g["gather.k"].t, g["gather.v"].t)
    torch.cuda.synchronize()
    assert same(g["gather.k"].t, k_ref) and same(g["gather.v"].t, v_ref)
    check_all(g)
    say(f"  {len(g)} guarded buffers intact")
