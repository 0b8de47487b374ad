"""Benchmark: tree-verify steps/sec and tree-attention HBM GB/s on one MI355X.

Workload (default): LLaMA2-13B-shaped verification step, batch 1 -- draft tree
of depth 6, top-k 10, m 10, Rerank to 60 nodes (T = 61 rows), vocab 32000;
tree attention through 40 layers of 40 heads x 128 with a bf16 KV cache at
context 4096 (40 distinct layer buffers, 3.46 GB, so nothing stays in the
256 MB last-level cache between layers); sampled verification at temperature 1
with Philox uniforms.  Inputs are seeded synthetic tensors of that shape.

One step = eagle_tree_expand x 6 + eagle_tree_rerank + eagle_tree_mask +
eagle_tree_attention x 40 + eagle_verify, enqueued on one stream.  Inputs are
resident in HBM before timing starts.

The JSON line carries:
  value     steps/s (whole job, one GPU)
  roofline  tree-attention HBM bandwidth: algorithmic bytes per launch (K + V of
            the ctx + T rows of every KV head, plus Q and O) / average launch
            time measured with HIP events on the launch stream, against the
            8 TB/s HBM peak.  A launch is one eagle_tree_attention call: the
            main kernel and its partial-merge kernel.  `traffic` (HBM bytes per
            launch from FETCH_SIZE / WRITE_SIZE counters, scaled by a copy of known
            size) is read from the committed counter summary when present.
  cpu_baseline  the CPU oracle on a bounded sample (tree + 12 attention layers +
            verify, single thread, about 10 s), scaled to one full step
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# HBM counter records, one per workload they were taken on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tree_attn_{}_traffic.json")


def attention_bytes_per_launch(w) -> int:
    """K + V over ctx + T rows per KV head, plus Q and O (bf16)."""
    elt = 4 if w.dtype == "f32" else 2
    kv = 0
    for c in w.ctx_lens():
        kv += 2 * w.n_kv_heads * (int(c) + w.T) * w.head_dim * elt
    qo = 2 * w.batch * w.T * w.n_q_heads * w.head_dim * elt
    return kv + qo


MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3        # fp32 vector


def attention_flops_per_launch(w, mask_words, ctx_lens) -> int:
    """QK^T and PV multiply-adds over the keys each tree row attends to (its
    context and its ancestors, itself included): 4 * D per (query head, key)."""
    total = 0
    for b in range(w.batch):
        keys = sum(int(ctx_lens[b]) + bin(int(x) & (2**64 - 1)).count("1") for x in mask_words[b])
        total += keys * w.n_q_heads * 4 * w.head_dim
    return total


# Host threads one GPU's job may use on the GPU machine (its CPU share), whatever the
# machine's core count.
HOST_THREAD_SHARE = 16


def host_cpu():
    """(logical CPUs the process may run on, CPU model string)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n, model


def _cpu_all_cores(w, mask, t_tree, t_verify):
    """The same oracle on the host cores this job may use: P threads (the logical
    CPUs available, capped at the per-GPU host share), each computing one distinct
    attention layer (the oracle is a C library; its calls run outside the GIL),
    wall time of the P layers, scaled to a full step."""
    import concurrent.futures as cf
    import oracle
    from draft_tree_verification_eagle_amd import workload as wl

    nproc, model = host_cpu()
    P = max(1, min(nproc, HOST_THREAD_SHARE, w.layers))
    inputs = []
    for layer in range(P):
        q, k, v, off, total = wl.attention_inputs(w, layer, device="cpu")
        inputs.append((q[0].float().numpy(), k.float().numpy(), v.float().numpy()))
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=P) as ex:
        list(ex.map(lambda x: oracle.attention(x[0], x[1], x[2], mask, w.ctx), inputs))
    t_par = time.perf_counter() - t0
    t_step = t_tree + w.layers * t_par / P + t_verify
    return {"value": 1.0 / t_step, "unit": "steps/s", "cores": P, "nproc": nproc, "cpu_model": model,
            "sample": f"{P} attention layers on {P} threads in {t_par:.2f}s wall, scaled to {w.layers} layers "
                      f"(tree and verification as in the one-thread figure); {nproc} logical CPUs available, "
                      f"threads capped at the {HOST_THREAD_SHARE}-thread host share of one GPU"}


def cpu_baseline(w, vs_draft, vs_root, target, temperature, seed, layers: int = 12):
    """Oracle timing on a bounded sample: full tree + `layers` distinct attention
    layers + one verification, single-threaded, scaled to the full step
    (tree + w.layers x mean layer time + verify)."""
    import oracle
    from draft_tree_verification_eagle_amd import workload as wl

    b = 0
    t0 = time.perf_counter()
    tree, kept, flat = oracle.build_tree(vs_draft[b], int(vs_root[b]), w.depth, w.topk, w.m, w.n, w.ctx)
    t_tree = time.perf_counter() - t0
    layers = max(1, min(layers, w.layers))
    t_layers = 0.0
    for layer in range(layers):
        q, k, v, off, total = wl.attention_inputs(w, layer, device="cpu")
        qf = q[0].float().numpy(); kf = k.float().numpy(); vf = v.float().numpy()
        t0 = time.perf_counter()
        oracle.attention(qf, kf, vf, flat["mask"], w.ctx)
        t_layers += time.perf_counter() - t0
    t_layer = t_layers / layers
    t0 = time.perf_counter()
    if temperature > 0:
        oracle.verify_sampled(target[b], flat["flat_token"], flat["flat_parent"], w.depth, temperature, seed, 0, 0)
    else:
        oracle.verify_greedy(target[b], flat["flat_token"], flat["flat_parent"], w.depth)
    t_verify = time.perf_counter() - t0
    t_step = t_tree + w.layers * t_layer + t_verify
    all_cores = _cpu_all_cores(w, flat["mask"], t_tree, t_verify)
    nproc, model = host_cpu()
    return {"value": 1.0 / t_step, "unit": "steps/s", "cores": 1, "kind": "oracle", "nproc": nproc,
            "cpu_model": model,
            "all_cores": all_cores,
            "sample": f"tree build + {layers} of {w.layers} attention layers (fp64, {t_layers:.1f}s) + 1 verification, "
                      f"one thread; step time = tree {t_tree:.3f}s + {w.layers} x layer {t_layer:.2f}s + verify "
                      f"{t_verify:.4f}s (the oracle evaluates only the rows its walk visits)",
            "oracle_attention_GBps": attention_bytes_per_launch(w) / t_layer / 1e9}


def measured_copy_gbs(mib: int = 256, reps: int = 5) -> float:
    """The box's streaming-copy bandwidth: a device-to-device copy of `mib` MiB,
    best of `reps` timed with HIP events, (read + write bytes) / time."""
    import torch
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    del src, dst
    return 2.0 * (mib << 20) / best / 1e9


def _graph_us(fn, reps):
    """Average GPU time of fn's launches: `reps` calls captured in one HIP graph
    and replayed, timed with HIP events on the replay stream (no host launch
    overhead between the kernels)."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def _time_draft_side(vs, w, stream, reps: int = 20):
    """Draft-side attention at the last draft layer: the rows of the frontier's root
    paths, the gather of their draft K/V behind a draft context of the same length
    and shape as the target's, and one tree-attention call over them (graph replays)."""
    import torch
    from draft_tree_verification_eagle_amd import binding as eb

    layer = w.depth
    T_sub = eb.eagle_draft_subtree_rows(vs.cfg, layer)
    dev = vs.ctx_len.device
    i32 = dict(dtype=torch.int32, device=dev)
    node = torch.empty((w.batch, T_sub), **i32); par = torch.empty((w.batch, T_sub), **i32)
    pos = torch.empty((w.batch, T_sub), **i32); qrow = torch.empty((w.batch, w.m), **i32)
    msk = torch.empty((w.batch, T_sub), dtype=torch.int64, device=dev)
    sub = lambda: eb.eagle_draft_subtree(vs.cfg, layer, vs.state, vs.ctx_len, node, par, pos, msk, qrow)
    subtree_us = _graph_us(sub, reps)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = torch.Generator(device=dev).manual_seed(7)
    Hkv, D = w.n_kv_heads, w.head_dim
    node_k = torch.randn((Hkv, w.batch * vs.cap, D), generator=g, device=dev).to(dt)
    node_v = torch.randn((Hkv, w.batch * vs.cap, D), generator=g, device=dev).to(dt)
    lens = vs.ctx_lens_np.astype(np.int64)
    off = np.zeros(w.batch, np.int64); off[1:] = np.cumsum(lens + T_sub)[:-1]
    total = int((lens + T_sub).sum())
    k = torch.randn((Hkv, total, D), generator=g, device=dev).to(dt)
    v = torch.randn((Hkv, total, D), generator=g, device=dev).to(dt)
    q = torch.randn((w.batch, T_sub, w.n_q_heads, D), generator=g, device=dev).to(dt)
    o = torch.empty_like(q)
    off_t = torch.from_numpy(off).to(dev)
    desc = eb.make_attn_desc(eb.EAGLE_BF16 if w.dtype == "bf16" else eb.EAGLE_F32, w.batch, T_sub, w.n_q_heads,
                             Hkv, D, vs.ctx_len, off_t, total, ctx_len_host=vs.ctx_lens_np, kv_row_off_host=off)
    ws = torch.zeros(max(eb.eagle_tree_attention_workspace(desc), 1), dtype=torch.uint8, device=dev)
    gather_us = _graph_us(lambda: eb.eagle_kv_gather(desc, node, vs.cap, w.batch * vs.cap, node_k, node_v, k, v),
                          reps)
    attn_us = _graph_us(lambda: eb.eagle_tree_attention(desc, q, k, v, msk, o, None, ws), reps)
    return {"layer": layer, "rows": T_sub, "subtree_us": round(subtree_us, 3), "gather_us": round(gather_us, 3),
            "attention_us": round(attn_us, 3),
            "what": "rows of the frontier's root paths, their draft K/V gathered behind a draft context of the "
                    "target's shape, one draft attention call"}


def time_extras(vs, w, stream, temperature, seed, reps: int = 20):
    """Rotary at the tree positions (one call per layer), KV commit of an accepted
    path (one call for all layers), the static-tree mask (graph replays, HIP
    events), and the whole decode step with rotary and commit included (eager)."""
    import torch
    from draft_tree_verification_eagle_amd import binding as eb

    print("[bench] timing rotary, KV commit, static mask", file=sys.stderr, flush=True)
    elt = 4 if w.dtype == "f32" else 2
    # the commit moves the deepest root path of each tree (the longest acceptance
    # this tree allows, every row of it away from its final place when the path
    # leaves the first-child chain)
    fp = vs.flat_parent.cpu().numpy()
    al = np.zeros(w.batch, np.int32)
    ap = np.full((w.batch, w.depth), -1, np.int32)
    moved = 0
    for b in range(w.batch):
        path, r = [], w.T - 1
        while r > 0:
            path.append(r); r = int(fp[b, r])
        path = path[::-1]
        al[b] = len(path); ap[b, :len(path)] = path
        stay = 0
        while stay < len(path) and path[stay] == stay + 1:
            stay += 1
        moved += len(path) - stay
    vs.accept_len.copy_(torch.from_numpy(al)); vs.accept_path.copy_(torch.from_numpy(ap))
    rope_us = _graph_us(lambda: vs.rope(), 2) / vs.n_layers
    attn_us = _graph_us(lambda: vs.attention(), 2) / vs.n_layers
    attn_rope_us = _graph_us(lambda: vs.attention_rope(), 2) / vs.n_layers
    rope_bytes = 2 * (w.batch * w.T * w.n_q_heads + w.batch * w.T * w.n_kv_heads) * w.head_dim * elt
    commit_us = _graph_us(lambda: vs.commit(), reps)
    commit_bytes = 2 * 2 * vs.n_layers * w.n_kv_heads * w.head_dim * elt * moved
    fpd = vs.flat_parent
    dep = torch.empty_like(vs.flat_depth); pos = torch.empty_like(vs.position); msk = torch.empty_like(vs.mask)
    static_us = _graph_us(lambda: eb.eagle_tree_mask_static(w.batch, w.T, fpd, vs.ctx_len, dep, pos, msk), reps)

    draft = _time_draft_side(vs, w, stream)

    def decode_step_fused():
        vs.tree()
        vs.attention_rope()
        vs.verify(temperature, seed, 0)
        vs.commit()

    def decode_step_separate():
        vs.tree()
        vs.rope()
        vs.attention()
        vs.verify(temperature, seed, 0)
        vs.commit()

    def eager_us(fn, n=10):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n
    full_us = eager_us(decode_step_fused)
    separate_us = eager_us(decode_step_separate)
    return {
        "rope": {"us_per_layer_call": round(rope_us, 3), "bytes_per_call": rope_bytes,
                 "GBps": round(rope_bytes / (rope_us * 1e-6) / 1e9, 1),
                 "what": "q and the K tree rows of one layer rotated in place at their tree positions"},
        "kv_commit": {"us_per_call": round(commit_us, 3), "accept_len": [int(x) for x in al],
                      "rows_moved": moved, "bytes_per_call": commit_bytes,
                      "GBps": round(commit_bytes / (commit_us * 1e-6) / 1e9, 1) if commit_bytes else None,
                      "what": f"K and V of the accepted rows moved behind the context in all {vs.n_layers} "
                              f"layers (path: the deepest root path of the tree)"},
        "attention_rope": {"us_per_layer_call": round(attn_rope_us, 3),
                           "attention_alone_us": round(attn_us, 3),
                           "added_us": round(attn_rope_us - attn_us, 3),
                           "what": "one layer's tree attention with the rotary at the tree positions inside it "
                                   "(eagle_tree_attention_rope), against the same call without rotary"},
        "mask_static": {"us_per_call": round(static_us, 3)},
        "draft_side": draft,
        "timing": "graph replays of the calls, HIP events",
        "decode_step_with_rope_and_commit": {
            "ms": round(full_us / 1e3, 4), "steps_per_s": round(1e6 / full_us, 2),
            "what": "expand x depth + rerank + mask + attention with rotary inside x layers + verify + KV commit, "
                    "eager launches"},
        "decode_step_with_separate_rope_call": {
            "ms": round(separate_us / 1e3, 4), "steps_per_s": round(1e6 / separate_us, 2),
            "what": "the same step with eagle_tree_rope called before plain attention in every layer"},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="llama2_13b")
    ap.add_argument("--graph", action="store_true", help="replay the step as one captured HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip timing rotary, KV commit and the static mask")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, copy MIB MiB device to device 3 times (a plain copy kernel of "
                         "known size whose FETCH_SIZE / WRITE_SIZE counters scale the attention's)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on exactly one GPU; --gpus must be 1"}))
        sys.exit(2)

    import torch
    from draft_tree_verification_eagle_amd import step as stepm
    from draft_tree_verification_eagle_amd import workload as wl

    w = wl.CONFIGS[args.config]
    temperature = w.temperatures[-1]
    seed = 12345
    torch.cuda.set_device(0)
    # A one-layer workload would sit in the 256 MB last-level cache across steps:
    # rotate over copies of its attention inputs totalling more than 512 MB
    # (distinct buffers, one used per step).  Multi-layer workloads already touch
    # a different layer's buffers at every call.
    rot = 1
    if w.layers == 1:
        rot = int(min(2048, max(16, -(-600_000_000 // attention_bytes_per_launch(w)))))
    print(f"[bench] allocating {args.config} inputs ({rot} copies of the attention inputs)" if rot > 1 else
          f"[bench] allocating {args.config} inputs", file=sys.stderr, flush=True)
    vs = stepm.VerifyStep(w, device="cuda:0", with_lse=False, layers=w.layers * rot)
    # target logits depend on the tree: build it once (untimed), plant, upload
    vs.tree()
    torch.cuda.synchronize()
    ft, fp = vs.flat_host()
    target = wl.plant(wl.target_logits_base(w), ft, fp, w.plant_frac, w.seed)
    vs.set_target(target)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    n_attn = w.layers  # attention calls per step
    layer_sets = [list(range(j * w.layers, (j + 1) * w.layers)) for j in range(rot)]

    def run_step(i):
        vs.tree()
        vs.attention(layer_sets[i % rot])
        vs.verify(temperature, seed, i)

    graph = None
    if args.graph:
        for i in range(3):
            run_step(i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_step(0)
        torch.cuda.synchronize()

    def one_step(i, ev=None, ev_start=None):
        if ev_start is not None:
            ev_start.record(stream)
        if graph is not None:
            graph.replay()
            return
        vs.tree()
        if ev is not None:
            ev[0].record(stream)
        vs.attention(layer_sets[i % rot])
        if ev is not None:
            ev[1].record(stream)
        vs.verify(temperature, seed, i)

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    step_evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        one_step(i, None if graph is not None else evs[i], step_evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step (wall {wall:.3f}s)", file=sys.stderr, flush=True)

    # per-step times from the events at each step's start
    bounds = step_evs + [t_end]
    step_ms = np.array([bounds[j].elapsed_time(bounds[j + 1]) for j in range(args.steps)])
    attn_us = None
    # attention launch time: events around the 40 launches of each timed step
    if graph is None:
        attn_ms = [a.elapsed_time(b) for a, b in evs]
        ms_per_launch = float(np.median(attn_ms)) / n_attn
        attn_us = np.array(attn_ms) * 1e3 / n_attn
    else:
        # graph mode: time the attention launches alone on the same stream
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(5):
            vs.attention(layer_sets[j % rot])
        e1.record(stream)
        torch.cuda.synchronize()
        ms_per_launch = e0.elapsed_time(e1) / (5 * n_attn)
    # calls around the step, timed after it (they rewrite q and the K/V caches in place)
    extras = None if args.no_extras or graph is not None or rot > 1 else time_extras(vs, w, stream, temperature, seed)
    copy_gbs = measured_copy_gbs()
    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 3 x {nbytes} bytes", file=sys.stderr, flush=True)
    bytes_launch = attention_bytes_per_launch(w)
    achieved = bytes_launch / (ms_per_launch * 1e-3) / 1e9
    flops_launch = attention_flops_per_launch(w, vs.mask.cpu().numpy(), vs.ctx_lens_np)
    tflops = flops_launch / (ms_per_launch * 1e-3) / 1e12
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    traffic = None
    traffic_file = TRAFFIC_FILE.format(w.name)
    if os.path.exists(traffic_file):
        # counters taken on an older kernel source do not describe this one
        try:
            rec = json.load(open(traffic_file))
            src = open(os.path.join(ROOT, rec["source"]), "rb").read()
            # the counters describe one workload and one kernel source
            if hashlib.sha256(src).hexdigest() == rec["source_sha256"] and rec.get("workload") == w.name:
                traffic = rec["bytes_per_launch"]
        except (OSError, KeyError, ValueError):
            traffic = None

    if w.name == "llama2_13b":
        metric = "tree-verify steps/sec + tree-attn HBM GB/s (% peak), 13B shape ctx 4096, 60 nodes"
    else:
        metric = f"tree-verify steps/sec + tree-attn HBM GB/s (% peak), {w.name}"
    kernel = ("tree_attn_bf16_kernel + tree_attn_merge_kernel (one eagle_tree_attention call)" if w.dtype == "bf16"
              else "tree_attn_f32_kernel (one eagle_tree_attention call)")
    if w.ctx_range is not None:
        ctx_label = f"ctx {w.ctx_range[0]}-{w.ctx_range[1]} (ragged, packed cache)"
        ctx_field = [int(x) for x in vs.ctx_lens_np]
    else:
        ctx_label, ctx_field = f"ctx {w.ctx}", w.ctx
    out = {
        "metric": metric,
        "value": round(1000.0 / ms_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.batch} x draft tree d{w.depth} k{w.topk} m{w.m} n{w.n} (T={w.T}), "
                        f"vocab {w.vocab}, tree attention {w.layers} layers x {w.n_q_heads}q/{w.n_kv_heads}kv heads "
                        f"x {w.head_dim}, {w.dtype} KV at {ctx_label}, verify temperature {temperature}",
            "batch": w.batch, "ctx_len": ctx_field, "tree_rows": w.T, "layers": w.layers,
            "graph": bool(args.graph), "parallelism": "single GPU",
            "attention_input_copies": rot,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "box_copy_GBs": round(copy_gbs, 1),
            "frac_of_box_copy": round(achieved / copy_gbs, 4),
            "kernel": kernel,
            "bytes_per_launch": bytes_launch,
            "us_per_launch": round(ms_per_launch * 1e3, 3),
            "flops_per_launch": flops_launch,
            "mfma_side": {"achieved_TFLOPs": round(tflops, 2), "peak_TFLOPs": mfma_peak,
                          "frac": round(tflops / mfma_peak, 4),
                          "flop_per_byte": round(flops_launch / bytes_launch, 1)},
        },
    }
    pct = lambda x: {"p10": round(float(np.percentile(x, 10)), 4), "median": round(float(np.median(x)), 4),
                     "p90": round(float(np.percentile(x, 90)), 4)}
    out["distribution"] = {"step_ms": pct(step_ms)}
    if attn_us is not None:
        out["distribution"]["attention_us_per_launch"] = pct(attn_us)
    if extras is not None:
        out["around_step"] = extras
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline (bounded sample)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, vs.draft_np, vs.root_np, target, temperature, seed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
