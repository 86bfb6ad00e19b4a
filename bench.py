#!/usr/bin/env python3
"""Benchmark of the grouped, weight-quantized MoE FFN on one MI355X.

A step is one pass of the whole layer on one batch of synthetic inputs that
already sit in HBM: route (softmax top-k) and align (group pairs by expert),
one launch up to 16 tokens -> grouped FFN (stage 1 + requant + stage 2) ->
combine.  Default workload:
fp8 activations x MXFP4 weights, hidden 4096, 512 experts, top-10, expert
inter 1024, 4096 tokens (40960 (token, expert) rows).

Weights are rewritten once into the library's streaming layout
(qmoe_prepack) at set-up.  Before every timed step a 512 MiB buffer is
read (a max reduction) to flush the 256 MB memory-side cache: the step then
finds none of its inputs in that cache, and no dirty lines of the flush
itself are left to be written back inside the step, as a write-based flush
would leave.  The step's four launches are captured once into a HIP graph
and replayed (no host launch gaps between the kernels); each replay is
timed with HIP events on the launch stream (the flush sits outside them)
and ms_per_step is their mean over the timed steps.  The last replay's
output must equal an eager step's bit for bit.  A separate eager pass with
events between the kernels gives the per-kernel breakdown (kernel_ms; its
route, align and combine intervals also hold host launch gaps).

Prints one JSON line on stdout (one per workload with --sweep); progress
goes to stderr.
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

METRIC = "grouped MoE FFN TFLOP/s + % MFMA/HBM roofline at M=4096 prefill, 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"a8w4": 5000.0, "w8a8": 5000.0, "w4a16": 2500.0, "w4a8": 5000.0}
DTYPE = {"a8w4": "fp8e4m3*fp4e2m1", "w8a8": "int8", "w4a16": "bf16", "w4a8": "int8*int4"}
# Counter calibration: HBM bytes per KiB that FETCH_SIZE / WRITE_SIZE report,
# measured on a plain 1 GiB device copy (__amd_rocclr_copyBuffer, run with
# --copy-calibration-mib 1024): FETCH_SIZE reads 524,300 KiB for 1 GiB read,
# WRITE_SIZE 1,048,576 KiB for 1 GiB written.
FETCH_FACTOR = 1024 * 2.0
WRITE_FACTOR = 1024 * 1.0
# FETCH_SIZE / WRITE_SIZE (KiB per launch, mean of 7 launches) of the
# dominant kernel on the default workload, and the hash of the kernel sources
# they were taken with; traffic is reported only while the sources match.
DOMINANT_COUNTERS = {
    "kernel": "stage1",
    "fetch_kib": 1195528.5,
    "write_kib": 165148.4,
    "sources_sha256_16": "bf2cf1111afff413",
    "workload": "a8w4_large@T4096",
    "block_m": 128,
    "weight_layout": "prepacked",
}
KERNEL_SOURCES = ("quantized_mixture_experts_moe_amd/csrc/gemm.hip",
                  "quantized_mixture_experts_moe_amd/csrc/gemm_common.h",
                  "quantized_mixture_experts_moe_amd/csrc/qmoe_internal.h")


def kernel_sources_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes_per_expert(shape, which: str) -> float:
    """Codes + scales of one expert's W13 ([2I, H]) or W2 ([H, I])."""
    n, kdim = (2 * shape.inter, shape.hidden) if which == "w13" else (shape.hidden, shape.inter)
    if shape.scheme == "w8a8":
        return n * kdim + n * 4
    if shape.scheme in ("w4a16", "w4a8"):
        return n * kdim / 2 + n * (kdim // 32) * 2
    return n * kdim / 2 + n * (kdim // 32)  # a8w4: e2m1 + e8m0


def algorithmic_bytes(shape, touched: int) -> dict:
    """Bytes each kernel must move at minimum (the per-unit figures times the
    units one launch processes): the weights (codes and scales) of the
    touched experts, the activations in their scheme format, the output
    once, and the routing.  The intermediate h and the per-pair outputs
    y_pairs are implementation overhead and are reported apart
    (``overhead_bytes``), not counted here."""
    T, H, I, k = shape.tokens, shape.hidden, shape.inter, shape.topk
    P = T * k
    xb = 2 if shape.scheme == "w4a16" else 1
    xs = 0 if shape.scheme == "w4a16" else 4
    w13 = touched * weight_bytes_per_expert(shape, "w13")
    w2 = touched * weight_bytes_per_expert(shape, "w2")
    s1 = w13 + T * (H * xb + xs)
    s2 = w2
    comb = T * H * 2 + P * 4
    step = w13 + w2 + T * (H * xb + xs) + T * H * 2 + T * shape.experts * 4 + P * 8
    return {"stage1": s1, "stage2": s2, "combine": comb, "step": step}


def overhead_bytes(shape) -> dict:
    """Bytes of the intermediates the algorithm does not need to move: h
    written by stage 1 (fp32 for the requantized schemes, bf16 for W4A16)
    and read back, and y_pairs written by stage 2 and read by combine."""
    P = shape.tokens * shape.topk
    hb = 2 if shape.scheme == "w4a16" else 4
    yb = 4 if shape.scheme == "w8a8" else 2
    return {"h_write": P * shape.inter * hb, "h_read": P * shape.inter * hb,
            "y_pairs_write": P * shape.hidden * yb, "y_pairs_read": P * shape.hidden * yb}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(shape, inp, target_s: float = 15.0) -> dict:
    """Time the CPU oracle on a bounded sample of the same workload: whole
    tokens drawn at random, routed by the oracle, every expert they touch
    run on their rows; BLAS threads = the cores this process may use."""
    import oracle as O
    from threadpoolctl import threadpool_limits

    from quantized_mixture_experts_moe_amd import synth

    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(0)
    n_tok = 2
    elapsed = 0.0
    total_flops = 0.0
    total_pairs = 0
    total_tok = 0
    with threadpool_limits(cores):
        while True:
            toks = rng.choice(shape.tokens, min(n_tok, shape.tokens), replace=False)
            ids, w = O.route(inp["logits"][toks], shape.topk)
            experts = sorted(set(ids.reshape(-1).tolist()))
            wts = {e: synth.expert_weights(shape, e) for e in experts}  # generation: not timed
            xs = None if inp["x_scale"] is None else inp["x_scale"][toks]
            t0 = time.perf_counter()
            O.moe_forward(shape.scheme, inp["x"][toks], xs, lambda e: wts[e], ids, w)
            dt = time.perf_counter() - t0
            elapsed += dt
            total_pairs += len(toks) * shape.topk
            total_tok += len(toks)
            total_flops += 6.0 * shape.hidden * shape.inter * len(toks) * shape.topk
            log(f"cpu oracle: {len(toks)} tokens in {dt:.2f}s")
            if elapsed >= target_s * 0.5 or n_tok >= 256 or len(toks) == shape.tokens:
                break
            n_tok = int(min(256, max(n_tok * 2, n_tok * (target_s - elapsed) / max(dt, 1e-3) / 2)))
    return {"value": total_flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"{total_tok} tokens ({total_pairs} token-expert rows) of {shape.name}, "
                      f"fp64 numpy oracle, {elapsed:.1f}s; weight generation not timed",
            "tokens_per_s": total_tok / elapsed}


SWEEP = ("w4a16_qwen3moe_t128", "w8a8_t2048", "a8w4_large@T1", "a8w4_large@T2",
         "a8w4_large@T4", "a8w4_large@T16", "a8w4_large@T64", "a8w4_large@T256",
         "a8w4_large@T1024", "a8w4_large@T4096", "a8w4_large@T8192", "a8w4_tp2@T4096",
         "a8w4_tp4@T4096", "w4a16_skewed_t8192", "w4a8_qwen3moe_t128", "w4a8_t2048",
         "w4a8_skewed_t8192")
# Batches the sweep also runs through the other path (the one-launch
# qmoe_decode above 4 tokens, the multi-launch path at 1-4 tokens).
SWEEP_BOTH_PATHS = ("a8w4_large@T1", "a8w4_large@T2", "a8w4_large@T4", "a8w4_large@T16")


def stage_flops(shape) -> dict:
    """Useful FLOPs of each GEMM stage (2 per multiply-add, no padding rows)."""
    P = shape.tokens * shape.topk
    return {"stage1": 4.0 * shape.hidden * shape.inter * P,
            "stage2": 2.0 * shape.hidden * shape.inter * P, "combine": 0.0}


def graph_step_ms(torch, ops, args, flush, b: dict, eager_step, body=None, outs=None):
    """Mean and median GPU time of one step run as a HIP graph: the step's
    launches (route and align, grouped FFN, combine; or the one decode
    launch: ``body``) captured once and replayed, so that no host launch gap
    sits between them.  The cache flush stays outside the graph and outside
    the events.  The last replay's outputs must equal a following eager
    step's bit for bit."""
    sh = b["shape"]
    if body is None:
        g, E, k = b["g"], sh.experts, sh.topk

        def body():
            ops.route_align(g["logits"], k, b["bm"], b["ids"], b["tw"], out=b["al"])
            ops.grouped_ffn(sh.scheme, g["x"], g["x_scale"], b["W"], b["al"], E, k,
                            ws=b["ws"], y_pairs=b["y"])
            ops.combine(b["y"], b["tw"], out_bf16=b["out_bf16"], out_f32=b["out_f32"],
                        want_f32=b["out_f32"] is not None)
    if outs is None:
        outs = [t for t in (b["out_bf16"], b["out_f32"]) if t is not None]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.warmup):
        if flush is not None:
            torch.amax(flush)
        graph.replay()
    torch.cuda.synchronize()
    if flush is not None:
        for i in range(args.steps):
            torch.amax(flush)
            ev[i][0].record()
            graph.replay()
            ev[i][1].record()
        torch.cuda.synchronize()
        ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    else:
        ev[0][0].record()
        for i in range(args.steps):
            graph.replay()
        ev[0][1].record()
        torch.cuda.synchronize()
        ms = np.array([ev[0][0].elapsed_time(ev[0][1]) / args.steps])
    got = [t.clone() for t in outs]
    eager_step()
    torch.cuda.synchronize()
    if not all(torch.equal(x, y) for x, y in zip(got, outs)):
        raise SystemExit("bench: graph replay output differs from the eager step")
    del graph
    log(f"{sh.name}: graph step {float(ms.mean()):.4f} ms")
    return float(ms.mean()), float(np.median(ms))


def roofline_of(shape, dom: str, kern_ms: float, nbytes: float, flops: float) -> dict:
    """Roofline entry of the dominant kernel: its bound from the arithmetic
    intensity against the ridge point peak_flops / peak_bandwidth."""
    peak_tf = MFMA_PEAK_TFLOPS[shape.scheme]
    if flops / nbytes > peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9):
        achieved = flops / (kern_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(achieved / peak_tf, 4)}
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}


def run_decode_workload(shape, inp, g, W, layout, args, torch, with_cpu, cpu_seconds) -> dict:
    """A batch of up to 16 tokens through qmoe_decode: the whole layer in one
    launch (routing from the logits to the combined output)."""
    from quantized_mixture_experts_moe_amd import ops

    T, E, k, H = shape.tokens, shape.experts, shape.topk, shape.hidden
    dev = torch.device("cuda:0")
    f32 = shape.scheme == "w8a8"
    r = ops.decode_forward(shape.scheme, g["logits"], g["x"], g["x_scale"], W, k, want_f32=f32,
                           want_y=False)
    ws = r["ws"]
    out = {key: r[key] for key in ("topk_ids", "topk_w", "out", "out_f32")}
    torch.cuda.synchronize()
    touched = int(torch.unique(out["topk_ids"]).numel())
    flush = None if args.no_flush else torch.ones(64 << 20, dtype=torch.int64, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()

    def launch():
        ops.decode_forward(shape.scheme, g["logits"], g["x"], g["x_scale"], W, k, want_f32=f32,
                           ws=ws, want_y=False, out=out)

    def step(ev=None):
        if flush is not None:
            torch.amax(flush)
        if ev is not None:
            ev[0].record()
        launch()
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    step_ms = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in range(args.steps)])
    # One launch per step: the events around it give the step's GPU time; a
    # HIP graph of a single kernel only adds the graph launch (reported
    # apart as ms_per_step_graph).
    eager_ms = float(step_ms.mean()) if flush is not None else wall_ms
    ms_per_step = eager_ms
    graph_ms = None
    outs = [t for t in (out["out"], out["out_f32"]) if t is not None]
    if not args.eager:
        graph_ms, _ = graph_step_ms(torch, ops, args, flush, dict(shape=shape), launch,
                                    body=launch, outs=outs)
    if ops.check_flags(ws) != 0:
        raise SystemExit("bench: the decode kernel reported a timed-out wait")
    kern = {"decode": float(step_ms.mean())}
    log(f"{shape.name}: one-launch decode kernel {kern['decode']:.4f} ms (eager events)")
    flops = shape.useful_flops()
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    ab = algorithmic_bytes(shape, touched)
    roof = roofline_of(shape, "decode", kern["decode"], ab["step"], flops)
    roof.update({"traffic": None, "kernel": f"decode ({shape.scheme}, one launch)",
                 "kernel_ms": round(kern["decode"], 4), "algorithmic_bytes": int(ab["step"]),
                 "algorithmic_flops": flops})
    step_gbs = ab["step"] / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE[shape.scheme], "data": "synthetic (seeded generator, weights random)",
        "config": {"workload": shape.name, "scheme": shape.scheme, "tokens": T, "hidden": H,
                   "inter": shape.inter, "experts": E, "topk": k, "path": "qmoe_decode",
                   "touched_experts": touched, "weight_layout": layout,
                   "cache_flush_between_steps": flush is not None,
                   "parallelism": "none (1 GPU)"},
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "timing": "HIP events around the step's one launch",
        "ms_per_step_eager": round(eager_ms, 4),
        "ms_per_step_graph": None if graph_ms is None else round(graph_ms, 4),
        "wall_ms_per_step": round(wall_ms, 4),
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "step_mfma_frac": round(tflops / MFMA_PEAK_TFLOPS[shape.scheme], 4),
        "kernel_ms": {n: round(v, 4) for n, v in kern.items()},
        "roofline": roof,
        "ms_per_step_stat": "mean over the timed steps (median in ms_per_step_median)",
    }
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(shape, inp, cpu_seconds)
    del ws, flush
    torch.cuda.empty_cache()
    return res


def run_workload(name: str, args, torch, with_cpu: bool, cpu_seconds: float = 20.0) -> dict:
    from quantized_mixture_experts_moe_amd import ops, synth
    from quantized_mixture_experts_moe_amd.shapes import default_block_m, shape_by_name

    shape = shape_by_name(name)
    bm = args.block_m or default_block_m(shape)
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    inp = synth.make_inputs(shape)
    log(f"generated {shape.name} in {time.perf_counter() - t0:.1f}s")

    def gpu(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    g = {k: gpu(v) for k, v in inp.items()}
    W = {k: g[k] for k in ("w13", "w13_scale", "w2", "w2_scale")}
    layout = "canonical" if args.canonical else "prepacked"
    if not args.canonical:
        W = ops.prepack_weights(shape.scheme, W)  # once, at set-up, outside the timed steps
        for key in ("w13", "w13_scale", "w2", "w2_scale"):
            del g[key]
    T, E, k, H = shape.tokens, shape.experts, shape.topk, shape.hidden
    one_launch = (T <= ops.DECODE_MAX_TOKENS and args.decode) or \
        (T <= ops.DECODE_PREFERRED_MAX_TOKENS and not args.grouped)
    if one_launch:
        return run_decode_workload(shape, inp, g, W, layout, args, torch, with_cpu, cpu_seconds)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    _, _, al = ops.route_align(g["logits"], k, bm, ids, tw)
    y, ws = ops.grouped_ffn(shape.scheme, g["x"], g["x_scale"], W, al, E, k)
    out_bf16, out_f32 = ops.combine(y, tw, want_bf16=True, want_f32=shape.scheme == "w8a8")
    torch.cuda.synchronize()
    touched = int(torch.unique(ids).numel())
    # The memory-side cache (256 MB) is flushed before every timed step by
    # reading a 512 MiB buffer; the flush sits between the step's events.
    flush = None if args.no_flush else torch.ones(64 << 20, dtype=torch.int64, device=dev)

    n_ev = 7
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    for row in evs:  # create the underlying events
        for e in row:
            e.record()
    torch.cuda.synchronize()

    def step(i, ev=None):
        if flush is not None:
            torch.amax(flush)
        if ev is not None:
            ev[0].record()
        ops.route_align(g["logits"], k, bm, ids, tw, out=al)
        if ev is not None:
            ev[1].record()
        ops.grouped_ffn(shape.scheme, g["x"], g["x_scale"], W, al, E, k, ws=ws, y_pairs=y,
                        stage_events=None if ev is None else ev[2:6])
        ops.combine(y, tw, out_bf16=out_bf16, out_f32=out_f32, want_f32=out_f32 is not None)
        if ev is not None:
            ev[6].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    def per_step(a, b):
        return np.array([evs[i][a].elapsed_time(evs[i][b]) for i in range(args.steps)])

    step_ms = per_step(0, 6)
    # Eager step time: the mean of the timed steps' GPU time (event 0 -> 6),
    # which leaves out the cache flush between steps; without the flush the
    # steps run back to back and the host clock is used.  At small sizes it
    # also holds the host's launch gaps between the kernels.
    eager_ms = float(step_ms.mean()) if flush is not None else wall_ms
    ms_per_step, graph_ms, graph_median = eager_ms, None, None
    if not args.eager:
        graph_ms, graph_median = graph_step_ms(torch, ops, args, flush, dict(
            shape=shape, g=g, W=W, ids=ids, tw=tw, al=al, y=y, ws=ws, bm=bm,
            out_bf16=out_bf16, out_f32=out_f32), lambda: step(0))
        ms_per_step = graph_ms
    kern = {"route_align": per_step(0, 1).mean(),
            "stage1": per_step(2, 3).mean(), "requant": per_step(3, 4).mean(),
            "stage2": per_step(4, 5).mean(), "combine": per_step(5, 6).mean(),
            "step_events": step_ms.mean()}
    kern = {n: float(v) for n, v in kern.items()}
    log(f"{shape.name}: per-kernel ms: " + ", ".join(f"{n} {v:.4f}" for n, v in kern.items()))

    flops = shape.useful_flops()
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    ab = algorithmic_bytes(shape, touched)
    sf = stage_flops(shape)
    dom = max(("stage1", "stage2", "combine"), key=lambda n: kern[n])
    peak_tf = MFMA_PEAK_TFLOPS[shape.scheme]
    roof = roofline_of(shape, dom, kern[dom], ab[dom], sf[dom])
    traffic = None
    c = DOMINANT_COUNTERS
    if (dom == c["kernel"] and shape.name == c["workload"] and bm == c["block_m"]
            and layout == c["weight_layout"] and kernel_sources_hash() == c["sources_sha256_16"]):
        traffic = int(round(c["fetch_kib"] * FETCH_FACTOR + c["write_kib"] * WRITE_FACTOR))
    roof.update({"traffic": traffic,
                 "kernel": f"{dom} ({shape.scheme}, block_m {bm})",
                 "kernel_ms": round(kern[dom], 4), "algorithmic_bytes": int(ab[dom]),
                 "algorithmic_flops": sf[dom]})
    step_gbs = ab["step"] / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE[shape.scheme], "data": "synthetic (seeded generator, weights random)",
        "config": {"workload": shape.name, "scheme": shape.scheme, "tokens": T, "hidden": H,
                   "inter": shape.inter, "experts": E, "topk": k, "block_m": bm,
                   "path": "route_align + grouped_ffn + combine",
                   "touched_experts": touched, "weight_layout": layout,
                   "cache_flush_between_steps": flush is not None,
                   "parallelism": "none (1 GPU)"},
        "ms_per_step_median": round(float(np.median(step_ms) if graph_median is None
                                          else graph_median), 4),
        "timing": "hip graph of the step, replayed" if graph_ms is not None else "eager launches",
        "ms_per_step_eager": round(eager_ms, 4),
        "wall_ms_per_step": round(wall_ms, 4),
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "step_mfma_frac": round(tflops / peak_tf, 4),
        "kernel_ms": {n: round(v, 4) for n, v in kern.items()},
        "roofline": roof,
        "overhead_bytes": overhead_bytes(shape),
        "ms_per_step_stat": "mean over the timed steps (median in ms_per_step_median)",
    }
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(shape, inp, cpu_seconds)
    del g, W, y, ws, flush
    torch.cuda.empty_cache()
    return res


# Workloads and token buckets of the tile table (aiter PR 6090, section
# Changes: token buckets 1-256, 1024, 4096, 8192 of the a8w4 block and its
# tensor-parallel shares; the other workloads at their own token counts).
TILE_SWEEP_POINTS = (
    ("a8w4_large", (1, 16, 64, 256, 1024, 4096, 8192)),
    ("a8w4_tp2", (1, 16, 64, 256, 1024, 4096, 8192)),
    ("a8w4_tp4", (1, 16, 64, 256, 1024, 4096, 8192)),
    ("w4a16_qwen3moe_t128", (128,)),
    ("w8a8_t2048", (2048,)),
    ("w4a8_qwen3moe_t128", (128, 2048)),
    ("w4a16_skewed_t8192", (8192,)),
    ("w4a8_skewed_t8192", (8192,)),
)
TILE_SWEEP_BLOCKS = (16, 32, 64, 128)
SCHEME_CODE_C = {"w4a16": 0, "w8a8": 1, "a8w4": 2, "w4a8": 3}
# QMOE_TILE values that mean "the library's rule" for every tile knob.
TILE_NEUTRAL = {"s1w": 0, "s1r": 0, "s1runs": -1, "s2w": 0, "s2p": 0, "s2h": -1}


def _knob_values(scheme: str, bm: int, inter: int, hidden: int) -> dict:
    """The tile knobs that apply to a call, and the values the sweep tries
    (the library refuses the others).  Keys are QMOE_TILE fields."""
    resident = scheme in ("a8w4", "w8a8") and inter <= 1024
    kv = {"s1runs": (0, 1, 2)}
    if bm >= 64:
        kv["s1w"] = (4, 8)
    if bm <= 32:
        kv["s1r"] = (4,)
    if resident:
        nt = hidden // 256
        kv["s2p"] = tuple(p for p in (1, 2, 4, 8, 16) if nt % p == 0 and
                          (scheme != "w8a8" or p <= 16))
        if bm >= 32:
            kv["s2h"] = (0, 1)
    elif bm >= 64:
        kv["s2w"] = (4, 8)
    return kv


def _env_str(cfg: dict) -> str:
    return ",".join(f"{k}={v}" for k, v in sorted(cfg.items()))


def _table_row(sh, T: int, bm: int, cfg: dict) -> str:
    """One C initializer of the tile table (field order of TileRow)."""
    c = {"s1w": 0, "s1r": 0, "s1runs": -1, "s2w": 0, "s2p": 0, "s2h": -1}
    c.update(cfg)
    return ("{%d, %d, %d, %d, %d, %d, %d, {%d, %d, %d, %d, %d, %d}},"
            % (SCHEME_CODE_C[sh.scheme], sh.hidden, sh.inter, sh.experts, sh.topk, T, bm,
               c["s1w"], c["s1r"], c["s1runs"], c["s2w"], c["s2p"], c["s2h"]))


def tile_sweep(args, torch) -> None:
    """Tile table by a gated sweep.  For each workload and token bucket: every
    block_m with the library's other choices, then, at the fastest block_m,
    each other knob in turn (stage-1 block waves, ring depth, schedule;
    stage-2 waves, column passes, half tiles), a value kept when it is at
    least 2% faster (the step's run-to-run spread is about 1%).  Accuracy gate: a configuration counts only if its
    output equals the reference (block_m 16, the library's choices) bit for
    bit.  Every timed configuration sets all knobs (the rule's values where
    it changes none), so the library's current table plays no part and each
    emitted row is the configuration measured.  Inputs are drawn once per
    workload at its largest bucket; a bucket
    takes the leading tokens.  One JSON line per timed configuration, one per
    bucket with the chosen row; --emit-table writes the rows as the
    library's tile_table.inc."""
    from quantized_mixture_experts_moe_amd import ops, synth
    from quantized_mixture_experts_moe_amd.shapes import shape_by_name

    dev = torch.device("cuda:0")
    flush = torch.ones(64 << 20, dtype=torch.int64, device=dev)
    rows = []
    for base, buckets in TILE_SWEEP_POINTS:
        if args.tile_only and base not in args.tile_only.split(","):
            continue
        full = shape_by_name(base).with_tokens(max(buckets))
        inp = synth.make_inputs(full)
        g = {}
        for key, a in inp.items():
            if a is not None:
                g[key] = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype ==
                                                              np.uint16 else a)).to(dev)
        if full.scheme == "w4a16":
            g["x"] = g["x"].view(torch.bfloat16)
        W = ops.prepack_weights(full.scheme, {kk: g.pop(kk) for kk in
                                              ("w13", "w13_scale", "w2", "w2_scale")})
        del inp
        E, k = full.experts, full.topk
        f32 = full.scheme == "w8a8"
        for T in buckets:
            sh = full.with_tokens(T)
            gt = {"logits": g["logits"][:T], "x": g["x"][:T],
                  "x_scale": None if "x_scale" not in g else g["x_scale"][:T]}

            def measure(bm, cfg):
                # Every knob given (the rule's value where the trial sets
                # none), so that no tile-table entry of the library applies
                # and the emitted row is exactly the configuration timed.
                os.environ["QMOE_TILE"] = _env_str({**TILE_NEUTRAL, **cfg})
                ids = torch.empty((T, k), dtype=torch.int32, device=dev)
                tw = torch.empty((T, k), dtype=torch.float32, device=dev)
                _, _, al = ops.route_align(gt["logits"], k, bm, ids, tw)
                y, ws = ops.grouped_ffn(sh.scheme, gt["x"], gt["x_scale"], W, al, E, k)
                ob, of = ops.combine(y, tw, want_bf16=True, want_f32=f32)

                def eager_step():
                    ops.route_align(gt["logits"], k, bm, ids, tw, out=al)
                    ops.grouped_ffn(sh.scheme, gt["x"], gt["x_scale"], W, al, E, k, ws=ws,
                                    y_pairs=y)
                    ops.combine(y, tw, out_bf16=ob, out_f32=of, want_f32=f32)

                torch.cuda.synchronize()
                ms, med = graph_step_ms(torch, ops, args, flush, dict(
                    shape=sh, g=gt, W=W, ids=ids, tw=tw, al=al, y=y, ws=ws, bm=bm,
                    out_bf16=ob, out_f32=of), eager_step)
                outs = (ob.clone(), of.clone() if f32 else None)
                del y, ws, al
                return ms, outs

            ref = None
            best = None  # (ms, bm, cfg)
            for bm in TILE_SWEEP_BLOCKS:
                ms, outs = measure(bm, {})
                if ref is None:
                    ref = outs
                gate = torch.equal(outs[0], ref[0]) and (not f32 or torch.equal(outs[1], ref[1]))
                print(json.dumps({"tile_sweep": base, "tokens": T, "block_m": bm, "cfg": "",
                                  "ms_per_step": round(ms, 4), "gate_bitexact": gate}),
                      flush=True)
                if gate and (best is None or ms < best[0]):
                    best = (ms, bm, {})
            ms0, bm, cfg = best
            default_ms = ms0
            for knob, values in _knob_values(sh.scheme, bm, sh.inter, sh.hidden).items():
                for v in values:
                    trial = dict(cfg)
                    trial[knob] = v
                    ms, outs = measure(bm, trial)
                    gate = torch.equal(outs[0], ref[0]) and (not f32 or
                                                             torch.equal(outs[1], ref[1]))
                    print(json.dumps({"tile_sweep": base, "tokens": T, "block_m": bm,
                                      "cfg": _env_str(trial), "ms_per_step": round(ms, 4),
                                      "gate_bitexact": gate}), flush=True)
                    if gate and ms < best[0] * 0.98:
                        best = (ms, bm, trial)
                cfg = best[2]
            os.environ.pop("QMOE_TILE", None)
            row = _table_row(sh, T, best[1], best[2])
            rows.append(row)
            print(json.dumps({"tile_best": base, "tokens": T, "block_m": best[1],
                              "cfg": _env_str(best[2]), "ms_per_step": round(best[0], 4),
                              "library_choices_ms": round(default_ms, 4), "row": row}),
                  flush=True)
        del g, W
        torch.cuda.empty_cache()
    if args.emit_table:
        src = os.path.join(ROOT, "quantized_mixture_experts_moe_amd", "csrc", "tile_table.inc")
        with open(src) as f:
            head = [line for line in f if line.startswith("//")]
        with open(args.emit_table, "w") as f:
            f.writelines(head)
            for row in rows:
                f.write(row + "\n")
        log(f"wrote {len(rows)} rows to {args.emit_table}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="a8w4_large@T4096")
    ap.add_argument("--sweep", action="store_true",
                    help="run every workload of the sweep, one JSON line each (CPU baseline on a "
                         "shorter sample per workload unless --no-cpu-baseline)")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="gated tile sweep (block_m, blocks, prefetch ring, schedule, stage-2 "
                         "passes) per workload and token bucket")
    ap.add_argument("--tile-only", default="",
                    help="comma-separated workloads of the tile sweep (default: all)")
    ap.add_argument("--emit-table", default="",
                    help="with --tile-sweep: write the chosen rows, with the comment lines of "
                         "the library's tile_table.inc, to this file")
    ap.add_argument("--block-m", type=int, default=0)
    ap.add_argument("--eager", action="store_true",
                    help="time the eager launches only (no HIP graph of the step)")
    ap.add_argument("--canonical", action="store_true",
                    help="feed the weights in their canonical layout (default: the streaming "
                         "layout qmoe_prepack writes once at set-up, outside the timed steps)")
    ap.add_argument("--no-flush", action="store_true",
                    help="no cache flush between timed steps (steps run back to back)")
    ap.add_argument("--grouped", action="store_true",
                    help="batches of up to 4 tokens take the multi-launch path (route and "
                         "align, grouped FFN, combine) instead of the one-launch qmoe_decode")
    ap.add_argument("--decode", action="store_true",
                    help="batches of up to 16 tokens take the one-launch qmoe_decode (the "
                         "default choice sends only batches of up to 4 tokens there)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB "
                         "(--steps times); used to scale the FETCH_SIZE/WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has "
              "no multi-GPU path (see the sharding plan in the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_bytes": n, "ms": dt * 1e3, "GBps_read": n / dt / 1e9}))
        return

    torch.cuda.set_device(torch.device("cuda:0"))
    if args.tile_sweep:
        tile_sweep(args, torch)
        return
    if args.sweep:
        from quantized_mixture_experts_moe_amd import ops
        for name in SWEEP:
            print(json.dumps(run_workload(name, args, torch, not args.no_cpu_baseline,
                                          min(args.cpu_seconds, 8.0))), flush=True)
            if name in SWEEP_BOTH_PATHS:
                other = argparse.Namespace(**vars(args))
                t = int(name.split("@T")[1])
                one_launch = t <= ops.DECODE_PREFERRED_MAX_TOKENS  # the default path
                other.grouped, other.decode = one_launch, not one_launch
                print(json.dumps(run_workload(name, other, torch, False)), flush=True)
        return
    res = run_workload(args.workload, args, torch, not args.no_cpu_baseline, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
