"""Benchmark of the W4A16 MoE expert layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--M M] [--no-cpu-baseline] [--sweep]

A step is one pass of the whole layer (align -> gate/up GEMM -> activation -> down GEMM ->
combine) over one batch of seeded synthetic inputs already resident in HBM.  The default
workload is one GPU's NVFP4 expert slice (32 of 256 experts, top-8, H = I = 4096, per-expert
RMSNorm before the weighted sum) on a batch of M = 4096 tokens with Zipf-skewed routing: the
largest configuration that fits one GPU (906 MB of weights, 2.3 TFLOP).

Timing: one step is one replay of a HIP graph of the layer's launches.  W untimed warm-up
steps, then K timed steps; before each, 1 GiB is read through the caches (so the weights come
from HBM, not from L2 or the memory-side cache), HIP events bracket the replay alone, and
value = M / the median step time.  "warm" (labelled, not the value) replays K steps back to
back with the weights left in the caches when they fit.  The roofline entry is for
the dominant kernel (the largest share of the layer's work): its average duration is taken
with HIP events on its launch stream around replays of a graph of back-to-back launches with the
arguments of a real step, and its algorithmic work per launch is the flops (prefill) or weight
bytes (decode) it must process.  The CPU
baseline is the float64 oracle on a bounded sample of the same workload on the host cores.

The W4AFP8 activation requant (moe_fp8_requant) has workloads of its own (`--workload
requant_...`, and in --sweep): its step is one launch over a masked [E, max_m, K] float8 batch,
its roofline is HBM on the algorithmic bytes (live rows x (2K + 4K/128): codes read and written,
group scales read), and its CPU baseline is the requant oracle.

Prints one JSON line.  With --sweep, prints one JSON line per configuration cell instead.
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
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s + weight-stream GB/s (decode) and TFLOP/s (prefill) vs roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "quantized_mixture_experts_align_amd", "csrc")
# every source the GEMM kernels are compiled from: a change to any of them voids old counters
GEMM_SRCS = ["moe_gemm.hip", "moe_gemm_common.h", "moe_gemm_mfma.h", "moe_gemm_decode.h",
             "moe_gemm_stream.h", "moe_gemm_int4.hip", "moe_gemm_nvfp4.hip", "moe_gemm_mxfp4.hip",
             "moe_gemm_int4zp.hip", "moe_gemm_stream_int4.hip", "moe_gemm_stream_nvfp4.hip",
             "moe_gemm_stream_mxfp4.hip", "moe_gemm_stream_int4zp.hip", "moe_gemm_int4zpf.hip",
             "moe_gemm_stream_int4zpf.hip", "moe_internal.h"]
FLUSH_BYTES = 1 << 30          # read between cold steps: more than L2 + MALL
LAUNCHES = 20                  # back-to-back launches per graph when timing one GEMM


REQUANT_SRCS = ["moe_requant.hip", "moe_internal.h"]


def gemm_source_hash(srcs=None) -> str:
    h = hashlib.sha256()
    for f in srcs or GEMM_SRCS:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def weight_bytes_per_expert(wl, proj: str) -> int:
    """Algorithmic weight bytes of one expert's projection: codes + scales (+ 4-bit zero points,
    + global scale, + bias), at the unpadded shape."""
    N, K = (2 * wl.I, wl.H) if proj == "w13" else (wl.H, wl.I)
    codes = N * K // 2
    groups = N * (K // wl.group)
    scales = groups * (2 if wl.qtype in ("int4_g128", "int4zp_g128", "int4zpf_g128") else 1)
    # zero points: 4-bit integers (counted packed), or float16
    zeros = groups // 2 if wl.qtype == "int4zp_g128" else (2 * groups if wl.qtype == "int4zpf_g128" else 0)
    gs = 4 if wl.qtype == "nvfp4_g16" else 0
    bias = 2 * N if wl.bias else 0
    return codes + scales + zeros + gs + bias


def load_traffic(kernel: str, workload: str, srcs=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None if there
    is none for this kernel/workload or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_sha256_16") != gemm_source_hash(srcs):
        return None
    return d.get("bytes_per_launch")


def _oracle_layer_call(wl, lw, inp, tokens):
    from oracle import moe as O
    return O.moe_layer(wl.qtype, inp.x, inp.topk_ids, inp.topk_weights, lw.w13, lw.w2,
                       expert_start=wl.expert_start, n_local=wl.n_local, act=wl.act, alpha=wl.alpha,
                       limit=wl.limit, norm_w_bits=lw.norm_w, eps=wl.eps,
                       interleaved_w13=wl.interleaved_w13, routed_scaling_factor=wl.routed_scaling_factor,
                       tokens=np.asarray(tokens))


def cpu_baseline(wl, lw, inp, budget_s: float = 15.0) -> dict:
    """The float64 oracle on a bounded sample of the same batch: whole tokens, chosen in batch
    order under a budget of dequantised experts (the oracle's dominant cost on the large
    weight sets), so that one timed run takes about `budget_s` seconds."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    M = inp.M
    lo, hi = wl.expert_start, wl.expert_start + wl.n_local
    local = [set(int(e) for e in row if lo <= e < hi) for row in np.asarray(inp.topk_ids)]
    first = next((t for t in range(M) if local[t]), 0)
    # calibration: the first token with a live slot
    t0 = time.perf_counter()
    _oracle_layer_call(wl, lw, inp, [first])
    per_expert = (time.perf_counter() - t0) / max(1, len(local[first]))
    budget = int(min(wl.n_local, max(len(local[first]), budget_s / max(per_expert, 1e-4))))
    chosen, touched = [], set()
    for t in range(M):
        if len(touched | local[t]) <= budget:
            chosen.append(t)
            touched |= local[t]
    live = sum(len([e for e in np.asarray(inp.topk_ids)[t] if lo <= e < hi]) for t in chosen)
    t0 = time.perf_counter()
    _oracle_layer_call(wl, lw, inp, chosen)
    dt = time.perf_counter() - t0
    T = len(chosen)
    return {"value": round(T / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle, whole layer (align, dequantisation of the touched experts, both "
                      f"GEMMs, activation, combine) on {T} of the {M} tokens, taken in batch order while "
                      f"they touch at most {budget} of the {wl.n_local} local experts ({len(touched)} "
                      f"touched, {live} live slots); one run, {dt:.1f} s wall, {threads} BLAS threads"}


_LAYERS: dict = {}   # prepared weights reused across cells of one weight set


def run_cell(name: str, M: int, steps: int, warmup: int, want_cpu: bool, seed=None,
             fused_combine: bool = False, block_m=None, group_m=(None, None), ng=(None, None)) -> dict:
    import torch
    import workloads as W
    from quantized_mixture_experts_align_amd import MoELayer
    import quantized_mixture_experts_align_amd as P

    wl = W.WORKLOADS[name]
    dev = torch.device("cuda", 0)
    if _LAYERS.get("seed") != wl.seed:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        lw = W.make_weights(wl)
        w13, w2, nw = W.device_weights(lw, dev)
        layer = MoELayer(wl.qtype, w13, w2, expert_start=wl.expert_start, n_local=wl.n_local,
                         top_k=wl.top_k, act=wl.act, alpha=wl.alpha, limit=wl.limit, post_norm_w=nw,
                         eps=wl.eps, interleaved_w13=wl.interleaved_w13,
                         n_global=wl.n_global)
        del w13, w2
        _LAYERS.update(seed=wl.seed, lw=lw, layer=layer)
    lw, layer = _LAYERS["lw"], _LAYERS["layer"]
    inp = W.make_inputs(wl, M, seed)
    x, ids, gw = W.device_inputs(inp, dev)
    ws = layer.workspace(M, block_m, device=dev)
    if group_m != (None, None) or ng != (None, None):
        # launch choices of the MFMA GEMMs only (their results are the same bit for bit)
        from quantized_mixture_experts_align_amd import _lib as L
        ws.cfgs = tuple(P.gemm_config(c.kernel, n or c.ng, c.ksplit, c.gemv_rows,
                                      c.group_m if gm is None else gm, c.block_order)
                        if c.kernel == L.GEMM_MFMA else c for c, n, gm in zip(ws.cfgs, ng, group_m))
    numel = M * wl.top_k
    local = (inp.topk_ids >= wl.expert_start) & (inp.topk_ids < wl.expert_start + wl.n_local)
    live = int(local.sum())
    touched = len(np.unique(inp.topk_ids[local]))
    flops_13 = 2.0 * live * (2 * wl.I) * wl.H
    flops_2 = 2.0 * live * wl.H * wl.I
    bytes_13 = touched * weight_bytes_per_expert(wl, "w13")
    bytes_2 = touched * weight_bytes_per_expert(wl, "w2")

    stream = torch.cuda.current_stream()
    for _ in range(3):
        layer(x, ids, gw, ws=ws, fused_combine=fused_combine)
    torch.cuda.synchronize()
    # ---- one step = one replay of a HIP graph of the layer's launches
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(x, ids, gw, ws=ws, fused_combine=fused_combine)
    torch.cuda.synchronize()
    flush = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device=dev)
    for _ in range(warmup):
        flush.sum()
        g.replay()
    torch.cuda.synchronize()
    # ---- value: K timed steps, each after reading 1 GiB through the caches (as the other layers'
    # weights would be read between two calls of this one), so that the weights come from HBM;
    # HIP events around the replay only, the median over the K steps.  A read, not a write: a
    # write would leave the memory-side cache full of dirty lines whose write-back then slows the
    # replay's reads (measured: about 3x on 128 MB).
    cold = []
    for _ in range(steps):
        flush.sum()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        g.replay()
        s1.record(stream)
        cold.append((s0, s1))
    torch.cuda.synchronize()
    cold_s = float(np.median([a.elapsed_time(b) for a, b in cold])) * 1e-3
    del flush
    # ---- warm (labelled, not the value): K replays back to back, weights left in L2 / the
    # memory-side cache when they fit
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps

    # ---- the two GEMMs alone: the arguments of a real step are recorded, then a HIP graph of
    # LAUNCHES back-to-back launches of each is replayed between HIP events on the launch stream
    # (the average per launch is the kernel's duration plus the graph's small launch gap)
    import quantized_mixture_experts_align_amd.ops as ops
    calls = {}
    orig, orig_act, orig_routed = ops.moe_w4a16_gemm, ops.moe_w4a16_gemm_act, ops.moe_w4a16_gemm_act_routed
    orig_cmb = ops.moe_w4a16_gemm_combine

    def record(fn, key):
        def wrapper(*a, **kw):
            calls[key] = (fn, a, kw)
            return fn(*a, **kw)
        return wrapper
    # gate/up GEMM (with the activation fused into it) and down GEMM
    # (small batches: the gate/up GEMM with the align fused into it)
    ops.moe_w4a16_gemm_act = record(orig_act, "gemm13")
    ops.moe_w4a16_gemm_act_routed = record(orig_routed, "gemm13")
    ops.moe_w4a16_gemm = record(orig, "gemm2")
    ops.moe_w4a16_gemm_combine = record(orig_cmb, "gemm2")  # (decode without norm: the weighted sum fused in)
    try:
        layer(x, ids, gw, ws=ws, fused_combine=fused_combine)
    finally:
        ops.moe_w4a16_gemm, ops.moe_w4a16_gemm_act, ops.moe_w4a16_gemm_act_routed = orig, orig_act, orig_routed
        ops.moe_w4a16_gemm_combine = orig_cmb
    torch.cuda.synchronize()
    dur = {}
    for key, (fn, a, kw) in calls.items():
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk):
            for _ in range(LAUNCHES):
                fn(*a, **kw)
        gk.replay()
        torch.cuda.synchronize()
        reps = max(5, steps // LAUNCHES)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            gk.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        dur[key] = e0.elapsed_time(e1) * 1e-3 / (reps * LAUNCHES)
        del gk

    # dominant kernel: the gate/up GEMM holds 2/3 of the flops and of the weight bytes; it is
    # compute-bound when its flops per weight byte exceed the machine balance
    d13 = dur["gemm13"]
    if flops_13 / bytes_13 > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        ach = flops_13 / d13 / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    else:
        ach = bytes_13 / d13 / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof["kernel"] = gemm13_kernel_name(layer, M, ws.block_m, calls["gemm13"][0] is orig_routed)
    roof["traffic"] = load_traffic("moe_gemm13", wl.name + f"_m{M}")
    roof["avg_launch_us"] = round(d13 * 1e6, 2)

    out = {
        "metric": METRIC, "value": round(M / cold_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(cold_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "qtype": wl.qtype, "M": M, "top_k": wl.top_k,
                   "n_local": wl.n_local, "n_global": wl.n_global, "H": wl.H, "I": wl.I,
                   "block_m": ws.block_m, "live_slots": live, "touched_experts": touched,
                   "fused_combine": fused_combine},
        "roofline": roof,
        "layer": {**layer_fracs(bytes_13 + bytes_2, flops_13 + flops_2, cold_s),
                  "weight_GBps": round((bytes_13 + bytes_2) / cold_s / 1e9, 1),
                  "TFLOPs": round((flops_13 + flops_2) / cold_s / 1e12, 2),
                  "gemm13_us": round(d13 * 1e6, 2), "gemm2_us": round(dur["gemm2"] * 1e6, 2),
                  "gemm2_fused_combine": calls["gemm2"][0] is orig_cmb,
                  "weight_bytes": bytes_13 + bytes_2, "flops": flops_13 + flops_2,
                  "note": "whole step, median of the K flushed replays (weights from HBM)"},
        "warm": {"ms_per_step": round(step_s * 1e3, 4), "tokens_per_s": round(M / step_s, 1),
                 "note": "K graph replays back to back (weights may stay in L2 / the memory-side cache)",
                 **layer_fracs(bytes_13 + bytes_2, flops_13 + flops_2, step_s)},
    }
    if want_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, lw, inp)
    return out


def run_requant_cell(name: str, steps: int, warmup: int, want_cpu: bool) -> dict:
    import torch
    import workloads as W
    from quantized_mixture_experts_align_amd import moe_fp8_requant, requant_choose

    wl = W.REQUANT_WORKLOADS[name]
    dev = torch.device("cuda", 0)
    inp = W.requant_inputs_for(wl)
    E, max_m, K = inp.x.shape
    x = torch.from_numpy(inp.x).to(dev)
    sc = torch.from_numpy(inp.scales).to(dev)
    mm = torch.from_numpy(inp.masked_m).to(dev)
    ts = torch.tensor([inp.tensor_scale], dtype=torch.float32, device=dev)
    out = torch.empty_like(x)
    rows = int(np.clip(inp.masked_m, 0, max_m).sum())
    nbytes = rows * (2 * K + 4 * (K // W.REQUANT_GROUP))
    # the launch hint from the rows the dispatch reports per expert, (rows + E) // E as in the page
    cfg = requant_choose(E, max_m, K, expected_rows=(rows + E) // E)
    stream = torch.cuda.current_stream()

    def launch():
        moe_fp8_requant(x, sc, mm, ts, W.REQUANT_GROUP, out=out, cfg=cfg)
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    # value: a graph of LAUNCHES back-to-back launches, HIP events on the launch stream
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(LAUNCHES):
            launch()
    for _ in range(max(1, warmup // LAUNCHES)):
        g.replay()
    torch.cuda.synchronize()
    reps = max(5, steps // LAUNCHES)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / (reps * LAUNCHES)
    # cold: one launch after reading 1 GiB through the caches, median over launches
    flush = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device=dev)
    cold = []
    for _ in range(max(50, min(steps, 200))):
        flush.sum()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        launch()
        s1.record(stream)
        cold.append((s0, s1))
    torch.cuda.synchronize()
    cold_s = float(np.median([a.elapsed_time(b) for a, b in cold])) * 1e-3
    del flush
    ach = nbytes / t / 1e9
    r = {
        "metric": "fp8 requant GB/s (algorithmic bytes) vs HBM roofline", "value": round(ach, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": reps * LAUNCHES, "warmup": warmup,
        "ms_per_step": round(t * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3fn/f32", "data": "synthetic",
        "config": {"workload": wl.name, "E": E, "max_m": max_m, "K": K, "live_rows": rows,
                   "group": W.REQUANT_GROUP, "expected_rows": (rows + E) // E,
                   "workgroups": cfg.workgroups, "unroll": cfg.unroll},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBS, 4), "kernel": "requant_kernel",
                     "traffic": load_traffic("requant_kernel", wl.name, REQUANT_SRCS), "avg_launch_us": round(t * 1e6, 3),
                     "bytes_per_launch": nbytes},
        "cold": {"us_per_launch": round(cold_s * 1e6, 3), "GBps": round(nbytes / cold_s / 1e9, 1),
                 "frac": round(nbytes / cold_s / 1e9 / PEAK_HBM_GBS, 4), "launches": len(cold),
                 "note": "median single launch after reading 1 GiB"},
    }
    if want_cpu:
        r["cpu_baseline"] = requant_cpu_baseline(inp, nbytes)
    return r


def requant_cpu_baseline(inp, nbytes: int, budget_s: float = 10.0) -> dict:
    from oracle import requant as R
    t0 = time.perf_counter()
    R.requant(inp.x, inp.scales, inp.masked_m, inp.tensor_scale)
    one = time.perf_counter() - t0
    reps = max(1, int(budget_s / max(one, 1e-3)))
    t0 = time.perf_counter()
    for _ in range(reps):
        R.requant(inp.x, inp.scales, inp.masked_m, inp.tensor_scale)
    dt = time.perf_counter() - t0
    return {"value": round(nbytes * reps / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"numpy requant oracle (single-threaded), the whole batch, {reps} runs, {dt:.1f} s wall"}


def layer_fracs(nbytes: float, flops: float, t: float) -> dict:
    """Fractions of the MI355X roofline reached by a whole step: of HBM peak on the touched
    weight bytes, of dense bf16 MFMA peak on the live-slot flops, and of the binding bound
    max(t_hbm, t_mfma) (1.0 = on the roofline)."""
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    return {"hbm_frac": round(t_hbm / t, 4), "mfma_frac": round(t_mfma / t, 4),
            "roof_frac": round(max(t_hbm, t_mfma) / t, 4)}


def gemm13_kernel_name(layer, M, block_m, routed: bool) -> str:
    from quantized_mixture_experts_align_amd import _lib as L
    c = layer.configs(M, block_m)[0]
    if c.kernel == L.GEMM_MFMA:
        name = "gemm_mfma_kernel"
    else:
        name = "gemm_stream_kernel" if c.gemv_rows == 0 else "gemm_decode_kernel"
    return name + (" (gate/up, align and activation fused)" if routed else " (gate/up, activation fused)")


def dense_reference(name: str, M: int, reps: int = 20) -> dict:
    """The MFMA ceiling this chip reaches on the layer's shapes without quantisation or grouping:
    torch's dense bf16 GEMM (hipBLASLt) of the same total shape -- [live slots, K] x [K, N] for
    each projection -- timed back to back with HIP events on random operands.  A calibration
    figure reported beside the layer, never part of it."""
    import torch
    import workloads as W
    wl = W.WORKLOADS[name]
    ids = np.asarray(W.make_inputs(wl, M).topk_ids)
    live = int(np.count_nonzero((ids >= wl.expert_start) & (ids < wl.expert_start + wl.n_local)))
    out = {"workload": name, "M": M, "live_slots": live, "gemms": {}}
    for proj, (k, n) in (("gate_up", (wl.H, 2 * wl.I)), ("down", (wl.I, wl.H))):
        a = torch.randn(live, k, dtype=torch.bfloat16, device="cuda")
        b = torch.randn(k, n, dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        flops = 2.0 * live * k * n
        out["gemms"][proj] = {"shape": [live, k, n], "us": round(t * 1e6, 1),
                              "TFLOPs": round(flops / t / 1e12, 1),
                              "frac": round(flops / t / (PEAK_BF16_TFLOPS * 1e12), 4)}
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="workload name (default: the NVFP4 EP8 slice "
                    "with Zipf routing, M=4096); one of the names in workloads.WORKLOADS")
    ap.add_argument("--M", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--block-m", type=int, default=None,
                    help="align block size (default: the library's choice); a launch option only")
    ap.add_argument("--group-m", type=int, default=None,
                    help="MFMA GEMMs: align blocks per XCD group (default: the library's choice)")
    ap.add_argument("--group-m2", type=int, default=None,
                    help="MFMA down GEMM only: align blocks per XCD group (overrides --group-m there)")
    ap.add_argument("--ng13", type=int, default=None, help="MFMA gate/up GEMM: tiles per wave")
    ap.add_argument("--ng2", type=int, default=None, help="MFMA down GEMM: tiles per wave")
    ap.add_argument("--sweep", action="store_true", help="one line per configuration cell")
    ap.add_argument("--fused-combine", action="store_true",
                    help="decode layers without norm: the weighted sum fused into the down GEMM")
    ap.add_argument("--dense-reference", action="store_true",
                    help="only time torch's dense bf16 GEMM (hipBLASLt) on the workload's GEMM shapes "
                         "with the live slots as rows: the MFMA ceiling without quantisation")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only copy a buffer of this many MiB 10 times (reference kernel of known "
                         "traffic for calibrating the HBM byte counters)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this layer is one GPU's expert slice and no multi-GPU "
              "path is built; run with --gpus 1", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no GPU visible)", file=sys.stderr)
        return 1
    if a.copy_mib:
        n = a.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 10}), flush=True)
        return 0
    import workloads as W
    if a.dense_reference:
        name = a.workload or W.HEADLINE
        M = a.M or (W.HEADLINE_M if name == W.HEADLINE else W.WORKLOADS[name].Ms[0])
        print(json.dumps(dense_reference(name, M)), flush=True)
        return 0
    if a.sweep:
        for name, wl in W.WORKLOADS.items():
            for M in wl.Ms:
                r = run_cell(name, M, a.steps, a.warmup, False)
                print(json.dumps(r), flush=True)
        for name in W.REQUANT_WORKLOADS:
            print(json.dumps(run_requant_cell(name, a.steps, a.warmup, False)), flush=True)
        return 0
    name = a.workload or W.HEADLINE
    if name in W.REQUANT_WORKLOADS:
        print(json.dumps(run_requant_cell(name, a.steps, a.warmup, not a.no_cpu_baseline)), flush=True)
        return 0
    if name not in W.WORKLOADS:
        print(f"unknown workload {name!r}; one of {list(W.WORKLOADS)}", file=sys.stderr)
        return 2
    M = a.M or (W.HEADLINE_M if name == W.HEADLINE else W.WORKLOADS[name].Ms[0])
    r = run_cell(name, M, a.steps, a.warmup, not a.no_cpu_baseline, fused_combine=a.fused_combine,
                 block_m=a.block_m, group_m=(a.group_m, a.group_m2 if a.group_m2 is not None else a.group_m),
                 ng=(a.ng13, a.ng2))
    print(json.dumps(r), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
