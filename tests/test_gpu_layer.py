"""Whole-layer GPU parity against the oracle: small shapes (several tiles, ragged tails) in
full, every workload at full size on sampled tokens, and edge cases."""
import numpy as np
import pytest
import torch

import workloads as W
import quantized_mixture_experts_align_amd as P
from quantized_mixture_experts_align_amd import _lib as L

from gpu_util import announce, layer_violations, make_layer, oracle_layer, rel_rms

pytestmark = pytest.mark.gpu


def _forward(layer, inp, **kw):
    out = layer(*W.device_inputs(inp), **kw)
    torch.cuda.synchronize()
    return W.bf16_to_float(out)


@pytest.mark.parametrize("M", [1, 3, 29, 130, 517])
@pytest.mark.parametrize("qtype", W.QTYPES)
def test_small_layer_matches_oracle(qtype, M):
    wl = W.small_workload(qtype)
    lw = W.make_weights(wl)
    inp = W.make_inputs(wl, M)
    announce(f"layer small {qtype} M={M}")
    got = _forward(make_layer(wl, lw), inp)
    ref = oracle_layer(wl, lw, inp)
    assert layer_violations(got, ref) == 0
    assert rel_rms(got, ref) < 0.01


@pytest.mark.parametrize("qtype", W.QTYPES)
def test_small_layer_every_gemm_kernel(qtype):
    wl = W.small_workload(qtype)
    lw = W.make_weights(wl)
    layer = make_layer(wl, lw)
    for M, B, cfg in [(7, 16, P.gemm_config(L.GEMM_DECODE, 4, 4, 4)),
                      (7, 16, P.gemm_config(L.GEMM_DECODE, 1, 1, 0)),
                      (90, 16, P.gemm_config(L.GEMM_MFMA, 1, 0, 0)),
                      (90, 32, P.gemm_config(L.GEMM_MFMA, 2, 0, 0)),
                      (300, 128, P.gemm_config(L.GEMM_MFMA, 4, 0, 0))]:
        inp = W.make_inputs(wl, M)
        announce(f"layer kernels {qtype} M={M} B={B} kernel={cfg.kernel}")
        got = _forward(layer, inp, ws=layer.workspace(M, B), cfg13=cfg, cfg2=cfg)
        ref = oracle_layer(wl, lw, inp)
        assert layer_violations(got, ref) == 0


@pytest.mark.parametrize("qtype", W.QTYPES)
def test_small_layer_relu2_routed_scaling(qtype):
    # the non-gated relu2 activation (GEMM1 has I rows) and a routed scaling factor, on the
    # streaming, dot-product and MFMA kernels.  (relu^2 makes the int4 outputs large -- RMS
    # about 2.6 at factor 1 for uint4b8, 6 for the float zero-point weights -- and the bar's
    # absolute term does not scale with them.  The dequantised int4 weights are rounded to bf16
    # before the bf16 MFMA; that rounding alone, applied to the float64 oracle's weights on the
    # CPU, puts the worst of these outputs at 1.25 times the bar at factor 0.625 (the float
    # zero-point workload at M = 150), 1.0 at 0.5 and 0.76 at 0.375.)
    wl = W.small_workload(qtype).replace(act="relu2", interleaved_w13=False, routed_scaling_factor=0.375)
    lw = W.make_weights(wl)
    layer = make_layer(wl, lw)
    assert layer.I == wl.I
    for M, B, cfg in [(6, 16, None), (6, 16, P.gemm_config(L.GEMM_DECODE, 2, 2, 4)), (150, 64, None),
                      (150, 32, P.gemm_config(L.GEMM_MFMA, 1, 0, 0))]:
        inp = W.make_inputs(wl, M)
        announce(f"layer relu2 {qtype} M={M} B={B}")
        got = _forward(layer, inp, ws=layer.workspace(M, B), cfg13=cfg, cfg2=cfg)
        ref = oracle_layer(wl, lw, inp)
        assert layer_violations(got, ref) == 0
        assert rel_rms(got, ref) < 0.01
        unf = _forward(layer, inp, ws=layer.workspace(M, B), cfg13=cfg, cfg2=cfg, fused_act=False)
        assert np.array_equal(got, unf)


def test_padded_intermediate_layer():
    # I = 288: zero-padded to 320 at prepare (GPT-OSS tile padding); same result as unpadded
    wl = W.small_workload("mxfp4_g32", I=288)
    lw = W.make_weights(wl)
    layer = make_layer(wl, lw, pad=True)
    assert layer.I == 320
    inp = W.make_inputs(wl, 77)
    got = _forward(layer, inp)
    assert layer_violations(got, oracle_layer(wl, lw, inp)) == 0


def test_off_slice_tokens_are_zero_and_runs_repeat_bitwise():
    wl = W.small_workload("nvfp4_g16")
    lw = W.make_weights(wl)
    inp = W.make_inputs(wl, 64)
    ids = inp.topk_ids.copy()
    ids[::4] = 60                        # outside the local range [8, 24)
    inp2 = W.LayerInputs(inp.x, ids, inp.topk_weights, inp.M)
    layer = make_layer(wl, lw)
    a = _forward(layer, inp2)
    b = _forward(layer, inp2)
    assert np.all(a[::4] == 0.0)
    assert np.array_equal(a, b)
    assert layer_violations(a, oracle_layer(wl, lw, inp2)) == 0


@pytest.mark.parametrize("qtype", W.QTYPES)
def test_degenerate_batches(qtype):
    # an empty batch; batches with no slot on the local slice (fused align at 1 token, the align
    # kernel at 100); a single token whose top-k all land on one local expert (repeated ids)
    wl = W.small_workload(qtype)
    lw = W.make_weights(wl)
    layer = make_layer(wl, lw)
    off = wl.expert_start + wl.n_local   # first global id outside the slice
    announce(f"layer degenerate {qtype}")
    x0 = torch.zeros((0, wl.H), dtype=torch.bfloat16, device="cuda")
    out0 = layer(x0, torch.zeros((0, wl.top_k), dtype=torch.int32, device="cuda"),
                 torch.zeros((0, wl.top_k), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert out0.shape == (0, wl.H)
    for M in (1, 100):
        inp = W.make_inputs(wl, M)
        inp = W.LayerInputs(inp.x, np.full_like(inp.topk_ids, off), inp.topk_weights, M)
        got = _forward(layer, inp)
        assert np.all(got == 0.0)
    inp = W.make_inputs(wl, 1)
    inp = W.LayerInputs(inp.x, np.full_like(inp.topk_ids, wl.expert_start + 1), inp.topk_weights, 1)
    got = _forward(layer, inp)
    ref = oracle_layer(wl, lw, inp)
    assert layer_violations(got, ref) == 0 and np.any(got != 0.0)


@pytest.mark.parametrize("qtype,kw,M", [
    ("int4_g128", dict(top_k=1), 70),                                  # top-1: slot = token
    ("nvfp4_g16", dict(n_global=16, expert_start=3, n_local=1), 40),    # one local expert
    ("mxfp4_g32", dict(top_k=16, n_global=32, n_local=32), 9),          # top-16: two-pass combine
    ("int4zp_g128", dict(top_k=8, n_global=16, expert_start=0, n_local=16), 8),   # 64 slots: fused align
    ("int4zp_g128", dict(top_k=5, n_global=16, expert_start=0, n_local=16), 13),  # 65 slots: align kernel
])
def test_layer_edge_shapes(qtype, kw, M):
    wl = W.small_workload(qtype).replace(**kw)
    lw = W.make_weights(wl)
    inp = W.make_inputs(wl, M)
    announce(f"layer edge {qtype} {kw} M={M}")
    got = _forward(make_layer(wl, lw), inp)
    ref = oracle_layer(wl, lw, inp)
    assert layer_violations(got, ref) == 0
    assert rel_rms(got, ref) < 0.01


# ----------------------------------------------------------------------------- full-size workloads
_CACHE = {}


def _workload_layer(name):
    wl = W.WORKLOADS[name]
    key = wl.seed
    if key not in _CACHE:
        _CACHE.clear()                   # keep one weight set resident at a time
        lw = W.make_weights(wl)
        _CACHE[key] = (lw, make_layer(wl, lw))
    return (wl,) + _CACHE[key]


def _sample(M, n, seed=0):
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(M, size=n, replace=False))


@pytest.mark.parametrize("name,M,n_sample", [(W.INT4_SMALL, 123, 123), (W.INT4_BIAS, 2304, 2304),
                                             (W.NVFP4_DECODE, 1, 1), (W.NVFP4_DECODE, 4, 4),
                                             (W.NVFP4_DECODE, 16, 5), (W.NVFP4_DECODE, 64, 5),
                                             (W.NVFP4_ZIPF, 256, 4), (W.NVFP4_ZIPF, 1024, 3), (W.NVFP4_ZIPF, 4096, 3),
                                             (W.MXFP4_SWIGLU, 1, 1), (W.MXFP4_SWIGLU, 32, 4),
                                             (W.MXFP4_SWIGLU, 2048, 4), (W.INT4ZP, 1, 1), (W.INT4ZP, 2304, 2304),
                                             (W.INT4_ACT_ORDER, 1, 1), (W.INT4_ACT_ORDER, 2304, 2304),
                                             (W.INT4ZPF, 1, 1), (W.INT4ZPF, 2304, 2304),
                                             (W.NVFP4_UNIFORM, 5760, 3), (W.NVFP4_UNIFORM, 23296, 3)])
def test_workload_layer_matches_oracle(name, M, n_sample):
    wl, lw, layer = _workload_layer(name)
    inp = W.make_inputs(wl, M)
    announce(f"layer {name} M={M} sampled tokens={n_sample}")
    got = _forward(layer, inp)
    toks = _sample(M, n_sample, seed=M)
    ref = oracle_layer(wl, lw, inp, tokens=toks)
    assert layer_violations(got[toks], ref) == 0
    assert rel_rms(got[toks], ref) < 0.01
    # every token whose slots all fall off the local slice is exactly zero
    off = np.all((inp.topk_ids < wl.expert_start) | (inp.topk_ids >= wl.expert_start + wl.n_local), axis=1)
    assert np.all(got[off] == 0.0)
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("qtype", W.QTYPES)
def test_small_layer_unfused_activation(qtype):
    wl = W.small_workload(qtype)
    lw = W.make_weights(wl)
    layer = make_layer(wl, lw)
    inp = W.make_inputs(wl, 130)
    got = _forward(layer, inp, fused_act=False)
    assert layer_violations(got, oracle_layer(wl, lw, inp)) == 0
    assert np.array_equal(got, _forward(layer, inp))      # fused and unfused give the same bytes


@pytest.mark.parametrize("qtype,M", [("nvfp4_g16", 1), ("mxfp4_g32", 100), ("int4_g128", 300), ("int4zp_g128", 5),
                                     ("int4zpf_g128", 200)])
def test_graph_replays_equal_eager_runs(qtype, M):
    # the layer captured once in a HIP graph (as bench.py times it), then replayed on three different
    # inputs copied into the captured tensors, eager work in between: every replay equals an eager run
    wl = W.small_workload(qtype)
    lw = W.make_weights(wl)
    layer = make_layer(wl, lw)
    announce(f"graph replay {qtype} M={M}")
    x, ids, gw = W.device_inputs(W.make_inputs(wl, M, seed=500))
    ws = layer.workspace(M, device=x.device)
    layer(x, ids, gw, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer(x, ids, gw, ws=ws)
    torch.cuda.synchronize()
    for seed in (501, 502, 503):
        x2, ids2, gw2 = W.device_inputs(W.make_inputs(wl, M, seed=seed))
        ref = layer(x2, ids2, gw2).clone()           # eager, its own workspace
        x.copy_(x2)
        ids.copy_(ids2)
        gw.copy_(gw2)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
