"""The down GEMM with the no-norm top-k weighted sum fused in (moe_w4a16_gemm_combine): its output
equals moe_w4a16_gemm followed by moe_combine bit for bit (tokens without a live slot included),
its arrival counters are left zero for the next call, and the whole decode layer with it meets
the layer bar against the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
import quantized_mixture_experts_align_amd as P
from quantized_mixture_experts_align_amd import _lib as L
from gpu_util import layer_violations, make_layer, oracle_layer

pytestmark = pytest.mark.gpu

_W2 = {}


def _w2(qtype):
    if qtype not in _W2:
        wl = W.small_workload(qtype, norm=False)
        lw = W.make_weights(wl)
        _, w2, _ = W.device_weights(lw)
        _W2[qtype] = (wl, P.moe_w4a16_prepare(qtype, w2["codes"], w2["scales"], w2.get("gs"), w2.get("bias"),
                                              0, w2.get("zeros")))
    return _W2[qtype]


def _compare(qtype, ids: np.ndarray, start: int, B: int, cfg=None, rsf=1.0, seed=0, counters=None):
    wl, W2 = _w2(qtype)
    M, k = ids.shape
    numel = M * k
    print(f"fused combine {qtype} M={M} k={k} start={start} B={B} rsf={rsf} "
          f"cfg={None if cfg is None else (cfg.ng, cfg.ksplit)}", flush=True)
    rng = np.random.default_rng(seed)
    a = torch.from_numpy(W._to_bf16_bits(rng.standard_normal((numel, W2.K)).astype(np.float32)).view(np.int16))
    a = a.cuda().view(torch.bfloat16)
    gw = torch.from_numpy(rng.random((M, k), dtype=np.float32)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    s, e, n, loc = P.moe_align(t, start, W2.desc.n_experts, B)
    y_ref = P.moe_w4a16_gemm(a, W2, s, e, n, numel, 1, B, cfg=cfg)
    ref = P.moe_combine(y_ref, gw, loc, None, routed_scaling_factor=rsf)
    if counters is None:
        counters = P.combine_counters(M, W2, a.device)
    y = torch.full((numel, W2.N), 7.0, dtype=torch.bfloat16, device="cuda")
    out = torch.full((M, W2.N), 7.0, dtype=torch.bfloat16, device="cuda")
    P.moe_w4a16_gemm_combine(a, W2, s, e, n, gw, loc, B, counters, y, out=out, routed_scaling_factor=rsf,
                             cfg=cfg)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))   # every row, dead tokens too
    live = torch.nonzero(loc.view(-1) >= 0).view(-1)
    assert torch.equal(y[live].view(torch.int16), y_ref[live].view(torch.int16))
    assert int(counters.abs().sum().item()) == 0                        # left zero for the next call
    return out


@pytest.mark.parametrize("qtype", W.QTYPES)
@pytest.mark.parametrize("M", [1, 3, 8])
def test_fused_combine_equals_gemm_then_combine(qtype, M):
    wl, _ = _w2(qtype)
    inp = W.make_inputs(wl, M, seed=500 + M)
    _compare(qtype, inp.topk_ids, wl.expert_start, 16, seed=M)


@pytest.mark.parametrize("seed", range(8))
def test_fused_combine_random_ids(seed):
    # junk ids, repeated experts inside a token, off-slice slots, tokens and batches with no live
    # slot, block sizes 1..16, every tile width and K split, a routed scaling factor
    rng = np.random.default_rng(600 + seed)
    qtype = W.QTYPES[seed % len(W.QTYPES)]
    wl, W2 = _w2(qtype)
    n_local = W2.desc.n_experts
    k = int(rng.integers(1, 9))
    M = int(rng.integers(1, 64 // k + 1))
    start = int(rng.integers(0, 6))
    ids = rng.integers(-3, start + n_local + 4, size=(M, k)).astype(np.int32)
    if seed == 5:
        ids[:] = start + n_local + 1          # nothing routed to this slice: every row is zero
    B = int(rng.choice([1, 4, 8, 16]))
    cfg = None
    if seed % 2:
        cfg = P.gemm_config(L.GEMM_DECODE, int(rng.choice([1, 2, 4])), int(rng.choice([1, 2, 4, 8])), 0)
    _compare(qtype, ids, start, B, cfg, rsf=1.0 if seed % 3 else 1.75, seed=seed)


def test_fused_combine_counters_serve_consecutive_calls():
    # one counter buffer, three calls with different batches: each call finds them zero
    wl, W2 = _w2("mxfp4_g32")
    counters = P.combine_counters(16, W2, "cuda")
    for i, M in enumerate((16, 5, 16)):
        inp = W.make_inputs(wl, M, seed=700 + i)
        _compare("mxfp4_g32", inp.topk_ids, wl.expert_start, 16, seed=i, counters=counters)


def test_fused_combine_rejections():
    wl, W2 = _w2("int4_g128")
    a = torch.zeros((4, W2.K), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    s, e, n, loc = P.moe_align(ids, 0, W2.desc.n_experts, 32)
    gw = torch.ones((2, 2), dtype=torch.float32, device="cuda")
    y = torch.empty((4, W2.N), dtype=torch.bfloat16, device="cuda")
    cnt = P.combine_counters(2, W2, "cuda")
    with pytest.raises(ValueError, match="block_m"):
        P.moe_w4a16_gemm_combine(a, W2, s, e, n, gw, loc, 32, cnt, y)
    s, e, n, loc = P.moe_align(ids, 0, W2.desc.n_experts, 16)
    with pytest.raises(ValueError, match="counters"):
        P.moe_w4a16_gemm_combine(a, W2, s, e, n, gw, loc, 16, cnt[:1], y)
    with pytest.raises(ValueError, match="streaming"):
        P.moe_w4a16_gemm_combine(a, W2, s, e, n, gw, loc, 16, cnt, y,
                                 cfg=P.gemm_config(L.GEMM_DECODE, 2, 1, 4))


@pytest.mark.parametrize("qtype,M", [("int4_g128", 1), ("int4_g128", 32), ("nvfp4_g16", 1), ("nvfp4_g16", 8),
                                     ("mxfp4_g32", 1), ("mxfp4_g32", 16), ("int4zp_g128", 3)])
def test_layer_with_fused_combine(qtype, M):
    wl = W.small_workload(qtype, norm=False)
    lw = W.make_weights(wl)
    inp = W.make_inputs(wl, M, seed=800 + M)
    layer = make_layer(wl, lw)
    x, ids, gw = W.device_inputs(inp)
    ws = layer.workspace(M)
    print(f"layer fused combine {wl.name} M={M}", flush=True)
    got_f = layer(x, ids, gw, ws=ws, fused_combine=True).clone()
    got_f2 = layer(x, ids, gw, ws=ws, fused_combine=True).clone()   # counters reused
    got_u = layer(x, ids, gw, ws=ws).clone()                         # the default: separate combine
    torch.cuda.synchronize()
    assert torch.equal(got_f.view(torch.int16), got_u.view(torch.int16))
    assert torch.equal(got_f2.view(torch.int16), got_u.view(torch.int16))
    assert int(ws.counters.abs().sum().item()) == 0
    ref = oracle_layer(wl, lw, inp)
    assert layer_violations(W.bf16_to_float(got_f), ref) == 0


def test_fused_combine_auto_config_on_long_k_weights():
    # 40 slots of K = 2048 down-projection weights: moe_gemm_choose picks the MFMA kernel there; the
    # fused weighted sum runs only in the streaming kernel, which then takes its own configuration
    wl = W.small_workload("mxfp4_g32", I=2048, norm=False)
    lw = W.make_weights(wl)
    _, w2, _ = W.device_weights(lw)
    W2 = P.moe_w4a16_prepare("mxfp4_g32", w2["codes"], w2["scales"], w2.get("gs"), w2.get("bias"), 0,
                             w2.get("zeros"))
    M, k = 10, wl.top_k
    assert M * k >= 32 and P.gemm_choose(W2, M * k, 16, 256).kernel == L.GEMM_MFMA
    inp = W.make_inputs(wl, M, seed=950)
    rng = np.random.default_rng(950)
    a = torch.from_numpy(W._to_bf16_bits(rng.standard_normal((M * k, W2.K)).astype(np.float32)).view(np.int16))
    a = a.cuda().view(torch.bfloat16)
    gw = torch.from_numpy(inp.topk_weights).cuda()
    ids = torch.from_numpy(inp.topk_ids).cuda()
    print(f"fused combine auto config mxfp4 K=2048 M={M} k={k}", flush=True)
    s, e, n, loc = P.moe_align(ids, wl.expert_start, W2.desc.n_experts, 16)
    y = torch.empty((M * k, W2.N), dtype=torch.bfloat16, device="cuda")
    got = P.moe_w4a16_gemm_combine(a, W2, s, e, n, gw, loc, 16, P.combine_counters(M, W2, "cuda"), y)
    ref = P.moe_combine(P.moe_w4a16_gemm(a, W2, s, e, n, M * k, 1, 16), gw, loc)         # MFMA kernel
    torch.cuda.synchronize()
    g, r = W.bf16_to_float(got), W.bf16_to_float(ref)
    rms = float(np.sqrt(np.mean(r * r)))
    assert rms > 0
    # the same products in another fp32 summation order, y rounded to bf16, then the weighted sum
    assert np.all(np.abs(g - r) <= 2.0 ** -6 * np.abs(r) + 2e-3 * rms), float(np.max(np.abs(g - r)))
