"""The fused route-and-align (moe_w4a16_gemm_act_routed, the single-token fast path widened to
128 slots): its align outputs and its activated gate/up output equal those of moe_align followed
by moe_w4a16_gemm_act bit for bit, and the whole layer with it meets the layer bar against the
oracle."""
import numpy as np
import pytest
import torch

import workloads as W
import quantized_mixture_experts_align_amd as P
from quantized_mixture_experts_align_amd import _lib as L
from gpu_util import layer_violations, make_layer, oracle_layer

pytestmark = pytest.mark.gpu

_W13 = {}


def _w13(qtype):
    if qtype not in _W13:
        wl = W.small_workload(qtype)
        lw = W.make_weights(wl)
        w13, _, _ = W.device_weights(lw)
        flags = L.PREP_GATE_UP | (L.PREP_INTERLEAVED if wl.interleaved_w13 else 0)
        _W13[qtype] = (wl, P.moe_w4a16_prepare(qtype, w13["codes"], w13["scales"], w13.get("gs"),
                                               w13.get("bias"), flags, w13.get("zeros")))
    return _W13[qtype]


def _compare(qtype, ids: np.ndarray, start: int, B: int, cfg=None, seed=0):
    wl, W13 = _w13(qtype)
    M, k = ids.shape
    print(f"routed {qtype} M={M} k={k} start={start} B={B} cfg={None if cfg is None else (cfg.ng, cfg.ksplit)}",
          flush=True)
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(W._to_bf16_bits(rng.standard_normal((M, wl.H)).astype(np.float32)).view(np.int16))
    x = x.cuda().view(torch.bfloat16)
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    s, e, n, loc = P.moe_align(t, start, W13.desc.n_experts, B)
    ref = P.moe_w4a16_gemm_act(wl.act, x, W13, s, e, n, M * k, k, B, wl.alpha, wl.limit, cfg=cfg)
    got, (s2, e2, n2, loc2) = P.moe_w4a16_gemm_act_routed(wl.act, x, W13, t, start, B, wl.alpha, wl.limit,
                                                           cfg=cfg)
    torch.cuda.synchronize()
    assert int(n2.item()) == int(n.item())
    assert torch.equal(s2, s) and torch.equal(e2, e) and torch.equal(loc2, loc)
    live = torch.nonzero(loc.view(-1) >= 0).view(-1)
    assert torch.equal(got[live].view(torch.int16), ref[live].view(torch.int16))   # rows of dead slots are not written


@pytest.mark.parametrize("qtype", W.QTYPES)
@pytest.mark.parametrize("M", [1, 2, 5])
def test_routed_equals_align_then_gemm_act(qtype, M):
    wl, _ = _w13(qtype)
    k = wl.top_k
    if M * k > 128:
        pytest.skip("more than 128 slots")
    inp = W.make_inputs(wl, M, seed=200 + M)
    _compare(qtype, inp.topk_ids, wl.expert_start, 16)


@pytest.mark.parametrize("seed", range(8))
def test_routed_random_ids(seed):
    # junk ids, repeated experts inside a token, off-slice slots, no live slot at all, block
    # sizes 1..16, up to 128 slots (one and two 64-slot batches), several launch shapes
    rng = np.random.default_rng(300 + seed)
    qtype = W.QTYPES[seed % len(W.QTYPES)]
    wl, W13 = _w13(qtype)
    n_local = W13.desc.n_experts
    k = int(rng.integers(1, 9))
    M = int(rng.integers(1, 128 // k + 1))
    start = int(rng.integers(0, 6))
    ids = rng.integers(-3, start + n_local + 4, size=(M, k)).astype(np.int32)
    if seed == 5:
        ids[:] = start + n_local + 1          # nothing routed to this slice
    B = int(rng.choice([1, 4, 8, 16]))
    cfg = None
    if seed % 2:
        cfg = P.gemm_config(L.GEMM_DECODE, int(rng.choice([2, 4])), int(rng.choice([1, 2, 4, 8])), 0)
    _compare(qtype, ids, start, B, cfg, seed)


def test_routed_two_batches():
    # 65..128 slots run as two 64-slot batches of one wave: ranks and block starts across the batches
    wl, W13 = _w13("nvfp4_g16")
    n_local, start = W13.desc.n_experts, wl.expert_start
    cases = [
        np.full((16, 8), start + 3),                                      # one expert, 128 slots
        np.concatenate([np.full(64, start + 3), np.full(64, start + 1)]).reshape(16, 8),  # later batch, lower expert
        np.concatenate([np.full(64, start + 2), np.full(1, start + 2)]).reshape(65, 1),   # 65 slots, one in batch 1
        np.concatenate([np.full(64, start + n_local + 5), np.arange(63) % n_local + start]).reshape(127, 1),  # batch 0 off-slice
        np.concatenate([np.arange(64) % n_local + start, np.full(64, -1)]).reshape(32, 4),                     # batch 1 junk
        (np.arange(128) * 7) % n_local + start,                           # every expert in both batches
    ]
    for i, ids in enumerate(cases):
        ids = np.asarray(ids, dtype=np.int32).reshape(-1, 8) if ids.size % 8 == 0 and ids.ndim == 1 else np.asarray(ids, dtype=np.int32)
        for B in (1, 5, 16):
            _compare("nvfp4_g16", ids, start, B, seed=i)


def test_routed_rejects_large_batches():
    wl, W13 = _w13("int4_g128")
    x = torch.zeros((65, wl.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((65, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="at most 128"):
        P.moe_w4a16_gemm_act_routed(wl.act, x, W13, ids, 0, 16)


@pytest.mark.parametrize("qtype,M", [("int4_g128", 1), ("int4_g128", 32), ("nvfp4_g16", 1), ("nvfp4_g16", 8),
                                     ("nvfp4_g16", 12), ("mxfp4_g32", 1), ("mxfp4_g32", 16)])
def test_layer_with_fused_align(qtype, M):
    # (nvfp4 M=12: 96 slots, about a quarter of them on the slice -- 16-slot blocks on the streaming
    # kernel, the align fused as two 64-slot batches)
    wl = W.small_workload(qtype)
    lw = W.make_weights(wl)
    inp = W.make_inputs(wl, M, seed=400 + M)
    layer = make_layer(wl, lw)
    x, ids, gw = W.device_inputs(inp)
    print(f"layer fused align {wl.name} M={M}", flush=True)
    got_f = layer(x, ids, gw, fused_align=True).clone()
    got_u = layer(x, ids, gw, fused_align=False).clone()
    torch.cuda.synchronize()
    assert torch.equal(got_f.view(torch.int16), got_u.view(torch.int16))
    ref = oracle_layer(wl, lw, inp)
    assert layer_violations(W.bf16_to_float(got_f), ref) == 0


def test_routed_auto_config_on_long_k_weights():
    # 40 slots of K = 2048 weights: for these moe_gemm_choose picks the MFMA kernel, while the fused
    # align runs only in the streaming kernel, which then takes its own default configuration
    wl = W.small_workload("nvfp4_g16", H=2048)
    lw = W.make_weights(wl)
    w13, _, _ = W.device_weights(lw)
    W13 = P.moe_w4a16_prepare("nvfp4_g16", w13["codes"], w13["scales"], w13.get("gs"), w13.get("bias"),
                              L.PREP_GATE_UP, w13.get("zeros"))
    M, k = 5, wl.top_k
    assert M * k >= 32 and P.gemm_choose(W13, M * k, 16, 256).kernel == L.GEMM_MFMA
    inp = W.make_inputs(wl, M, seed=900)
    x, ids, _ = W.device_inputs(inp)
    print(f"routed auto config nvfp4 K=2048 M={M} k={k}", flush=True)
    got, (s2, e2, n2, loc2) = P.moe_w4a16_gemm_act_routed(wl.act, x, W13, ids, wl.expert_start, 16, wl.alpha,
                                                           wl.limit)
    s, e, n, loc = P.moe_align(ids, wl.expert_start, W13.desc.n_experts, 16)
    ref = P.moe_w4a16_gemm_act(wl.act, x, W13, s, e, n, M * k, k, 16, wl.alpha, wl.limit)   # MFMA kernel
    torch.cuda.synchronize()
    assert int(n2.item()) == int(n.item())
    assert torch.equal(s2, s) and torch.equal(e2, e) and torch.equal(loc2, loc)
    live = torch.nonzero(loc.view(-1) >= 0).view(-1)
    assert live.numel() > 0
    g, r = W.bf16_to_float(got[live]), W.bf16_to_float(ref[live])
    # the same products in another fp32 summation order: gate and up each rounded to bf16, then the
    # activation, rounded again
    rms = float(np.sqrt(np.mean(r * r)))
    assert np.all(np.abs(g - r) <= 2.0 ** -6 * np.abs(r) + 2e-3 * rms), float(np.max(np.abs(g - r)))
