"""The align's block schedule (moe_align_sched) and the MFMA GEMM's use of it.

The schedule is a launch order, not part of the method: its expected value is its definition
(in `_expected`) applied to the oracle's align, and a GEMM that takes its blocks in it must give the
same bytes as one that takes them in align order."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe as O
import quantized_mixture_experts_align_amd as P
from quantized_mixture_experts_align_amd import _lib as L

pytestmark = pytest.mark.gpu


def _expected(ids, start, n_local, B):
    """The schedule's definition on the oracle's align: the live blocks stable-sorted by falling
    count of live 16-slot groups, then -1 up to the capacity."""
    rs, _, rn, _ = O.moe_align(ids, start, n_local, B)
    numel = ids.size
    nb = rn // B
    groups = [-(-int((rs[b * B:(b + 1) * B] < numel).sum()) // 16) for b in range(nb)]
    order = sorted(range(nb), key=lambda b: (-groups[b], b))
    _, cap_blocks = P.align_capacity(ids.shape[0], ids.shape[1], n_local, B)
    return np.array(order + [-1] * (cap_blocks - nb), dtype=np.int32)


def _check(ids, start, n_local, B):
    print(f"schedule M={ids.shape[0]} k={ids.shape[1]} start={start} n_local={n_local} B={B}", flush=True)
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    plain = P.moe_align(t, start, n_local, B)
    _, b_len = P.align_capacity(ids.shape[0], ids.shape[1], n_local, B)
    sched = torch.full((b_len,), -7, dtype=torch.int32, device="cuda")
    with_s = P.moe_align(t, start, n_local, B, schedule=sched)
    torch.cuda.synchronize()
    for a, b in zip(plain, with_s):   # the align outputs are unchanged, bit for bit
        assert torch.equal(a, b)
    assert np.array_equal(sched.cpu().numpy(), _expected(ids, start, n_local, B))


@pytest.mark.parametrize("name,M,B", [(W.INT4_BIAS, 2304, 64), (W.NVFP4_ZIPF, 256, 64), (W.NVFP4_ZIPF, 1024, 128),
                                      (W.NVFP4_ZIPF, 4096, 128), (W.NVFP4_UNIFORM, 5760, 128),
                                      (W.NVFP4_UNIFORM, 23296, 128), (W.MXFP4_SWIGLU, 2048, 128),
                                      (W.NVFP4_DECODE, 64, 16)])
def test_schedule_workload_routing(name, M, B):
    wl = W.WORKLOADS[name]
    _check(W.make_inputs(wl, M).topk_ids, wl.expert_start, wl.n_local, B)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("B", [1, 7, 16, 20, 32, 64, 128, 256])
def test_schedule_random_slices(seed, B):
    # junk ids, up to 512 local experts, one and several align workgroups (over 4096 slots)
    rng = np.random.default_rng(500 + seed)
    M, k = int(rng.choice([1, 37, 700, 1500])), int(rng.integers(1, 9))
    n_local = int(rng.choice([1, 3, 32, 128, 300, 512]))
    start = int(rng.integers(0, 50))
    ids = rng.integers(-5, start + n_local + 40, size=(M, k)).astype(np.int32)
    _check(ids, start, n_local, B)


def test_schedule_edge_cases():
    rng = np.random.default_rng(12)
    _check(np.zeros((0, 8), np.int32), 0, 32, 64)                          # no tokens
    _check(np.full((37, 4), 1000, np.int32), 0, 128, 32)                   # everything off-slice
    _check(np.full((300, 2), 5, np.int32), 5, 1, 64)                       # one expert, short last block
    _check(np.full((256, 2), 5, np.int32), 5, 1, 128)                      # one expert, whole blocks
    # every expert an exact multiple of the block (all blocks full)
    _check(np.repeat(np.arange(16, dtype=np.int32), 64).reshape(-1, 4), 0, 16, 32)
    # last blocks one row short of full and one row long: 16-slot group counts 8 and 1
    ids = np.concatenate([np.full(127, 0), np.full(129, 1), np.full(113, 2), np.full(112, 3)]).astype(np.int32)
    _check(ids.reshape(-1, 1), 0, 4, 128)
    _check(rng.integers(0, 1024, (2000, 8)).astype(np.int32), 256, 512, 128)  # 512 experts, 4 spans


def _gemm_pair(qtype, which, M, B, ng, group_m, act=None):
    wl = W.small_workload(qtype)
    lw = W.make_weights(wl)
    inp = W.make_inputs(wl, M)
    w13, w2, _ = W.device_weights(lw)
    if which == 13:
        flags = L.PREP_GATE_UP | (L.PREP_INTERLEAVED if wl.interleaved_w13 else 0)
        Wp = P.moe_w4a16_prepare(qtype, w13["codes"], w13["scales"], w13.get("gs"), w13.get("bias"), flags,
                                 w13.get("zeros"))
        A = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
        top_k = wl.top_k
    else:
        Wp = P.moe_w4a16_prepare(qtype, w2["codes"], w2["scales"], w2.get("gs"), w2.get("bias"), 0, w2.get("zeros"))
        rng = np.random.default_rng(M)
        bits = W._to_bf16_bits(rng.standard_normal((M * wl.top_k, wl.I)).astype(np.float32))
        A = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        top_k = 1
    ids = torch.from_numpy(inp.topk_ids).cuda()
    _, b_len = P.align_capacity(M, wl.top_k, wl.n_local, B)
    sched = torch.empty(b_len, dtype=torch.int32, device="cuda")
    s, e, n, loc = P.moe_align(ids, wl.expert_start, wl.n_local, B, schedule=sched)
    numel = M * wl.top_k
    outs = []
    for bo in (None, sched):
        cfg = P.gemm_config(L.GEMM_MFMA, ng, 0, 0, group_m, bo)
        if act is None:
            outs.append(P.moe_w4a16_gemm(A, Wp, s, e, n, numel, top_k, B, cfg=cfg))
        else:
            outs.append(P.moe_w4a16_gemm_act(act, A, Wp, s, e, n, numel, top_k, B, cfg=cfg))
    torch.cuda.synchronize()
    live = torch.nonzero(loc.view(-1) >= 0).view(-1)
    return outs[0][live], outs[1][live], sched


@pytest.mark.parametrize("qtype", ["nvfp4_g16", "int4_g128", "mxfp4_g32"])
@pytest.mark.parametrize("B,ng", [(32, 2), (64, 4), (128, 4), (128, 1)])
@pytest.mark.parametrize("group_m", [1, 2, 8])
@pytest.mark.parametrize("which", [13, 2])
def test_gemm_with_schedule_is_bitwise_equal(qtype, B, ng, group_m, which):
    print(f"gemm schedule {qtype} W{which} B={B} ng={ng} group_m={group_m}", flush=True)
    a, b, sched = _gemm_pair(qtype, which, 300, B, ng, group_m)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    if B == 32:   # (here every expert has whole blocks and a short last one: the order changes)
        s = sched.cpu().numpy()
        nb = int((s >= 0).sum())
        assert nb > 4 and not np.array_equal(s[:nb], np.arange(nb))


@pytest.mark.parametrize("qtype,act", [("nvfp4_g16", "silu_mul"), ("mxfp4_g32", "swiglu_alpha")])
@pytest.mark.parametrize("B", [32, 128])
def test_fused_act_gemm_with_schedule_is_bitwise_equal(qtype, act, B):
    a, b, _ = _gemm_pair(qtype, 13, 300, B, 4, 1, act=act)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_schedule_naming_no_block_skips_it():
    # a schedule whose entries name no live block: its workgroups exit, nothing is written
    qtype, B = "nvfp4_g16", 64
    wl = W.small_workload(qtype)
    lw = W.make_weights(wl)
    inp = W.make_inputs(wl, 100)
    _, w2, _ = W.device_weights(lw)
    Wp = P.moe_w4a16_prepare(qtype, w2["codes"], w2["scales"], w2.get("gs"), None, 0)
    s, e, n, _ = P.moe_align(torch.from_numpy(inp.topk_ids).cuda(), wl.expert_start, wl.n_local, B)
    numel = 100 * wl.top_k
    A = torch.ones((numel, wl.I), dtype=torch.bfloat16, device="cuda")
    _, b_len = P.align_capacity(100, wl.top_k, wl.n_local, B)
    for fill in (-1, 1 << 20, 0x7FFFFFF0):
        bad = torch.full((b_len,), fill, dtype=torch.int32, device="cuda")
        out = torch.full((numel, Wp.N), 3.0, dtype=torch.bfloat16, device="cuda")
        P.moe_w4a16_gemm(A, Wp, s, e, n, numel, 1, B, out=out, cfg=P.gemm_config(L.GEMM_MFMA, 2, 0, 0, 1, bad))
        torch.cuda.synchronize()
        assert torch.all(out == 3.0)


@pytest.mark.parametrize("qtype,B,H,I", [("nvfp4_g16", 64, 2048, 2048), ("mxfp4_g32", 128, 2048, 2112),
                                         ("int4_g128", 32, 512, 384)])
def test_layer_schedule_is_bitwise_equal(qtype, B, H, I):
    # the layer's workspace carries the schedule for long-K weights (both K >= 2048); the same
    # layer without it gives the same bytes.  Short K (int4 here): no schedule.
    from gpu_util import make_layer
    wl = W.small_workload(qtype, H=H, I=I)
    layer = make_layer(wl, W.make_weights(wl))
    M = 300
    x, ids, gw = W.device_inputs(W.make_inputs(wl, M))
    ws = layer.workspace(M, block_m=B)
    if min(H, I) < 2048:
        assert ws.sched is None
        return
    assert ws.sched is not None and all(c.block_order == ws.sched.data_ptr() for c in ws.cfgs)
    y1 = layer(x, ids, gw, ws=ws).clone()
    c13, c2 = (P.gemm_config(c.kernel, c.ng, c.ksplit, c.gemv_rows, c.group_m) for c in ws.cfgs)
    y2 = layer(x, ids, gw, ws=ws, cfg13=c13, cfg2=c2).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
