"""Per-kernel GPU parity: prepare + grouped GEMM (every kernel and tile shape), activation,
combine and the norm-weight binding, each against the oracle on the same inputs."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe as O
from oracle import formats as F
import quantized_mixture_experts_align_amd as P
from quantized_mixture_experts_align_amd import _lib as L

from gpu_util import gemm_tolerance, rel_rms

pytestmark = pytest.mark.gpu


def _bf16_dev(a_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a_bits.view(np.int16)).cuda().view(torch.bfloat16)


def _gemm_case(qtype, which, M, B, cfg, wl_kw=None):
    """Run GEMM1 (which=13) or GEMM2 (which=2) of a small workload on the GPU and return
    (got, ref) over the live slots, in prepared column order."""
    wl = W.small_workload(qtype, **(wl_kw or {}))
    lw = W.make_weights(wl)
    inp = W.make_inputs(wl, M)
    w13, w2, _ = W.device_weights(lw)
    if which == 13:
        flags = L.PREP_GATE_UP | (L.PREP_INTERLEAVED if wl.interleaved_w13 else 0)
        Wp = P.moe_w4a16_prepare(qtype, w13["codes"], w13["scales"], w13.get("gs"), w13.get("bias"), flags,
                                 w13.get("zeros"))
        proj, top_k = lw.w13, wl.top_k
        A_bits = inp.x
    else:
        Wp = P.moe_w4a16_prepare(qtype, w2["codes"], w2["scales"], w2.get("gs"), w2.get("bias"), 0, w2.get("zeros"))
        proj, top_k = lw.w2, 1
        rng = np.random.default_rng(M)
        A_bits = W._to_bf16_bits(rng.standard_normal((M * wl.top_k, wl.I)).astype(np.float32))
    ids = torch.from_numpy(inp.topk_ids).cuda()
    s, e, n, loc = P.moe_align(ids, wl.expert_start, wl.n_local, B)
    numel = M * wl.top_k
    out = P.moe_w4a16_gemm(_bf16_dev(A_bits), Wp, s, e, n, numel, top_k, B, cfg=cfg)
    torch.cuda.synchronize()
    got = W.bf16_to_float(out)
    local = loc.cpu().numpy().reshape(-1)
    A = F.decode_bf16(A_bits)
    rows = np.nonzero(local >= 0)[0]
    ref = np.zeros((rows.size, Wp.N))
    for j, slot in enumerate(rows):
        ex = local[slot]
        Wd = O.dequant(qtype, proj.codes[ex], proj.scales[ex], None if proj.gs is None else proj.gs[ex],
                       None if proj.zeros is None else proj.zeros[ex])
        h = Wd @ A[slot // top_k]
        if proj.bias is not None:
            h = h + F.decode_bf16(proj.bias[ex])
        if which == 13:
            g, u = O.split_gate_up(h, wl.interleaved_w13)
            h = np.concatenate([g, u])
        ref[j] = h
    return got[rows], ref, out[torch.from_numpy(rows).cuda()]   # rows of dead slots are never written


CFGS = {
    "decode_gemv": (16, P.gemm_config(L.GEMM_DECODE, 4, 4, 4)),
    "decode_mfma": (16, P.gemm_config(L.GEMM_DECODE, 2, 2, 0)),
    "decode_k1": (16, P.gemm_config(L.GEMM_DECODE, 1, 1, 2)),
    "decode_stream_ks8": (16, P.gemm_config(L.GEMM_DECODE, 2, 8, 0)),
    "decode_stream_ng4": (16, P.gemm_config(L.GEMM_DECODE, 4, 1, 0)),
    "decode_stream_ng1": (16, P.gemm_config(L.GEMM_DECODE, 1, 4, 0)),
    "mfma16": (16, P.gemm_config(L.GEMM_MFMA, 1, 0, 0)),
    "mfma32": (32, P.gemm_config(L.GEMM_MFMA, 2, 0, 0)),
    "mfma64": (64, P.gemm_config(L.GEMM_MFMA, 4, 0, 0)),
    "mfma128": (128, P.gemm_config(L.GEMM_MFMA, 4, 0, 0)),
    "auto": (None, None),
}


@pytest.mark.parametrize("which", [13, 2])
@pytest.mark.parametrize("kind", list(CFGS))
@pytest.mark.parametrize("qtype", W.QTYPES)
def test_gemm_matches_oracle(qtype, kind, which):
    B, cfg = CFGS[kind]
    M = 5 if kind.startswith("decode") else 61
    if B is None:
        wl = W.small_workload(qtype)
        B = P.choose_block_m(M * wl.top_k, wl.n_local, 0, wl.H)
    print(f"gemm {qtype} {kind} W{which} M={M} B={B}", flush=True)
    got, ref, _ = _gemm_case(qtype, which, M, B, cfg)
    err = np.abs(got - ref)
    assert np.all(err <= gemm_tolerance(ref)), f"max err {err.max()} rel rms {rel_rms(got, ref)}"
    assert rel_rms(got, ref) < (4e-3 if qtype in ("int4_g128", "int4zp_g128", "int4zpf_g128") else 2e-3)


@pytest.mark.parametrize("qtype", W.QTYPES)
def test_mfma_result_is_independent_of_tile_width(qtype):
    outs = []
    for ng in (1, 2, 4):
        print(f"mfma ng={ng} {qtype}", flush=True)
        _, _, out = _gemm_case(qtype, 13, 200, 64, P.gemm_config(L.GEMM_MFMA, ng, 0, 0))
        outs.append(out)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("kind", ["mfma16", "mfma64", "mfma128"])
@pytest.mark.parametrize("which", [13, 2])
def test_mfma_store_paths_agree(kind, which):
    # The MFMA epilogue stages its outputs through LDS and stores 16 bytes per lane when the output
    # is 16-byte aligned with a row pitch of a multiple of 8 elements, else 8 bytes per lane
    # directly: an output 8 bytes off alignment with a pitch of N + 4 takes the second path, and
    # both give the same bytes (columns beyond N untouched).
    B, cfg = CFGS[kind]
    qtype = "nvfp4_g16"
    wl = W.small_workload(qtype)
    lw = W.make_weights(wl)
    M = 61
    inp = W.make_inputs(wl, M)
    w13, w2, _ = W.device_weights(lw)
    if which == 13:
        Wp = P.moe_w4a16_prepare(qtype, w13["codes"], w13["scales"], w13.get("gs"), w13.get("bias"),
                                 L.PREP_GATE_UP, w13.get("zeros"))
        A, top_k = _bf16_dev(inp.x), wl.top_k
    else:
        Wp = P.moe_w4a16_prepare(qtype, w2["codes"], w2["scales"], w2.get("gs"), w2.get("bias"), 0, w2.get("zeros"))
        rng = np.random.default_rng(3)
        A = _bf16_dev(W._to_bf16_bits(rng.standard_normal((M * wl.top_k, wl.I)).astype(np.float32)))
        top_k = 1
    s, e, n, _ = P.moe_align(torch.from_numpy(inp.topk_ids).cuda(), wl.expert_start, wl.n_local, B)
    numel = M * wl.top_k
    N = Wp.N
    print(f"store paths W{which} {kind} N={N}", flush=True)
    aligned = torch.zeros((numel, N), dtype=torch.bfloat16, device="cuda")
    buf = torch.full((numel * (N + 4) + 4,), 7.0, dtype=torch.bfloat16, device="cuda")
    offset = buf[4:].view(numel, N + 4)
    assert offset.data_ptr() % 16 == 8 and (N + 4) % 8 == 4
    P.moe_w4a16_gemm(A, Wp, s, e, n, numel, top_k, B, out=aligned, cfg=cfg)
    P.moe_w4a16_gemm(A, Wp, s, e, n, numel, top_k, B, out=offset, cfg=cfg)
    torch.cuda.synchronize()
    live = torch.from_numpy(np.nonzero((inp.topk_ids.reshape(-1) >= wl.expert_start)
                                       & (inp.topk_ids.reshape(-1) < wl.expert_start + wl.n_local))[0]).cuda()
    assert torch.equal(aligned[live].view(torch.int16), offset[live, :N].contiguous().view(torch.int16))
    assert torch.all(offset[:, N:] == 7.0)
    if which == 13:   # the fused activation's epilogue (I = N / 2 columns per row)
        I = N // 2
        a_al = torch.zeros((numel, I), dtype=torch.bfloat16, device="cuda")
        buf2 = torch.full((numel * (I + 4) + 4,), 7.0, dtype=torch.bfloat16, device="cuda")
        a_off = buf2[4:].view(numel, I + 4)
        cfg_act = P.gemm_config(L.GEMM_MFMA, max(2, cfg.ng), 0, 0)   # (gate/up tile pairs)
        P.moe_w4a16_gemm_act("silu_mul", A, Wp, s, e, n, numel, top_k, B, out=a_al, cfg=cfg_act)
        P.moe_w4a16_gemm_act("silu_mul", A, Wp, s, e, n, numel, top_k, B, out=a_off, cfg=cfg_act)
        torch.cuda.synchronize()
        assert torch.equal(a_al[live].view(torch.int16), a_off[live, :I].contiguous().view(torch.int16))
        assert torch.all(a_off[:, I:] == 7.0)


@pytest.mark.parametrize("gemv_rows", [4, 0])
def test_decode_is_reproducible(gemv_rows):
    cfg = P.gemm_config(L.GEMM_DECODE, 2, 4, gemv_rows)
    a = _gemm_case("nvfp4_g16", 13, 3, 16, cfg)[2]
    b = _gemm_case("nvfp4_g16", 13, 3, 16, cfg)[2]
    assert torch.equal(a, b)


def test_gemm_pad_intermediate():
    # I = 288 is not a multiple of 64: the down projection's K is padded to 320 with zeros
    wl = W.small_workload("mxfp4_g32", I=288, H=448)
    lw = W.make_weights(wl)
    w13, w2, _ = W.device_weights(lw)
    Wp = P.moe_w4a16_prepare("mxfp4_g32", w2["codes"], w2["scales"], None, w2["bias"], L.PREP_PAD)
    assert Wp.K == 320 and Wp.N == 448
    W13 = P.moe_w4a16_prepare("mxfp4_g32", w13["codes"], w13["scales"], None, w13["bias"],
                              L.PREP_GATE_UP | L.PREP_INTERLEAVED | L.PREP_PAD)
    assert W13.N == 640


@pytest.mark.parametrize("kind,limit", [("silu_mul", math.inf), ("swiglu_alpha", math.inf), ("swiglu_alpha", 7.0),
                                        ("relu2", math.inf)])
def test_act_matches_oracle(kind, limit):
    rng = np.random.default_rng(3)
    R, I = 77, 320
    cols = I if kind == "relu2" else 2 * I
    h_bits = W._to_bf16_bits((rng.standard_normal((R, cols)) * 3).astype(np.float32))
    loc = rng.integers(-1, 4, size=R).astype(np.int32)
    out = torch.full((R, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    P.moe_act(kind, _bf16_dev(h_bits), I, torch.from_numpy(loc).cuda(), 1.702, limit, out=out)
    torch.cuda.synchronize()
    got = W.bf16_to_float(out)
    h = F.decode_bf16(h_bits)
    g, u = h[:, :I], h[:, I:]
    if kind == "relu2":
        ref = O.act_relu2(h)
    else:
        ref = O.act_silu_mul(g, u) if kind == "silu_mul" else O.act_swiglu_alpha(g, u, 1.702, limit)
    live = loc >= 0
    assert np.all(np.isnan(got[~live]))                 # dead rows untouched
    err = np.abs(got[live] - ref[live])
    assert np.all(err <= 2.0 ** -8 * np.abs(ref[live]) + 1e-6), err.max()


# single-pass kernel (top_k <= 8, H <= 8192; M <= 256 also reads y of dead slots, unused) and
# the two-pass kernel beyond that
@pytest.mark.parametrize("H,norm,M,k", [(512, False, 45, 8), (512, False, 2305, 2), (256, False, 18, 3),
                                        (4096, True, 45, 8), (2880, False, 45, 8),
                                        (2880, True, 45, 8), (64, True, 45, 8), (4096, True, 300, 8),
                                        (512, False, 300, 2), (2880, True, 45, 4), (8192, True, 20, 8),
                                        (512, True, 20, 16), (16384, True, 5, 8)])
@pytest.mark.parametrize("rsf", [1.0, 2.5])
def test_combine_matches_oracle(H, norm, M, k, rsf):
    rng = np.random.default_rng(H + M + k)
    y_bits = W._to_bf16_bits(rng.standard_normal((M * k, H)).astype(np.float32))
    g = rng.random((M, k)).astype(np.float32)
    loc = rng.integers(-1, 3, size=(M, k)).astype(np.int32)
    loc[0] = -1                                            # a token with no live slot
    y_dev = _bf16_dev(y_bits)
    y_dev.view(M, k, H)[torch.from_numpy(loc < 0).cuda()] = float("nan")   # dead rows never read
    nw_bits = W._to_bf16_bits(rng.normal(0, 0.1, H).astype(np.float32)) if norm else None
    nw_dev = P.moe_norm_weight(_bf16_dev(nw_bits)) if norm else None
    out = P.moe_combine(y_dev, torch.from_numpy(g).cuda(), torch.from_numpy(loc).cuda(), nw_dev, 1e-8,
                        routed_scaling_factor=rsf)
    torch.cuda.synchronize()
    got = W.bf16_to_float(out)
    ref = O.combine(F.decode_bf16(y_bits), g, loc, O.norm_weight(nw_bits) if norm else None, 1e-8, rsf)
    assert np.all(got[0] == 0)
    err = np.abs(got - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref ** 2))), err.max()
    if norm:
        assert np.array_equal(W.bf16_to_float(nw_dev), O.norm_weight(nw_bits))


@pytest.mark.parametrize("act", ["own", "relu2"])
@pytest.mark.parametrize("kind", ["decode", "decode_gemv", "mfma"])
@pytest.mark.parametrize("qtype", W.QTYPES)
def test_fused_activation_equals_gemm_then_act(qtype, kind, act):
    """GEMM1 with the activation in its epilogue gives the same bytes as moe_w4a16_gemm
    followed by moe_act (both round the GEMM values to bf16 before the activation); "own" is
    the workload's gated activation, relu2 the non-gated one (a plain projection)."""
    wl = W.small_workload(qtype)
    if act == "relu2":
        wl = wl.replace(act="relu2", interleaved_w13=False)
    lw = W.make_weights(wl)
    ng = 1 if act == "relu2" else 2
    M, B, cfg = {"decode": (5, 16, P.gemm_config(L.GEMM_DECODE, ng, 4, 0)),
                 "decode_gemv": (5, 16, P.gemm_config(L.GEMM_DECODE, 2, 2, 2)),
                 "mfma": (150, 64, P.gemm_config(L.GEMM_MFMA, ng, 0, 0))}[kind]
    inp = W.make_inputs(wl, M)
    w13, _, _ = W.device_weights(lw)
    flags = 0 if act == "relu2" else L.PREP_GATE_UP | (L.PREP_INTERLEAVED if wl.interleaved_w13 else 0)
    W13 = P.moe_w4a16_prepare(qtype, w13["codes"], w13["scales"], w13.get("gs"), w13.get("bias"), flags,
                              w13.get("zeros"))
    s, e, n, loc = P.moe_align(torch.from_numpy(inp.topk_ids).cuda(), wl.expert_start, wl.n_local, B)
    x = _bf16_dev(inp.x)
    numel = M * wl.top_k
    h = P.moe_w4a16_gemm(x, W13, s, e, n, numel, wl.top_k, B, cfg=cfg)
    I = W13.N if act == "relu2" else W13.N // 2
    a_ref = P.moe_act(wl.act, h, I, loc.view(-1), wl.alpha, 7.0)
    a = P.moe_w4a16_gemm_act(wl.act, x, W13, s, e, n, numel, wl.top_k, B, wl.alpha, 7.0, cfg=cfg)
    torch.cuda.synchronize()
    live = torch.from_numpy(np.nonzero(loc.cpu().numpy().reshape(-1) >= 0)[0]).cuda()
    assert torch.equal(a[live], a_ref[live])
