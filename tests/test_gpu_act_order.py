"""GPU parity of act-order int4 (g_idx grouping): the prepared column order, the activation
gather, and the whole layer against the CPU oracle for both int4 formats, on the streaming
(decode) and MFMA (prefill) GEMMs; the plain grouping given as act-order equals the plain layer
bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import announce, layer_violations, make_layer, oracle_layer, rel_rms

pytestmark = pytest.mark.gpu


def _act_order_workload(qtype, **kw):
    return W.small_workload(qtype).replace(act_order=True, **kw)


def _perm_of(Wp, E, K):
    """The prepared column order (int32 [E, K]) read back from the prepared buffer."""
    off = Wp.desc.perm - Wp.buffer.data_ptr()
    assert 0 <= off and off + E * K * 4 <= Wp.buffer.numel()
    return Wp.buffer[off: off + E * K * 4].view(torch.int32).view(E, K).cpu().numpy()


@pytest.mark.parametrize("qtype", ["int4_g128", "int4zp_g128", "int4zpf_g128"])
def test_prepared_column_order_is_the_stable_sort_of_g_idx(qtype):
    wl = _act_order_workload(qtype)
    lw = W.make_weights(wl)
    layer = make_layer(wl, lw)
    torch.cuda.synchronize()
    for Wp, ew in ((layer.W13, lw.w13), (layer.W2, lw.w2)):
        E, K = ew.g_idx.shape
        got = _perm_of(Wp, E, K)
        want = np.argsort(ew.g_idx, axis=1, kind="stable")
        assert np.array_equal(got, want)


@pytest.mark.parametrize("offset", [0, 1])
def test_permute_cols_matches_a_gather(offset):
    # offset 0: rows staged in LDS; offset 1: a source view 2 bytes off alignment (direct gather)
    from quantized_mixture_experts_align_amd import moe_permute_cols
    wl = _act_order_workload("int4_g128")
    lw = W.make_weights(wl)
    layer = make_layer(wl, lw)
    E, H = lw.w13.g_idx.shape
    rng = np.random.default_rng(3)
    M, k = 23, 3
    big = torch.from_numpy(rng.standard_normal((M, H + 8)).astype(np.float32)).to(torch.bfloat16).cuda()
    x = big[:, offset: offset + H]
    slot_e = rng.integers(-1, E + 1, size=M * k).astype(np.int32)        # dead (-1) and off-range (E)
    out = torch.full((M * k, H), 7.0, dtype=torch.bfloat16, device="cuda")
    moe_permute_cols(x, layer.W13, torch.from_numpy(slot_e).cuda(), k, out=out)
    torch.cuda.synchronize()
    perm = np.argsort(lw.w13.g_idx, axis=1, kind="stable")
    xs = x.cpu()
    for r in range(M * k):
        e = slot_e[r]
        if 0 <= e < E:
            assert torch.equal(out[r].cpu(), xs[r // k][torch.from_numpy(perm[e])]), r
        else:
            assert (out[r] == 7.0).all(), r


@pytest.mark.parametrize("qtype", ["int4_g128", "int4zp_g128", "int4zpf_g128"])
@pytest.mark.parametrize("M", [1, 4, 37, 300])
def test_act_order_layer_matches_oracle(qtype, M):
    # M = 1, 4, 37: 16-slot blocks (streaming kernel); M = 300: 64-slot blocks (MFMA kernel)
    wl = _act_order_workload(qtype, bias=True)
    lw = W.make_weights(wl)
    inp = W.make_inputs(wl, M, seed=M)
    layer = make_layer(wl, lw)
    ws = layer.workspace(M)
    announce(f"act-order layer {qtype} M={M} block_m={ws.block_m}")
    out = layer(*W.device_inputs(inp), ws=ws)
    torch.cuda.synchronize()
    got = W.bf16_to_float(out)
    ref = oracle_layer(wl, lw, inp)
    assert layer_violations(got, ref) == 0
    assert rel_rms(got, ref) < 0.01
    if not np.abs(ref).any():      # (a batch routed only off the slice: nothing to compare)
        return
    # the act-order weights differ from the plain reading of the same codes
    plain = oracle_layer(wl, W.LayerWeights(W.ExpertWeights(lw.w13.codes, lw.w13.scales, None, lw.w13.bias,
                                                             lw.w13.N, lw.w13.K, lw.w13.zeros),
                                            W.ExpertWeights(lw.w2.codes, lw.w2.scales, None, lw.w2.bias,
                                                            lw.w2.N, lw.w2.K, lw.w2.zeros), None), inp)
    assert rel_rms(plain, ref) > 0.1


@pytest.mark.parametrize("M", [4, 300])
def test_plain_grouping_as_act_order_equals_the_plain_layer(M):
    wl = W.small_workload("int4_g128").replace(bias=True)
    lw = W.make_weights(wl)
    inp = W.make_inputs(wl, M, seed=7)
    plain = make_layer(wl, lw)
    for ew in (lw.w13, lw.w2):
        ew.g_idx = np.tile((np.arange(ew.K) // 128).astype(np.int32), (wl.n_local, 1))
    ao = make_layer(wl, lw)
    assert all(ao.act_order) and not any(plain.act_order)
    xs = W.device_inputs(inp)
    a = plain(*xs)
    b = ao(*xs)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("variant", ["relu2", "interleaved"])
def test_act_order_with_relu2_and_interleaved_rows(variant):
    # the column order combined with the prepare's other row mappings: the non-gated relu2
    # projection (GEMM1 has I rows), and gate/up rows arriving interleaved (gate j = row 2j)
    kw = dict(act="relu2", routed_scaling_factor=0.625) if variant == "relu2" else dict(interleaved_w13=True)
    wl = _act_order_workload("int4_g128", bias=True, **kw)
    lw = W.make_weights(wl)
    for M in (5, 300):
        inp = W.make_inputs(wl, M, seed=11 + M)
        layer = make_layer(wl, lw)
        ws = layer.workspace(M)
        announce(f"act-order {variant} M={M} block_m={ws.block_m}")
        out = layer(*W.device_inputs(inp), ws=ws)
        torch.cuda.synchronize()
        got = W.bf16_to_float(out)
        ref = oracle_layer(wl, lw, inp)
        assert layer_violations(got, ref) == 0
        assert rel_rms(got, ref) < 0.01

