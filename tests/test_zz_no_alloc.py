"""moe_w4a16_gemm_combine_noalloc (the fused down GEMM + weighted sum with its arrival counters in
the library's own scratch memory, for callers that cannot allocate): called through the C ABI, its
outputs equal those of moe_w4a16_gemm_combine with caller-owned counters bit for bit, on two calls
in a row (the second on a smaller batch), for every weight format; batches beyond the scratch
array's size are rejected before any launch."""
import numpy as np
import pytest
import torch

import workloads as W
import quantized_mixture_experts_align_amd as P
from quantized_mixture_experts_align_amd import _lib as L
from quantized_mixture_experts_align_amd import ops

pytestmark = pytest.mark.gpu


def _setup(qtype):
    wl = W.small_workload(qtype, norm=False)
    lw = W.make_weights(wl)
    _, w2, _ = W.device_weights(lw)
    W2 = P.moe_w4a16_prepare(qtype, w2["codes"], w2["scales"], w2.get("gs"), w2.get("bias"), 0, w2.get("zeros"))
    return wl, W2


def _batch(wl, W2, M, seed, B):
    rng = np.random.default_rng(seed)
    k = wl.top_k
    ids = W.make_inputs(wl, M, seed=seed).topk_ids
    a = torch.from_numpy(W._to_bf16_bits(rng.standard_normal((M * k, W2.K)).astype(np.float32)).view(np.int16))
    a = a.cuda().view(torch.bfloat16)
    gw = torch.from_numpy(rng.random((M, k), dtype=np.float32)).cuda()
    s, e, n, loc = P.moe_align(torch.from_numpy(ids).cuda(), wl.expert_start, W2.desc.n_experts, B)
    return a, gw, s, e, n, loc


@pytest.mark.parametrize("qtype", W.QTYPES)
def test_noalloc_equals_caller_counters_on_two_calls(qtype):
    wl, W2 = _setup(qtype)
    B = 16
    for M, seed, rsf in ((8, 900, 1.0), (3, 901, 1.75)):       # the second call on a smaller batch
        print(f"noalloc {qtype} M={M}", flush=True)
        a, gw, s, e, n, loc = _batch(wl, W2, M, seed, B)
        numel = M * wl.top_k
        counters = P.combine_counters(M, W2, a.device)
        y_ref = torch.full((numel, W2.N), 7.0, dtype=torch.bfloat16, device="cuda")
        ref = torch.full((M, W2.N), 7.0, dtype=torch.bfloat16, device="cuda")
        P.moe_w4a16_gemm_combine(a, W2, s, e, n, gw, loc, B, counters, y_ref, out=ref, routed_scaling_factor=rsf)
        y = torch.full((numel, W2.N), 7.0, dtype=torch.bfloat16, device="cuda")
        out = torch.full((M, W2.N), 7.0, dtype=torch.bfloat16, device="cuda")
        ops.moe_w4a16_gemm_combine_noalloc(a, W2, s, e, n, gw, loc, B, y, out, routed_scaling_factor=rsf)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))       # every row
        live = torch.nonzero(loc.view(-1) >= 0).view(-1)
        assert torch.equal(y[live].view(torch.int16), y_ref[live].view(torch.int16))


def test_noalloc_rejects_batches_beyond_its_scratch():
    wl, W2 = _setup("mxfp4_g32")
    strips = -(-(W2.N // 16) // 4)                  # four tiles per wave: the fewest strips
    M = L.NOALLOC_MAX_COUNTERS // strips + 1
    cfg = P.gemm_config(L.GEMM_DECODE, 4, 1, 0)
    a = torch.zeros((M * wl.top_k, W2.K), dtype=torch.bfloat16, device="cuda")
    gw = torch.zeros((M, wl.top_k), dtype=torch.float32, device="cuda")
    loc = torch.full((M, wl.top_k), -1, dtype=torch.int32, device="cuda")
    s = torch.zeros(16, dtype=torch.int32, device="cuda")
    y = torch.empty((1, W2.N), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, W2.N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="scratch"):
        ops.moe_w4a16_gemm_combine_noalloc(a, W2, s, s, s, gw, loc, 16, y, out, cfg=cfg)
