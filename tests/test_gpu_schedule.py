"""The prefill schedule on the GPU: the MFMA kernel's result does not depend on the align block
size, so skipping the all-padding 16-slot groups of an expert's last block changes no bit;
the residency that moe_gemm_choose weighs tile counts with comes from the occupancy API."""
import numpy as np
import pytest
import torch

import workloads as W
import quantized_mixture_experts_align_amd as P
from quantized_mixture_experts_align_amd import _lib as L

from gpu_util import announce, layer_violations, make_layer, oracle_layer

pytestmark = pytest.mark.gpu


def _skewed_ids(wl, M, seed):
    # Zipf-like: most slots on a few local experts, a long tail with 1..15 rows (ragged tails of
    # every length inside a 128-slot block), some slots off the slice
    rng = np.random.default_rng(seed)
    p = (np.arange(wl.n_global) + 1.0) ** -1.3
    p /= p.sum()
    ids = np.empty((M, wl.top_k), dtype=np.int32)
    for t in range(M):
        ids[t] = rng.choice(wl.n_global, size=wl.top_k, replace=False, p=p)
    return ids


@pytest.mark.parametrize("qtype", W.QTYPES)
def test_mfma_result_is_independent_of_block_size_under_skew(qtype):
    wl = W.small_workload(qtype)
    lw = W.make_weights(wl)
    layer = make_layer(wl, lw)
    M = 300
    inp = W.make_inputs(wl, M)
    inp = W.LayerInputs(inp.x, _skewed_ids(wl, M, 7), inp.topk_weights, M)
    outs = {}
    for B in (32, 64, 128):
        for ng in (2, 4):
            announce(f"schedule {qtype} B={B} ng={ng}")
            cfg = P.gemm_config(L.GEMM_MFMA, ng, 0, 0)
            x, ids, gw = W.device_inputs(inp)
            out = layer(x, ids, gw, ws=layer.workspace(M, B), cfg13=cfg, cfg2=cfg)
            torch.cuda.synchronize()
            outs[(B, ng)] = out.clone()
    ref = outs[(32, 2)]
    for key, o in outs.items():
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), key
    got = W.bf16_to_float(ref)
    assert layer_violations(got, oracle_layer(wl, lw, inp)) == 0


def test_occupancy_api_residency_and_the_choice_that_uses_it():
    wl = W.WORKLOADS[W.NVFP4_ZIPF].replace(n_local=2)       # the slice's shapes, two experts
    lw = W.make_weights(W.small_workload("nvfp4_g16").replace(H=4096, I=4096, n_local=2))
    layer = make_layer(W.small_workload("nvfp4_g16").replace(H=4096, I=4096, n_local=2), lw)
    for Wp, gated in ((layer.W13, True), (layer.W2, False)):
        for B in (32, 64, 128):
            r = P.gemm_occupancy(Wp, B, gated)
            announce(f"residency gated={gated} B={B}: {r}")
            assert r[1] >= 1 and r[2] >= 1 and r[1] >= r[2]
            assert (r[0] == 0) if gated else (r[0] >= r[1])
            # the choice without residency asks the device for exactly this
            for numel in (512, 4096, 32768):
                a = P.gemm_choose(Wp, numel, B, 256)
                b = P.gemm_choose(Wp, numel, B, 256, resident=r)
                assert (a.kernel, a.ng, a.group_m) == (b.kernel, b.ng, b.group_m)
    # the 128-slot, four-tile gate/up kernel fits two workgroups per CU (its launch bound)
    assert P.gemm_occupancy(layer.W13, 128, True)[2] >= 2
    del wl
