"""Full-size parity with deterministic coverage, in the launch configuration bench.py times.

For the large workloads (NVFP4 slice with Zipf routing at 256 / 1024 / 4096 tokens and with
uniform routing at 23296, the NVFP4 decode slice at 64, MXFP4 GPT-OSS at 2048):

* GEMM level: every slot routed to the hottest, a middle and the last non-empty local expert
  is compared element by element with the float64 oracle -- the gate/up GEMM with its fused
  activation against the oracle's activated intermediate on the same input rows, and the down
  GEMM against the float64 product of the same expert's weights with the GPU's own activated
  rows (so each GEMM is checked on its own input);
* layer level: tokens are chosen from the align output so that every local expert, every
  expert's last (partly padded) block, every 16-slot group position of a block and every row
  position inside a group are hit, and their outputs are compared with the oracle's layer.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe as O
from oracle import formats as F

from gpu_util import announce, gemm_tolerance, layer_violations, make_layer, oracle_layer, rel_rms

pytestmark = pytest.mark.gpu

CELLS = [(W.NVFP4_ZIPF, 256), (W.NVFP4_ZIPF, 1024), (W.NVFP4_ZIPF, 4096), (W.NVFP4_DECODE, 64),
         (W.MXFP4_SWIGLU, 2048), (W.NVFP4_UNIFORM, 23296)]

_CACHE = {}


def _layer(name):
    wl = W.WORKLOADS[name]
    if _CACHE.get("seed") != wl.seed:
        _CACHE.clear()
        torch.cuda.empty_cache()
        lw = W.make_weights(wl)
        _CACHE.update(seed=wl.seed, lw=lw, layer=make_layer(wl, lw))
    return wl, _CACHE["lw"], _CACHE["layer"]


def _run(name, M):
    """One eager forward with the layer's default configuration (the one bench.py graphs) and
    everything the checks need from it."""
    wl, lw, layer = _layer(name)
    inp = W.make_inputs(wl, M)
    x, ids, gw = W.device_inputs(inp)
    ws = layer.workspace(M, device=x.device)
    out = layer(x, ids, gw, ws=ws)
    torch.cuda.synchronize()
    numel = M * wl.top_k
    return dict(wl=wl, lw=lw, layer=layer, inp=inp, ws=ws, out=W.bf16_to_float(out),
                a=W.bf16_to_float(ws.a[:numel]),
                y=W.bf16_to_float(ws.buf13[: numel * layer.H].view(numel, layer.H)),
                sorted=ws.sorted_ids.cpu().numpy(), eids=ws.expert_ids.cpu().numpy(),
                ntpp=int(ws.ntpp.item()), B=ws.block_m)


def act_tolerance(ref: np.ndarray) -> np.ndarray:
    """Bound for the activated intermediate a = bf16(act(bf16(h))) against the oracle's.  Both
    sides round h to bf16, from an fp32 sum on the GPU and from the float64 one in the oracle, so
    near a rounding boundary of h they may pick neighbouring values (1 ulp of gate or up); the
    activation passes that on as about one ulp of a (silu(g) u and the SwiGLU variant are linear
    in up and close to linear in a large gate), and a's own rounding can add one more.  Three bf16
    ulps are at most 3 * 2^-7 |a| < 2^-5 |a|; the RMS term covers small |a| near a zero of the
    activation, where the relative effect of a gate flip is larger."""
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return 2.0 ** -5 * np.abs(ref) + 0.01 * rms + 1e-30


def _dequant(p, e, qtype):
    return O.dequant(qtype, p.codes[e], p.scales[e], None if p.gs is None else p.gs[e],
                     None if p.zeros is None else p.zeros[e])


def _act(wl, h):
    gate, up = O.split_gate_up(h, wl.interleaved_w13)
    if wl.act == "silu_mul":
        return O.act_silu_mul(gate, up)
    return O.act_swiglu_alpha(gate, up, wl.alpha, wl.limit)


@pytest.mark.parametrize("name,M", CELLS)
def test_gemms_on_every_slot_of_hot_middle_and_last_expert(name, M):
    r = _run(name, M)
    wl, lw, inp = r["wl"], r["lw"], r["inp"]
    local = O.route_local(inp.topk_ids, wl.expert_start, wl.n_local).reshape(-1)
    counts = np.bincount(local[local >= 0], minlength=wl.n_local)
    live = np.nonzero(counts)[0]
    order = live[np.argsort(-counts[live], kind="stable")]
    experts = sorted({int(order[0]), int(order[len(order) // 2]), int(live[-1])})
    x = F.decode_bf16(inp.x)
    for e in experts:
        slots = np.nonzero(local == e)[0]
        announce(f"full-size GEMMs {name} M={M} expert {e}: {slots.size} slots")
        # gate/up GEMM + activation: the oracle's stored intermediates (bf16 h, bf16 a)
        W13 = _dequant(lw.w13, e, wl.qtype)
        h = x[slots // wl.top_k] @ W13.T
        if lw.w13.bias is not None:
            h = h + F.decode_bf16(lw.w13.bias[e])[None, :]
        ref_a = O.round_to_bf16(_act(wl, O.round_to_bf16(h)))
        got_a = r["a"][slots][:, : wl.I]
        err = np.abs(got_a - ref_a)
        assert np.all(err <= act_tolerance(ref_a)), f"gate/up expert {e}: max err {err.max()}"
        assert rel_rms(got_a, ref_a) < 2e-3
        # down GEMM on the GPU's own activated rows, against the float64 product
        W2 = _dequant(lw.w2, e, wl.qtype)
        ref_y = got_a @ W2.T
        if lw.w2.bias is not None:
            ref_y = ref_y + F.decode_bf16(lw.w2.bias[e])[None, :]
        got_y = r["y"][slots]
        err = np.abs(got_y - ref_y)
        assert np.all(err <= gemm_tolerance(ref_y)), f"down expert {e}: max err {err.max()}"
        assert rel_rms(got_y, ref_y) < 2e-3


def _covering_tokens(r):
    """Tokens whose slots cover every align block's 16-slot group positions and row positions
    (cycling over blocks), every expert's last block and its last live row."""
    B, ntpp, k = r["B"], r["ntpp"], r["wl"].top_k
    numel = r["inp"].M * k
    sorted_ids = r["sorted"][:ntpp]
    groups = max(1, B // 16)
    picks = set()
    nblocks = ntpp // B
    for b in range(nblocks):
        rows = sorted_ids[b * B:(b + 1) * B]
        nlive = int(np.sum(rows < numel))
        if nlive == 0:
            continue
        # one slot at group position b mod groups, row position b mod 16 (clamped to live rows)
        pos = min((b % groups) * 16 + (b // groups) % 16, nlive - 1)
        picks.add(int(rows[pos]))
        last_block = b + 1 == nblocks or r["eids"][b + 1] != r["eids"][b]
        if last_block:
            picks.add(int(rows[nlive - 1]))            # the expert's last live row
            for g in range(groups):                    # and every group of its last block
                if g * 16 < nlive:
                    picks.add(int(rows[g * 16]))
    # the first full block: every row position of every group
    full = next((b for b in range(nblocks) if np.all(sorted_ids[b * B:(b + 1) * B] < numel)), None)
    if full is not None:
        for g in range(groups):
            picks.add(int(sorted_ids[full * B + g * 16 + (g % 16)]))
    return np.array(sorted({s // k for s in picks}), dtype=np.int64)


@pytest.mark.parametrize("name,M", CELLS)
def test_layer_on_tokens_covering_every_block_position(name, M):
    r = _run(name, M)
    wl, lw, inp = r["wl"], r["lw"], r["inp"]
    toks = _covering_tokens(r)
    local = O.route_local(inp.topk_ids, wl.expert_start, wl.n_local)
    hit = np.unique(local[toks][local[toks] >= 0])
    assert np.array_equal(hit, np.unique(local[local >= 0]))   # every non-empty expert is hit
    announce(f"full-size layer {name} M={M}: {toks.size} covering tokens, block_m {r['B']}")
    ref = oracle_layer(wl, lw, inp, tokens=toks)
    got = r["out"][toks]
    assert layer_violations(got, ref) == 0
    assert rel_rms(got, ref) < 0.01
