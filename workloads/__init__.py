"""Seeded synthetic inputs for the W4A16 MoE expert layer.

This module only draws random data in the canonical layouts; it holds none of
the layer's arithmetic (no dequantisation, routing, GEMM, activation or
combine).  Both the CPU oracle (through the tests) and the HIP path consume
exactly the arrays produced here, so the two sides see identical bytes.

Canonical layouts (shared vocabulary of every caller):

* ``codes``   uint8 ``[E, N, K/2]``: two 4-bit codes per byte, the low nibble
  holds the even K index.
* ``scales``  ``[E, N, K/g]``: bf16 bit patterns (uint16) for int4 (g = 128),
  float8 e4m3fn codes (uint8) for NVFP4 (g = 16), E8M0 codes (uint8) for
  MXFP4 (g = 32).
* ``gs``      float32 ``[E]``: NVFP4 per-expert global scale (else ``None``).
* ``zeros``   uint8 ``[E, N, K/128]``: zero points 0..15 of the asymmetric int4
  format (``int4zp_g128``: unsigned codes, bf16 scales like int4); float16 bit
  patterns (uint16) in the same layout for the float zero-point format
  (``int4zpf_g128``); else ``None``.
* ``bias``    bf16 bits ``[E, N]`` or ``None``.
* ``x``       bf16 bits ``[M, H]``; ``topk_ids`` int32 ``[M, k]`` global ids;
  ``topk_weights`` float32 ``[M, k]``; ``norm_w`` bf16 bits ``[H]``.

For the gate/up projection N = 2I with gate rows ``[0, I)`` then up rows
``[I, 2I)``, except for the MXFP4 workload whose rows arrive interleaved
(``gate0, up0, gate1, up1, ...``) the way GPT-OSS checkpoints store them.

Workloads follow the shapes of the pages: the sglang Marlin MoE unit test
(int4, E=8, top-2, H=512, I=1024), the Muse Spark EP8 expert slice (NVFP4,
256 experts of which 32 are local, top-8, H=I=4096) and GPT-OSS MXFP4
(E=128, top-4, H=I=2880).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

QTYPES = ("int4_g128", "nvfp4_g16", "mxfp4_g32", "int4zp_g128", "int4zpf_g128")
GROUP = {"int4_g128": 128, "nvfp4_g16": 16, "mxfp4_g32": 32, "int4zp_g128": 128, "int4zpf_g128": 128}

# stream ids of the seed sequence
_S_WEIGHTS, _S_HIDDEN, _S_ROUTING, _S_AUX = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    """One layer configuration; ``M`` tokens are drawn per call of make_inputs."""
    name: str
    qtype: str
    n_global: int          # experts in the model
    expert_start: int      # first local expert
    n_local: int           # local experts [expert_start, expert_start + n_local)
    top_k: int
    H: int
    I: int
    Ms: tuple
    bias: bool = False
    act: str = "silu_mul"  # or "swiglu_alpha", or "relu2" (non-gated: GEMM1 has I rows)
    routed_scaling_factor: float = 1.0
    alpha: float = 1.702
    limit: float = float("inf")
    norm: bool = False
    eps: float = 1e-8
    interleaved_w13: bool = False
    routing: str = "uniform"   # or "zipf"
    zipf_s: float = 1.2
    seed: int = 0              # seed id of the weights (and default input seed)
    act_order: bool = False    # int4 formats: a random g_idx per expert and projection

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def group(self) -> int:
        return GROUP[self.qtype]


# The workloads, by name: int4 layers of 8 experts (123 tokens; 2304 tokens with biases),
# one GPU's NVFP4 slice of 32 of 256 experts (uniform decode batches; Zipf-routed prefill
# batches, same weights), a 128-expert MXFP4 GPT-OSS-style layer, and the int4 layer's shapes
# with asymmetric int4 weights (integer zero points; float16 zero points, with biases) and
# with act-order (g_idx) int4 weights.
WORKLOADS = {w.name: w for w in [
    Workload("int4_m123_e8_top2_h512_i1024", "int4_g128", 8, 0, 8, 2, 512, 1024,
             (123,), seed=0),
    Workload("int4_bias_m2304_e8_top2_h512_i1024", "int4_g128", 8, 0, 8, 2, 512, 1024,
             (2304,), bias=True, seed=1),
    Workload("nvfp4_ep8_slice_decode_h4096_i4096", "nvfp4_g16", 256, 0, 32, 8, 4096, 4096,
             (1, 4, 16, 64), norm=True, seed=2),
    Workload("nvfp4_ep8_slice_zipf_prefill_h4096_i4096", "nvfp4_g16", 256, 0, 32, 8, 4096, 4096,
             (256, 1024, 4096), norm=True, routing="zipf", seed=2),
    Workload("mxfp4_swiglu_e128_top4_h2880_i2880", "mxfp4_g32", 128, 0, 128, 4, 2880, 2880,
             (1, 32, 2048), bias=True, act="swiglu_alpha", interleaved_w13=True, seed=4),
    Workload("int4zp_e8_top2_h512_i1024", "int4zp_g128", 8, 0, 8, 2, 512, 1024,
             (1, 2304), seed=5),
    Workload("int4_actorder_bias_e8_top2_h512_i1024", "int4_g128", 8, 0, 8, 2, 512, 1024,
             (1, 2304), bias=True, act_order=True, seed=6),
    Workload("int4zpf_bias_e8_top2_h512_i1024", "int4zpf_g128", 8, 0, 8, 2, 512, 1024,
             (1, 2304), bias=True, seed=7),
    # the Zipf batches' counterpart without skew: the same slice and weights, uniform routing, and
    # M chosen so that the live slots about match those of Zipf M = 1024 and 4096 (5800 against
    # 5760 and 23280 against 23283 at seed 2)
    Workload("nvfp4_ep8_slice_uniform_prefill_h4096_i4096", "nvfp4_g16", 256, 0, 32, 8, 4096, 4096,
             (5760, 23296), norm=True, seed=2),
]}
(INT4_SMALL, INT4_BIAS, NVFP4_DECODE, NVFP4_ZIPF, MXFP4_SWIGLU, INT4ZP, INT4_ACT_ORDER, INT4ZPF,
 NVFP4_UNIFORM) = WORKLOADS
# the layer bench.py measures by default: the largest configuration that fits one GPU (the NVFP4
# EP8 slice with Zipf routing at 4096 tokens: 906 MB of weights, 23283 live slots at seed 2)
HEADLINE, HEADLINE_M = NVFP4_ZIPF, 4096


def _rng(a: int, b: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([a, b, stream])


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (torch's round-to-nearest-even cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


@dataclass
class ExpertWeights:
    """One projection's canonical weights for the local experts."""
    codes: np.ndarray
    scales: np.ndarray
    gs: Optional[np.ndarray]
    bias: Optional[np.ndarray]
    N: int
    K: int
    zeros: Optional[np.ndarray] = None
    g_idx: Optional[np.ndarray] = None   # int32 [E, K]: group of each input column (act-order)


@dataclass
class LayerWeights:
    w13: ExpertWeights
    w2: ExpertWeights
    norm_w: Optional[np.ndarray]


@dataclass
class LayerInputs:
    x: np.ndarray
    topk_ids: np.ndarray
    topk_weights: np.ndarray
    M: int


def _projection(rng: np.random.Generator, wl: Workload, E: int, N: int, K: int) -> ExpertWeights:
    g = wl.group
    codes = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    zeros = None
    if wl.qtype == "int4_g128":
        scales = _to_bf16_bits(rng.uniform(0.002, 0.02, size=(E, N, K // g)).astype(np.float32))
        gs = None
    elif wl.qtype == "int4zp_g128":
        scales = _to_bf16_bits(rng.uniform(0.002, 0.02, size=(E, N, K // g)).astype(np.float32))
        # a min/max quantiser puts a roughly zero-centred group's zero point near the middle of
        # 0..15; the tails still reach both ends
        zeros = np.clip(np.rint(rng.normal(7.5, 2.5, size=(E, N, K // g))), 0, 15).astype(np.uint8)
        gs = None
    elif wl.qtype == "int4zpf_g128":
        scales = _to_bf16_bits(rng.uniform(0.002, 0.02, size=(E, N, K // g)).astype(np.float32))
        # float zero points (the offset a quantiser stores unrounded): not integers, clustered
        # about the middle of 0..15 as for roughly zero-centred groups.  (The spread matters:
        # each group's mean weight is (7.5 - z) s, an offset that grows the layer's outputs, and
        # with a spread of 2.5 the bf16 rounding of the dequantised weights alone -- applied to
        # the oracle's float64 weights on the CPU -- put one output of the full-size layer at 1.01
        # times the layer bar; with 1.0 the worst is at 0.66.)
        zeros = np.clip(rng.normal(7.5, 1.0, size=(E, N, K // g)), 0.0, 15.0).astype(np.float16).view(np.uint16)
        gs = None
    elif wl.qtype == "nvfp4_g16":
        scales = _to_e4m3_codes(np.exp2(rng.uniform(4.0, 8.0, size=(E, N, K // g))).astype(np.float32))
        gs = (4.92e-5 * rng.uniform(0.75, 1.25, size=(E,))).astype(np.float32)
    elif wl.qtype == "mxfp4_g32":
        scales = rng.integers(118, 122, size=(E, N, K // g), dtype=np.uint8)
        gs = None
    else:
        raise ValueError(wl.qtype)
    return ExpertWeights(codes, scales, gs, None, N, K, zeros)


def make_g_idx(rng: np.random.Generator, E: int, K: int, group: int = 128) -> np.ndarray:
    """int32 [E, K]: a random act-order grouping per expert, every group holding `group` columns."""
    rank = np.argsort(rng.random((E, K)), axis=1, kind="stable")      # a random permutation per expert
    g = np.empty((E, K), dtype=np.int32)
    np.put_along_axis(g, rank, (np.arange(K) // group).astype(np.int32)[None, :].repeat(E, 0), axis=1)
    return g


def make_weights(wl: Workload) -> LayerWeights:
    """Canonical weights of the local experts (only these are ever passed on)."""
    E, H, I = wl.n_local, wl.H, wl.I
    if H % wl.group or I % wl.group:
        raise ValueError("H and I must be multiples of the quantisation group")
    rng = _rng(wl.seed, 0, _S_WEIGHTS)
    n13 = I if wl.act == "relu2" else 2 * I   # gate/up rows, or the non-gated projection
    w13 = _projection(rng, wl, E, n13, H)
    w2 = _projection(rng, wl, E, H, I)
    if wl.act_order:
        if wl.group != 128:
            raise ValueError("act-order is defined for the int4 formats")
        # GPTQ desc_act grouping: columns ranked by a random order, 128 consecutive ranks per
        # group (drawn from a stream of its own: the other weights do not change)
        ao = _rng(wl.seed, 1, _S_WEIGHTS)
        w13.g_idx = make_g_idx(ao, E, H)
        w2.g_idx = make_g_idx(ao, E, I)
    aux = _rng(wl.seed, 0, _S_AUX)
    if wl.bias:
        w13.bias = _to_bf16_bits(aux.normal(0.0, 0.1, size=(E, n13)).astype(np.float32))
        w2.bias = _to_bf16_bits(aux.normal(0.0, 0.1, size=(E, H)).astype(np.float32))
    norm_w = None
    if wl.norm:
        norm_w = _to_bf16_bits(aux.normal(0.0, 0.1, size=(H,)).astype(np.float32))
    return LayerWeights(w13, w2, norm_w)


def _distinct_topk(keys: np.ndarray, k: int) -> np.ndarray:
    # k largest keys per row, as distinct column indices
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def make_inputs(wl: Workload, M: int, seed: Optional[int] = None) -> LayerInputs:
    s = wl.seed if seed is None else seed
    hid = _rng(s, M, _S_HIDDEN)
    x = _to_bf16_bits(hid.standard_normal((M, wl.H), dtype=np.float32))
    r = _rng(s, M, _S_ROUTING)
    E = wl.n_global
    if wl.routing == "uniform":
        keys = r.random((M, E))
    elif wl.routing == "zipf":
        # Gumbel-top-k: k distinct draws without replacement with P(e) ~ (e+1)^-s
        logp = -wl.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        keys = logp[None, :] + r.gumbel(size=(M, E))
    else:
        raise ValueError(wl.routing)
    ids = _distinct_topk(keys, wl.top_k)
    logits = r.standard_normal((M, wl.top_k))
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return LayerInputs(x, ids, w, M)


def small_workload(qtype: str, **kw) -> Workload:
    """Reduced shapes that the oracle finishes in well under a second while the
    GPU kernels still see several tiles and ragged tails."""
    base = {
        "int4_g128": Workload("int4_small", "int4_g128", 8, 0, 8, 2, 512, 384, (37,), seed=100),
        "nvfp4_g16": Workload("nvfp4_small", "nvfp4_g16", 64, 8, 16, 8, 512, 320, (29,),
                              norm=True, seed=101),
        "mxfp4_g32": Workload("mxfp4_small", "mxfp4_g32", 16, 0, 16, 4, 448, 320, (41,),
                              bias=True, act="swiglu_alpha", interleaved_w13=True, seed=102),
        "int4zp_g128": Workload("int4zp_small", "int4zp_g128", 12, 2, 8, 2, 512, 384, (37,),
                                bias=True, seed=103),
        "int4zpf_g128": Workload("int4zpf_small", "int4zpf_g128", 10, 1, 8, 2, 512, 384, (37,),
                                 seed=104),
    }[qtype]
    return base.replace(**kw) if kw else base


# ----------------------------------------------------------------------------- device copies
def device_weights(lw: LayerWeights, device="cuda") -> tuple:
    """(w13, w2, post_norm_w) as device tensors in the canonical layouts (bf16 for bf16 bits)."""
    def proj(p: ExpertWeights, bf16_scales: bool) -> dict:
        d = {"codes": torch.from_numpy(p.codes).to(device)}
        s = torch.from_numpy(p.scales.view(np.int16) if bf16_scales else p.scales).to(device)
        d["scales"] = s.view(torch.bfloat16) if bf16_scales else s
        if p.gs is not None:
            d["gs"] = torch.from_numpy(p.gs).to(device)
        if p.bias is not None:
            d["bias"] = torch.from_numpy(p.bias.view(np.int16)).to(device).view(torch.bfloat16)
        if p.zeros is not None:
            z = p.zeros.view(np.int16) if p.zeros.dtype == np.uint16 else p.zeros   # float16 bits
            d["zeros"] = torch.from_numpy(z).to(device)
        if p.g_idx is not None:
            d["g_idx"] = torch.from_numpy(p.g_idx).to(device)
        return d
    int4 = lw.w13.scales.dtype == np.uint16
    nw = None
    if lw.norm_w is not None:
        nw = torch.from_numpy(lw.norm_w.view(np.int16)).to(device).view(torch.bfloat16)
    return proj(lw.w13, int4), proj(lw.w2, int4), nw


def device_inputs(inp: LayerInputs, device="cuda") -> tuple:
    """(x bf16 [M, H], topk_ids int32 [M, k], topk_weights fp32 [M, k]) on the device."""
    x = torch.from_numpy(inp.x.view(np.int16)).to(device).view(torch.bfloat16)
    return x, torch.from_numpy(inp.topk_ids).to(device), torch.from_numpy(inp.topk_weights).to(device)


def bf16_to_float(t: torch.Tensor) -> np.ndarray:
    """A bf16 device tensor as float64 numpy (exact)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


# ----------------------------------------------------------------------------- fp8 requant inputs
# The W4AFP8 activation requant ("sglang PR 35760" summary): after the low-latency dispatch
# expert e holds max_m row slots of K float8 e4m3fn values, the first masked_m[e] live, with
# one float32 scale per row and 128-wide group.  Shapes follow the page: K = 7168 (56 groups of
# 128, the DeepSeek-V3 hidden size its geometry tests use), 256 local experts with one row each
# (the decode case it quotes), and a skew axis in which one hot expert takes `skew` times the
# mean row count while the others share the rest, keeping the total fixed.
REQUANT_GROUP = 128


@dataclass(frozen=True)
class RequantWorkload:
    name: str
    E: int              # local experts
    K: int              # hidden size, a multiple of 128
    rows: int           # mean live rows per expert
    skew: int = 1       # the hot expert (index 0) takes skew * rows
    max_m: int = 0      # row slots per expert (0: just enough for the hot expert)
    seed: int = 0


REQUANT_WORKLOADS = {w.name: w for w in [
    RequantWorkload("requant_e256_k7168_rows1", 256, 7168, 1, max_m=8, seed=1),
    RequantWorkload("requant_e32_k7168_rows32_skew16", 32, 7168, 32, skew=16, seed=2),
    RequantWorkload("requant_e8_k7168_rows256", 8, 7168, 256, seed=3),
]}
REQUANT_HEADLINE = REQUANT_WORKLOADS["requant_e256_k7168_rows1"]


def requant_counts(wl: RequantWorkload) -> np.ndarray:
    """Live rows per expert (int32 [E]): uniform, or expert 0 hot with skew * rows and the
    remainder shared as evenly as integers allow."""
    total = wl.E * wl.rows
    if wl.skew <= 1 or wl.E == 1:
        return np.full(wl.E, wl.rows, dtype=np.int32)
    hot = min(total, wl.skew * wl.rows)
    rest = total - hot
    c = np.full(wl.E - 1, rest // (wl.E - 1), dtype=np.int64)
    c[: rest % (wl.E - 1)] += 1
    return np.concatenate([[hot], c]).astype(np.int32)


def requant_max_m(wl: RequantWorkload) -> int:
    return wl.max_m or int(requant_counts(wl).max())


@dataclass
class RequantInputs:
    x: np.ndarray            # uint8 [E, max_m, K] float8 e4m3fn codes (every slot filled)
    scales: np.ndarray       # float32 [E, max_m, K/128] per row and group (logical order)
    masked_m: np.ndarray     # int32 [E]
    tensor_scale: np.float32


def make_requant_inputs(E: int, max_m: int, K: int, masked_m, seed: int,
                        tensor_scale_factor: float = 1.0) -> RequantInputs:
    """Per-token-group quantised activations: values N(0, 1) times a log-normal row magnitude
    with a few 20x outliers, each (row, group) scaled so that its largest magnitude maps to 448
    and cast to float8 e4m3fn (torch's cast); the per-tensor scale is the largest group scale
    times `tensor_scale_factor` (below 1 some values saturate)."""
    assert K % REQUANT_GROUP == 0
    G = K // REQUANT_GROUP
    rng = _rng(seed, 0x5EC, _S_HIDDEN)
    masked_m = np.asarray(masked_m, dtype=np.int32)
    live = np.arange(max_m)[None, :] < np.clip(masked_m, 0, max_m)[:, None]
    L = int(live.sum())
    # rows that are not live hold arbitrary codes and scales (a kernel must neither use nor write them)
    x = rng.integers(0, 256, size=(E, max_m, K), dtype=np.uint8)
    scales = np.exp2(rng.uniform(-4, 4, size=(E, max_m, G))).astype(np.float32)
    mag = np.exp(rng.normal(0.0, 0.5, size=(L, 1))).astype(np.float32)
    a = rng.standard_normal((L, K), dtype=np.float32) * mag
    a[rng.random((L, K), dtype=np.float32) < 1e-3] *= 20.0
    g = a.reshape(L, G, REQUANT_GROUP)
    amax = np.maximum(np.abs(g).max(axis=-1), np.float32(1e-6))
    s_live = (amax / np.float32(448.0)).astype(np.float32)
    x[live] = _to_e4m3_codes((g / s_live[..., None]).reshape(L, K))
    scales[live] = s_live
    ts = np.float32((s_live.max() if L else np.float32(1.0)) * np.float32(tensor_scale_factor))
    return RequantInputs(x, scales, masked_m, ts)


def requant_inputs_for(wl: RequantWorkload, tensor_scale_factor: float = 1.0) -> RequantInputs:
    return make_requant_inputs(wl.E, requant_max_m(wl), wl.K, requant_counts(wl), wl.seed,
                               tensor_scale_factor)
