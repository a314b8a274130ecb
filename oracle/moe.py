"""The oracle's MoE expert layer: route -> align -> GEMM1 -> act -> GEMM2 -> combine.

Test infrastructure only (see the package docstring).  Everything is float64
except the three tensors the pages store as bf16 between kernels (the gate/up
projection output ``cache1``, the activation output ``cache2`` and the down
projection output ``cache3`` of the Muse Spark experiment's ``kernel_fn``);
with ``bf16_intermediates=True`` those are rounded to bf16 (nearest, ties to
even), with ``False`` the whole layer stays float64.

Readings of points the pages leave open (each is listed with its reason in the
design notes of the repository):

* assignments to experts outside the local range are dropped by the align
  (the experiment maps them to -1 through ``expert_map``);
* inside one expert's segment the slots are in ascending flat order
  ``t * top_k + s``; segments are padded with the sentinel ``numel = M * top_k``;
  empty experts get no block; the unused tail holds the sentinel / -1;
* GEMM1 reads activation row ``slot // top_k``; both GEMMs write row ``slot``;
* the post-expert RMSNorm is weight-first: ``z = y * bf16(1 + w)``, then
  ``z * (mean(z^2) + eps)^-1/2`` -- the order of ``_expert_norm_factors``;
* biases are added to the matmul output before the activation / before the
  top-k weighting, as in the sglang PR 31552 reference loop;
* ``relu2`` is the non-gated activation of that loop: GEMM1 has I rows (no
  gate/up halves) and ``a = relu(h)^2``;
* ``routed_scaling_factor`` (passed as 1.0 in that test, not defined on the
  pages) multiplies the combined output of each token;
* asymmetric int4 (the ``w1_zeros`` / ``w2_zeros`` arguments of the Marlin MoE call
  in sglang PR 31552): unsigned codes, one zero point and one bf16 scale per group
  of 128 along K, the weight ``(u - z) * s``.  With integer zero points
  (``int4zp_g128``) z is 0..15, stored one per byte in ``[N, K/128]`` like the
  scales; with float zero points (``int4zpf_g128``, the Marlin template's
  ``is_zp_float`` flag, whose comment names float16) z is a float16 value, stored
  as its bit pattern in the same ``[N, K/128]`` layout;
* act-order int4 (the ``g_idx1`` / ``g_idx2`` arguments of that call; the pages pass the
  setup's result through without defining it): ``g_idx[k]`` names the group of 128 whose
  scale (and zero point) input column ``k`` uses; every group holds 128 columns, in any
  order (the GPTQ ``desc_act`` grouping).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .formats import (decode_bf16, decode_e2m1, decode_e4m3fn, decode_e8m0, decode_fp16, decode_uint4,
                      decode_uint4b8, round_to_bf16)

_GROUP = {"int4_g128": 128, "nvfp4_g16": 16, "mxfp4_g32": 32, "int4zp_g128": 128, "int4zpf_g128": 128}
INT4_FORMATS = ("int4_g128", "int4zp_g128", "int4zpf_g128")


# ----------------------------------------------------------------------------- routing
def route_local(topk_ids: np.ndarray, expert_start: int, n_local: int) -> np.ndarray:
    """Global expert id -> local id, -1 when outside [start, start + n_local).

    The experiment's ``prepare`` builds ``expert_map`` (-1 everywhere, ``arange``
    on the local range) and ``kernel_fn`` gathers ``expert_map[topk_ids]``.
    Pinned by a brute-force per-element test and by the zero-output property.
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    loc = ids - expert_start
    ok = (ids >= expert_start) & (ids < expert_start + n_local)
    return np.where(ok, loc, -1).astype(np.int32)


def align_capacity(numel: int, n_local: int, block_m: int) -> tuple:
    """Buffer sizes of the align outputs: (len(sorted_token_ids), len(expert_ids)).

    At most min(n_local, numel) experts are non-empty and each wastes at most
    block_m - 1 padding entries, so the padded total never exceeds
    numel + min(n_local, numel) * (block_m - 1); rounded up to whole blocks.
    """
    worst = numel + min(n_local, numel) * (block_m - 1)
    blocks = -(-worst // block_m)
    return blocks * block_m, blocks


def moe_align(topk_ids: np.ndarray, expert_start: int, n_local: int, block_m: int):
    """Stable counting sort of the (token, slot) assignments by local expert.

    What ``moe_align_block_size(local_ids, block_size_m, ...)`` returns in the
    experiment's ``kernel_fn``: ``sorted_ids``, one expert id per block of
    ``block_m`` entries, and the padded total.  Returns
    ``(sorted_token_ids, expert_ids, num_tokens_post_padded, slot_local_ids)``.
    Pinned against ``numpy.argsort(kind="stable")``, a hand-worked golden and
    invariants (tests/test_oracle_align.py).
    """
    local = route_local(topk_ids, expert_start, n_local).reshape(-1)
    numel = local.size
    cap, cap_blocks = align_capacity(numel, n_local, block_m)
    sorted_ids = np.full(cap, numel, dtype=np.int32)
    expert_ids = np.full(cap_blocks, -1, dtype=np.int32)
    pos = 0
    for e in range(n_local):
        slots = np.nonzero(local == e)[0]                   # ascending flat order
        if slots.size == 0:
            continue
        padded = -(-len(slots) // block_m) * block_m
        sorted_ids[pos:pos + len(slots)] = slots
        expert_ids[pos // block_m:(pos + padded) // block_m] = e
        pos += padded
    return sorted_ids, expert_ids, pos, local.reshape(np.shape(topk_ids))


# ----------------------------------------------------------------------------- weights
def _nibbles(codes: np.ndarray) -> np.ndarray:
    """[N, K/2] bytes -> [N, K] nibbles, the low nibble holding the even K index."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = c & 0x0F
    out[..., 1::2] = c >> 4
    return out


def dequant(qtype: str, codes: np.ndarray, scales: np.ndarray, gs: Optional[float] = None,
            zeros: Optional[np.ndarray] = None, g_idx: Optional[np.ndarray] = None) -> np.ndarray:
    """Dense float64 [N, K] weight of one expert.

    * int4_g128: ``(u - 8) * s[n, G(k)]`` with bf16 ``s`` (uint4b8, group 128).
    * int4zp_g128: ``(u - z[n, G(k)]) * s[n, G(k)]``, unsigned ``u``, integer
      zero point ``z`` in 0..15, bf16 ``s`` (asymmetric int4, group 128).
    * int4zpf_g128: the same with ``z`` a float16 value (its bit pattern given).
    * nvfp4_g16: ``e2m1 * e4m3[n, k // 16] * gs`` (one fp32 global scale per
      expert and projection, as the experiment's ``_marlin_layer`` passes it).
    * mxfp4_g32: ``e2m1 * 2^(E[n, k // 32] - 127)``.
    ``G(k) = k // 128``, or with act-order ``G(k) = g_idx[k]`` (the ``g_idx`` of the Marlin MoE
    call in sglang PR 31552: the quantisation group of input column ``k``, each group holding
    128 columns in any order; int4 formats only).
    Pinned by constant-code closed forms, a tiny brute-force matmul and, for act-order, the
    plain path on the column-sorted weights.
    """
    q = _nibbles(codes)
    g = _GROUP[qtype]
    if g_idx is not None and qtype not in INT4_FORMATS:
        raise ValueError("act-order (g_idx) is defined for the int4 formats only")
    K = q.shape[-1]
    grp = (np.arange(K) // g) if g_idx is None else np.asarray(g_idx, dtype=np.int64)
    if qtype == "int4_g128":
        s = decode_bf16(scales)
        return decode_uint4b8(q) * s[..., grp]
    if qtype in ("int4zp_g128", "int4zpf_g128"):
        if zeros is None:
            raise ValueError("asymmetric int4 needs the zero points")
        z = np.asarray(zeros, dtype=np.float64) if qtype == "int4zp_g128" else decode_fp16(zeros)
        return (decode_uint4(q) - z[..., grp]) * decode_bf16(scales)[..., grp]
    if qtype == "nvfp4_g16":
        if gs is None:
            raise ValueError("NVFP4 needs the per-expert global scale")
        return decode_e2m1(q) * np.repeat(decode_e4m3fn(scales), g, axis=-1) * float(gs)
    if qtype == "mxfp4_g32":
        return decode_e2m1(q) * np.repeat(decode_e8m0(scales), g, axis=-1)
    raise ValueError(qtype)


def split_gate_up(h: np.ndarray, interleaved: bool) -> tuple:
    """Gate and up halves of the GEMM1 output.

    Contiguous halves (gate ``[0, I)``, up ``[I, 2I)``) as the experiment's
    ``Weights`` comment states; GPT-OSS rows arrive interleaved
    ``[gate0, up0, gate1, up1, ...]`` (sglang PR 28231,
    ``deinterleave_moe_mxfp4_w13_for_marlin``), i.e. gate j is row 2j and up j
    is row 2j + 1.  Pinned by the page's de-interleave golden.
    """
    if interleaved:
        return h[..., 0::2], h[..., 1::2]
    i = h.shape[-1] // 2
    return h[..., :i], h[..., i:]


# ----------------------------------------------------------------------------- activations
def _sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def act_silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """``silu(gate) * up`` -- ``silu_and_mul`` of the experiment.  Pinned by
    hand-computed values (math.exp)."""
    return gate * _sigmoid(gate) * up


def act_swiglu_alpha(gate: np.ndarray, up: np.ndarray, alpha: float, limit: float) -> np.ndarray:
    """GPT-OSS activation of sglang PR 28231
    (``swiglu_gpt_oss_sigmoid_alpha_contiguous``): gate clamped from above by
    ``limit``, up clamped to ``[-limit, limit]``, then
    ``gate * sigmoid(alpha * gate) * (up + 1)``.  Pinned by hand values."""
    g = np.minimum(gate, limit)
    u = np.clip(up, -limit, limit)
    return g * _sigmoid(alpha * g) * (u + 1.0)


def act_relu2(h: np.ndarray) -> np.ndarray:
    """Non-gated ``relu(h)^2`` of the sglang PR 31552 reference loop
    (``torch.square(torch.relu(intermediate))``, ``activation="relu2"``,
    ``is_gated=False``).  Pinned by hand values."""
    return np.square(np.maximum(h, 0.0))


GATED = {"silu_mul": True, "swiglu_alpha": True, "relu2": False}


# ----------------------------------------------------------------------------- experts
def expert_forward(xrows: np.ndarray, W13: np.ndarray, b13: Optional[np.ndarray],
                   W2: np.ndarray, b2: Optional[np.ndarray], act: str, alpha: float,
                   limit: float, interleaved: bool, bf16_intermediates: bool = True) -> dict:
    """One expert on the rows routed to it, as in the sglang PR 31552 reference
    loop: ``x @ W1.T (+ b1)`` -> activation -> ``@ W2.T (+ b2)``.  Returns the
    three intermediates (``h`` in the input row order of W13)."""
    rnd = round_to_bf16 if bf16_intermediates else (lambda v: v)
    h = xrows @ W13.T
    if b13 is not None:
        h = h + b13[None, :]
    h = rnd(h)
    if act == "relu2":
        a = act_relu2(h)
    else:
        gate, up = split_gate_up(h, interleaved)
        if act == "silu_mul":
            a = act_silu_mul(gate, up)
        elif act == "swiglu_alpha":
            a = act_swiglu_alpha(gate, up, alpha, limit)
        else:
            raise ValueError(act)
    a = rnd(a)
    y = a @ W2.T
    if b2 is not None:
        y = y + b2[None, :]
    y = rnd(y)
    return {"h": h, "a": a, "y": y}


# ----------------------------------------------------------------------------- combine
def norm_weight(post_norm_w_bits: np.ndarray) -> np.ndarray:
    """The effective norm weight bf16(1 + w) that the experiment's ``prepare``
    binds once (``(w.float() + 1).to(bfloat16)``)."""
    return round_to_bf16(decode_bf16(post_norm_w_bits) + 1.0)


def combine(Y: np.ndarray, topk_weights: np.ndarray, slot_local: np.ndarray,
            norm_w: Optional[np.ndarray], eps: float, routed_scaling_factor: float = 1.0) -> np.ndarray:
    """Top-k weighted sum over the live slots of each token.

    Without a norm: ``out[t] = sum_s g[t, s] * y[t, s]`` (the reference loop's
    ``index_add_`` of ``routed * topk_weights``).  With the post-expert norm
    (``_expert_norm_factors`` then ``_expert_norm_sum``):
    ``z = y * norm_w``, ``factor = g * (sum(z^2) / H + eps)^-1/2`` and
    ``out[t] = sum_s factor * z``.  Dead slots (local id -1) contribute
    nothing.  ``routed_scaling_factor`` multiplies the sum.  Pinned by the
    RMSNorm special case and hand values.
    """
    M, k = np.shape(topk_weights)
    H = Y.shape[-1]
    Yr = Y.reshape(M, k, H)
    g = np.asarray(topk_weights, dtype=np.float64)
    out = np.zeros((M, H), dtype=np.float64)
    for s in range(k):                               # one top-k slot at a time
        live = np.asarray(slot_local)[:, s] >= 0
        y = Yr[live, s]
        if norm_w is None:
            out[live] += g[live, s][:, None] * y
        else:
            z = y * norm_w[None, :]
            inv = 1.0 / np.sqrt(np.sum(z * z, axis=1) / H + eps)
            out[live] += (g[live, s] * inv)[:, None] * z
    return out * routed_scaling_factor


# ----------------------------------------------------------------------------- layer
def _gidx_of(w, e):
    g = getattr(w, "g_idx", None)
    return None if g is None else g[e]


def _zeros_of(w, e):
    z = getattr(w, "zeros", None)
    return None if z is None else z[e]


def moe_layer(qtype: str, x_bits: np.ndarray, topk_ids: np.ndarray, topk_weights: np.ndarray,
              w13, w2, *, expert_start: int, n_local: int, act: str = "silu_mul",
              alpha: float = 1.702, limit: float = math.inf, norm_w_bits=None,
              eps: float = 1e-8, interleaved_w13: bool = False, routed_scaling_factor: float = 1.0,
              bf16_intermediates: bool = True, tokens=None, return_intermediates: bool = False):
    """The whole expert layer for one GPU's expert slice.

    ``w13`` / ``w2`` carry ``codes``, ``scales``, ``gs`` (or None), ``bias``
    (or None), for asymmetric int4 ``zeros`` and, for act-order int4, ``g_idx`` (int
    ``[E, K]``) for the ``n_local`` local experts in the canonical layouts.
    ``tokens`` restricts the evaluation to a subset of tokens (each token's
    output depends only on its own slots), returning rows in that order.
    """
    topk_ids = np.asarray(topk_ids)
    M, k = topk_ids.shape
    tok = np.arange(M) if tokens is None else np.asarray(tokens, dtype=np.int64)
    x = decode_bf16(x_bits)
    slot_local = route_local(topk_ids, expert_start, n_local)
    sub_local = slot_local[tok]                     # [T, k]
    H = x.shape[1]
    Y = np.full((len(tok) * k, H), np.nan)
    inter = {"h": {}, "a": {}, "y": {}}
    flat = sub_local.reshape(-1)
    for e in range(n_local):
        rows = np.nonzero(flat == e)[0]             # ascending (token, slot) order
        if rows.size == 0:
            continue
        W13 = dequant(qtype, w13.codes[e], w13.scales[e], None if w13.gs is None else w13.gs[e],
                      _zeros_of(w13, e), _gidx_of(w13, e))
        W2 = dequant(qtype, w2.codes[e], w2.scales[e], None if w2.gs is None else w2.gs[e], _zeros_of(w2, e),
                     _gidx_of(w2, e))
        b13 = None if w13.bias is None else decode_bf16(w13.bias[e])
        b2 = None if w2.bias is None else decode_bf16(w2.bias[e])
        r = expert_forward(x[tok[rows // k]], W13, b13, W2, b2, act, alpha, limit,
                           interleaved_w13, bf16_intermediates)
        Y[rows] = r["y"]
        if return_intermediates:
            for name in ("h", "a", "y"):
                for j, row in enumerate(rows):
                    inter[name][int(tok[row // k] * k + row % k)] = r[name][j]
    nw = None if norm_w_bits is None else norm_weight(norm_w_bits)
    out = combine(Y, np.asarray(topk_weights)[tok], sub_local, nw, eps, routed_scaling_factor)
    if return_intermediates:
        return out, inter
    return out
