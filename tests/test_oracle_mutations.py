"""Planted mistakes in the oracle (CPU only): each plausible error -- a dropped term, a wrong
sign, index or order, a transposed operand -- is patched into the oracle in turn, and at least
one of the oracle's pins must then fail.  This checks the pins, not the GPU path."""
import math

import numpy as np
import pytest

import oracle.formats as F
import oracle.moe as O
import test_oracle_align as TA
import test_oracle_layer as TL


def _swap_gate_up(orig):
    def f(h, interleaved):
        g, u = orig(h, interleaved)
        return u, g
    return f


def _combine_eps_outside(Y, topk_weights, slot_local, norm_w, eps, routed_scaling_factor=1.0):
    M, k = np.shape(topk_weights)
    H = Y.shape[-1]
    Yr = Y.reshape(M, k, H)
    out = np.zeros((M, H))
    for s in range(k):
        live = np.asarray(slot_local)[:, s] >= 0
        y = Yr[live, s]
        if norm_w is None:
            out[live] += np.asarray(topk_weights)[live, s][:, None] * y
        else:
            z = y * norm_w[None, :]
            inv = 1.0 / (np.sqrt(np.sum(z * z, axis=1) / H) + eps)      # eps outside the root
            out[live] += (np.asarray(topk_weights)[live, s] * inv)[:, None] * z
    return out * routed_scaling_factor


def _align_reversed_segments(topk_ids, expert_start, n_local, block_m):
    s, e, n, loc = ORIG["moe_align"](topk_ids, expert_start, n_local, block_m)
    s = s.copy()
    for b in range(n // block_m):        # descending slot order inside each block
        blk = s[b * block_m:(b + 1) * block_m]
        live = blk[blk < loc.size]
        blk[:live.size] = live[::-1]
    return s, e, n, loc



def _expert_forward_variant(skip="", h_before_bias=False):
    """The oracle's expert step with one of its bf16 roundings (of h, a or y) left out, or with
    h rounded before its bias is added."""
    def f(xrows, W13, b13, W2, b2, act, alpha, limit, interleaved, bf16_intermediates=True):
        rnd = O.round_to_bf16 if bf16_intermediates else (lambda v: v)
        h = xrows @ W13.T
        if h_before_bias:
            h = rnd(h)
        if b13 is not None:
            h = h + b13[None, :]
        if skip != "h" and not h_before_bias:
            h = rnd(h)
        if act == "relu2":
            a = O.act_relu2(h)
        else:
            gate, up = O.split_gate_up(h, interleaved)
            a = O.act_silu_mul(gate, up) if act == "silu_mul" else O.act_swiglu_alpha(gate, up, alpha, limit)
        if skip != "a":
            a = rnd(a)
        y = a @ W2.T
        if b2 is not None:
            y = y + b2[None, :]
        if skip != "y":
            y = rnd(y)
        return {"h": h, "a": a, "y": y}
    return f


ORIG = {"moe_align": O.moe_align}

MUTATIONS = {
    "gate/up swapped": ("split_gate_up", lambda: _swap_gate_up(O.split_gate_up)),
    "bias dropped": ("expert_forward", lambda: (lambda x, W13, b13, W2, b2, *a, **k:
                                                ORIG_EF(x, W13, None, W2, b2, *a, **k))),
    "eps outside the square root": ("combine", lambda: _combine_eps_outside),
    "norm weight ignored": ("combine", lambda: (lambda Y, g, loc, nw, eps, routed_scaling_factor=1.0:
                                                ORIG_COMBINE(Y, g, loc, None if nw is None else np.ones_like(nw), eps,
                                                             routed_scaling_factor))),
    "routed scaling ignored": ("combine", lambda: (lambda Y, g, loc, nw, eps, routed_scaling_factor=1.0:
                                                   ORIG_COMBINE(Y, g, loc, nw, eps, 1.0))),
    "nibble order swapped": ("_nibbles", lambda: (lambda c: ORIG_NIB(c).reshape(*np.shape(c)[:-1], -1, 2)[..., ::-1]
                                                  .reshape(ORIG_NIB(c).shape))),
    "int4 offset 7": ("decode_uint4b8", lambda: (lambda q: np.asarray(q, dtype=np.float64) - 7.0)),
    "alpha dropped": ("act_swiglu_alpha", lambda: (lambda g, u, alpha, limit: ORIG_SW(g, u, 1.0, limit))),
    "up clamped from above only": ("act_swiglu_alpha", lambda: (
        lambda g, u, alpha, limit: np.minimum(g, limit) * O._sigmoid(alpha * np.minimum(g, limit))
        * (np.minimum(u, limit) + 1.0))),
    "silu of up instead of gate": ("act_silu_mul", lambda: (lambda g, u: u * O._sigmoid(u) * g)),
    "relu without the square": ("act_relu2", lambda: (lambda h: np.maximum(h, 0.0))),
    "square without the relu": ("act_relu2", lambda: (lambda h: np.square(h))),
    "segments reversed": ("moe_align", lambda: _align_reversed_segments),
    "h not rounded to bf16": ("expert_forward", lambda: _expert_forward_variant(skip="h")),
    "a not rounded to bf16": ("expert_forward", lambda: _expert_forward_variant(skip="a")),
    "y not rounded to bf16": ("expert_forward", lambda: _expert_forward_variant(skip="y")),
    "h rounded before its bias": ("expert_forward", lambda: _expert_forward_variant(h_before_bias=True)),
    "off-slice kept": ("route_local", lambda: (lambda ids, start, n: (np.asarray(ids) % n).astype(np.int32))),
    "global scale missing": ("dequant", lambda: (lambda q, c, s, gs=None, zeros=None, g_idx=None:
                                                 ORIG_DQ(q, c, s, None if gs is None else 1.0, zeros, g_idx))),
    "zero point ignored": ("dequant", lambda: (lambda q, c, s, gs=None, zeros=None, g_idx=None:
                                               ORIG_DQ("int4_g128", c, s, None, None, g_idx) if q == "int4zp_g128"
                                               else ORIG_DQ(q, c, s, gs, zeros, g_idx))),
    "zero point sign flipped": ("dequant", lambda: (lambda q, c, s, gs=None, zeros=None, g_idx=None:
                                             ORIG_DQ(q, c, s, gs, None if zeros is None else (16 - zeros.astype(np.int64)) % 16, g_idx)
                                             if q == "int4zp_g128" else ORIG_DQ(q, c, s, gs, zeros, g_idx))),
    "zero point of the wrong group": ("dequant", lambda: (lambda q, c, s, gs=None, zeros=None, g_idx=None:
                                                          ORIG_DQ(q, c, s, gs, None if zeros is None else zeros[..., ::-1], g_idx)
                                                          if q == "int4zp_g128" else ORIG_DQ(q, c, s, gs, zeros, g_idx))),
    "float zero point read as bf16": ("decode_fp16", lambda: F.decode_bf16),
    "float zero point rounded to an integer": ("decode_fp16", lambda: (lambda b: np.rint(F.decode_fp16(b)))),
    "float zero point ignored": ("decode_fp16", lambda: (lambda b: np.zeros(np.shape(b)))),
    "act-order grouping ignored": ("dequant", lambda: (lambda q, c, s, gs=None, zeros=None, g_idx=None:
                                                       ORIG_DQ(q, c, s, gs, zeros))),
    "act-order group of the sorted position": ("dequant", lambda: (lambda q, c, s, gs=None, zeros=None, g_idx=None:
                                                                   ORIG_DQ(q, c, s, gs, zeros, None if g_idx is None
                                                                           else np.sort(g_idx)))),
}
ORIG_EF, ORIG_COMBINE, ORIG_NIB, ORIG_SW, ORIG_DQ = (O.expert_forward, O.combine, O._nibbles,
                                                      O.act_swiglu_alpha, O.dequant)

PINS = [
    (TL.test_dequant_constant_closed_forms, {}),
    (TL.test_dequant_matches_per_element_brute_force, dict(qtype="nvfp4_g16", N=5, K=48)),
    (TL.test_dequant_matches_per_element_brute_force, dict(qtype="int4zp_g128", N=3, K=384)),
    (TL.test_dequant_asymmetric_int4_closed_forms, {}),
    (TL.test_dequant_matches_per_element_brute_force, dict(qtype="int4zpf_g128", N=3, K=384)),
    (TL.test_dequant_float_zero_point_closed_forms, {}),
    (TL.test_dequant_asymmetric_int4_with_zero_point_8_is_uint4b8, {}),
    (TL.test_dequant_act_order_brute_force_and_identity_grouping, dict(qtype="int4_g128")),
    (TL.test_dequant_act_order_is_the_plain_format_on_sorted_columns, dict(qtype="int4zp_g128")),
    (TL.test_silu_mul_hand_values, {}),
    (TL.test_swiglu_alpha_hand_values, {}),
    (TL.test_relu2_hand_values, {}),
    (TL.test_combine_norm_weight_first_and_eps_placement, {}),
    (TL.test_combine_reduces_to_rmsnorm_and_weighted_sum, {}),
    (TL.test_combine_routed_scaling_factor, {}),
    (TL.test_layer_int4_one_token_one_expert_closed_form, {}),
    (TL.test_layer_nvfp4_norm_closed_form_with_dead_slot, {}),
    (TL.test_layer_mxfp4_swiglu_interleaved_bias_closed_form, dict(limit=math.inf)),
    (TL.test_layer_mxfp4_swiglu_interleaved_bias_closed_form, dict(limit=1.0)),
    (TL.test_layer_int4_relu2_non_gated_bias_closed_form, {}),
    (TL.test_layer_int4_bf16_intermediates_closed_form, {}),
    (TL.test_layer_relu2_bf16_intermediates_closed_form, {}),
    (TA.test_golden_small, {}),
    (TA.test_matches_sort_brute_force, dict(M=64, k=8, E_glob=256, start=32, n_local=32, B=8)),
    (TA.test_route_local_brute_force, {}),
]


def _failing_pins():
    # only a failed assertion counts: a mutation that breaks a call signature must not pass
    failed = []
    for fn, kw in PINS:
        try:
            fn(**kw)
        except AssertionError:
            failed.append(fn.__name__)
    return failed


def test_pins_pass_on_the_unmodified_oracle():
    assert _failing_pins() == []


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, make = MUTATIONS[name]
    monkeypatch.setattr(O, attr, make())
    assert _failing_pins(), f"no pin catches: {name}"
