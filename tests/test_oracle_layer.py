"""Pins of the oracle's dequantisation, activations, combine and whole layer
(CPU only): closed forms computed by hand with ``math``, a per-element brute
force, the page's de-interleave golden and invariants of the definition."""
import json
import math
import os
import struct
from types import SimpleNamespace as NS

import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe as O
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _silu(v):
    return v / (1.0 + math.exp(-v))


def _sig(v):
    return 1.0 / (1.0 + math.exp(-v))


def _bf16(v):
    """bits of a float that is exactly bf16-representable (checked)."""
    b = struct.unpack("<I", struct.pack("<f", v))[0]
    assert b & 0xFFFF == 0, v
    return b >> 16


def _const_proj(n_rows_codes, K, scale_code, dtype_scale, group, gs=None, bias=None):
    """One expert; row r gets nibble n_rows_codes[r] in every K position."""
    codes = np.array([[c | (c << 4)] * (K // 2) for c in n_rows_codes], dtype=np.uint8)[None]
    scales = np.full((1, len(n_rows_codes), K // group), scale_code, dtype=dtype_scale)
    return NS(codes=codes, scales=scales,
              gs=None if gs is None else np.array([gs], dtype=np.float32),
              bias=None if bias is None else np.array([bias], dtype=np.uint16))


# ----------------------------------------------------------------------------- dequant
def _brute_dequant_matvec(qtype, codes, scales, gs, x, zeros=None, g_idx=None):
    """Per-element reading of the packed layout, independent of the oracle's
    vectorised unpack: byte k//2 of row n, low nibble for even k; with act-order the group of
    column k is g_idx[k] instead of k // 128."""
    N, Kh = codes.shape
    K = Kh * 2
    grp = [k // 128 for k in range(K)] if g_idx is None else [int(v) for v in g_idx]
    e4m3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().tolist()
    out = []
    for n in range(N):
        acc = 0.0
        for k in range(K):
            byte = int(codes[n, k // 2])
            u = (byte >> 4) if (k & 1) else (byte & 0xF)
            if qtype == "int4_g128":
                s = struct.unpack("<f", struct.pack("<I", int(scales[n, grp[k]]) << 16))[0]
                w = (u - 8) * s
            elif qtype == "int4zp_g128":
                s = struct.unpack("<f", struct.pack("<I", int(scales[n, grp[k]]) << 16))[0]
                w = (u - int(zeros[n, grp[k]])) * s
            elif qtype == "int4zpf_g128":
                s = struct.unpack("<f", struct.pack("<I", int(scales[n, grp[k]]) << 16))[0]
                z = struct.unpack("<e", struct.pack("<H", int(zeros[n, grp[k]])))[0]   # binary16
                w = (u - z) * s
            else:
                sign = -1.0 if u & 8 else 1.0
                e, m = (u >> 1) & 3, u & 1
                v = sign * (m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))
                if qtype == "nvfp4_g16":
                    w = v * e4m3[int(scales[n, k // 16])] * float(gs)
                else:
                    w = v * 2.0 ** (int(scales[n, k // 32]) - 127)
            acc += w * x[k]
        out.append(acc)
    return np.array(out)


@pytest.mark.parametrize("qtype,N,K", [("int4_g128", 3, 256), ("nvfp4_g16", 5, 48), ("mxfp4_g32", 4, 96),
                                        ("int4zp_g128", 3, 384), ("int4zpf_g128", 3, 384)])
def test_dequant_matches_per_element_brute_force(qtype, N, K):
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    g = W.GROUP[qtype]
    zeros = None
    if qtype in ("int4_g128", "int4zp_g128", "int4zpf_g128"):
        scales = W._to_bf16_bits(rng.uniform(0.002, 0.02, (N, K // g)).astype(np.float32))
        gs = None
        if qtype == "int4zp_g128":
            zeros = rng.integers(0, 16, size=(N, K // g), dtype=np.uint8)
        if qtype == "int4zpf_g128":     # any float16, also outside 0..15 and non-integer
            zeros = rng.uniform(-4.0, 20.0, size=(N, K // g)).astype(np.float16).view(np.uint16)
    elif qtype == "nvfp4_g16":
        scales = rng.integers(0x20, 0x70, size=(N, K // g), dtype=np.uint8)
        gs = np.float32(3.1e-3)
    else:
        scales = rng.integers(118, 130, size=(N, K // g), dtype=np.uint8)
        gs = None
    x = rng.standard_normal(K)
    got = O.dequant(qtype, codes, scales, gs, zeros) @ x
    ref = _brute_dequant_matvec(qtype, codes, scales, gs, x, zeros)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def _pack_nibbles(q):
    """[..., K] nibbles -> [..., K/2] bytes, low nibble = even k."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def _act_order_case(qtype, N, K, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = W._to_bf16_bits(rng.uniform(0.002, 0.02, (N, K // 128)).astype(np.float32))
    zeros = rng.integers(0, 16, size=(N, K // 128), dtype=np.uint8) if qtype == "int4zp_g128" else None
    g_idx = W.make_g_idx(rng, 1, K)[0]
    return codes, scales, zeros, g_idx


@pytest.mark.parametrize("qtype", ["int4_g128", "int4zp_g128"])
def test_dequant_act_order_brute_force_and_identity_grouping(qtype):
    codes, scales, zeros, g_idx = _act_order_case(qtype, 3, 384, 5)
    assert np.array_equal(np.bincount(g_idx), [128, 128, 128])       # 128 columns per group
    x = np.random.default_rng(6).standard_normal(384)
    got = O.dequant(qtype, codes, scales, None, zeros, g_idx) @ x
    assert np.allclose(got, _brute_dequant_matvec(qtype, codes, scales, None, x, zeros, g_idx),
                       rtol=1e-12, atol=1e-12)
    # the grouping of the plain format, written out, is the plain format
    plain = np.arange(384) // 128
    assert np.array_equal(O.dequant(qtype, codes, scales, None, zeros, plain),
                          O.dequant(qtype, codes, scales, None, zeros))


@pytest.mark.parametrize("qtype", ["int4_g128", "int4zp_g128"])
def test_dequant_act_order_is_the_plain_format_on_sorted_columns(qtype):
    # sorting the columns by group turns an act-order weight into a plain one with the same
    # scales (GPTQ desc_act): dequant(codes, g_idx)[:, perm] == dequant(codes[:, perm])
    codes, scales, zeros, g_idx = _act_order_case(qtype, 5, 512, 9)
    perm = np.argsort(g_idx, kind="stable")
    q = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(5, 512)
    sorted_codes = _pack_nibbles(q[:, perm])
    act = O.dequant(qtype, codes, scales, None, zeros, g_idx)
    assert np.array_equal(act[:, perm], O.dequant(qtype, sorted_codes, scales, None, zeros))
    assert not np.array_equal(act, O.dequant(qtype, codes, scales, None, zeros))


def test_layer_act_order_equals_plain_layer_on_permuted_columns():
    # the layer with act-order weights equals the plain layer whose GEMM1 columns (with x) and
    # GEMM2 columns (with GEMM1's intermediate features: gate and up rows, biases) are
    # permuted into group order (float64 throughout)
    wl = W.small_workload("int4_g128").replace(bias=True, act_order=True, n_global=8, n_local=8)
    lw = W.make_weights(wl)
    inp = W.make_inputs(wl, 9)
    kw = dict(expert_start=0, n_local=8, act="silu_mul", bf16_intermediates=False)
    ref = O.moe_layer("int4_g128", inp.x, inp.topk_ids, inp.topk_weights, lw.w13, lw.w2, **kw)
    E, I, H = 8, wl.I, wl.H
    out = np.zeros_like(ref)
    for e in range(E):   # one expert at a time: each has its own column orders
        p1 = np.argsort(lw.w13.g_idx[e], kind="stable")
        p2 = np.argsort(lw.w2.g_idx[e], kind="stable")
        q13 = np.stack([lw.w13.codes[e] & 0xF, lw.w13.codes[e] >> 4], axis=-1).reshape(2 * I, H)[:, p1]
        rows = np.concatenate([p2, I + p2])                      # gate and up rows in p2 order
        c13 = _pack_nibbles(q13[rows])[None]
        q2 = np.stack([lw.w2.codes[e] & 0xF, lw.w2.codes[e] >> 4], axis=-1).reshape(H, I)[:, p2]
        w13 = NS(codes=c13, scales=lw.w13.scales[e][rows][None], gs=None, bias=lw.w13.bias[e][rows][None])
        w2 = NS(codes=_pack_nibbles(q2)[None], scales=lw.w2.scales[e][None], gs=None, bias=lw.w2.bias[e][None])
        ids = np.where(inp.topk_ids == e, 0, -1).astype(np.int32)
        xb = np.ascontiguousarray(inp.x[:, p1])
        out += O.moe_layer("int4_g128", xb, ids, inp.topk_weights, w13, w2,
                           **dict(kw, expert_start=0, n_local=1))
    assert np.allclose(out, ref, rtol=1e-9, atol=1e-9)


def test_dequant_constant_closed_forms():
    # int4: nibble 13 -> 5, scale 2^-7 ; NVFP4: code 0xB -> -1.5, e4m3 0x40 = 2, gs 0.25 ;
    # MXFP4: code 0x7 -> 6, E8M0 130 -> 8
    d = O.dequant("int4_g128", np.full((2, 64), 0xDD, np.uint8), np.full((2, 1), _bf16(2.0 ** -7), np.uint16))
    assert np.all(d == 5 * 2.0 ** -7)
    d = O.dequant("nvfp4_g16", np.full((2, 8), 0xBB, np.uint8), np.full((2, 1), 0x40, np.uint8), 0.25)
    assert np.all(d == -1.5 * 2 * 0.25)
    d = O.dequant("mxfp4_g32", np.full((2, 16), 0x77, np.uint8), np.full((2, 1), 130, np.uint8))
    assert np.all(d == 48.0)
    # nibble order: low nibble is the even K index
    d = O.dequant("mxfp4_g32", np.full((1, 16), 0x72, np.uint8), np.full((1, 1), 127, np.uint8))
    assert d[0, 0] == 1.0 and d[0, 1] == 6.0


def test_dequant_asymmetric_int4_closed_forms():
    # unsigned nibble 13 with zero point 5 -> 8; zero point 13 -> 0; the second group of a row
    # takes its own zero point; nibble 2 (odd k of byte 0x2D) below zero point 5 -> -3
    s = np.full((2, 2), _bf16(2.0 ** -7), np.uint16)
    z = np.array([[5, 13], [13, 5]], np.uint8)
    d = O.dequant("int4zp_g128", np.full((2, 128), 0xDD, np.uint8), s, None, z)
    assert np.all(d[0, :128] == 8 * 2.0 ** -7) and np.all(d[0, 128:] == 0.0)
    assert np.all(d[1, :128] == 0.0) and np.all(d[1, 128:] == 8 * 2.0 ** -7)
    d = O.dequant("int4zp_g128", np.full((1, 64), 0x2D, np.uint8), s[:1, :1], None, np.full((1, 1), 5, np.uint8))
    assert d[0, 0] == 8 * 2.0 ** -7 and d[0, 1] == -3 * 2.0 ** -7


def test_dequant_float_zero_point_closed_forms():
    # float16 zero points: 7.5 (0x4780), 0.1 (0x2E66 = 0.0999755859375, not 0.1) and -2 (0xC000);
    # nibble 13 (0xDD), scale 2^-7
    s = np.full((1, 3), _bf16(2.0 ** -7), np.uint16)
    z = np.array([[0x4780, 0x2E66, 0xC000]], np.uint16)
    d = O.dequant("int4zpf_g128", np.full((1, 192), 0xDD, np.uint8), s, None, z)
    assert np.all(d[0, :128] == 5.5 * 2.0 ** -7)
    assert np.all(d[0, 128:256] == (13 - 0.0999755859375) * 2.0 ** -7)
    assert np.all(d[0, 256:] == 15 * 2.0 ** -7)


def test_dequant_integer_float_zero_points_are_the_integer_format():
    # float16 zero points holding the integers 0..15 give the integer zero-point format exactly
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 256, size=(4, 256), dtype=np.uint8)
    s = W._to_bf16_bits(rng.uniform(0.002, 0.02, (4, 4)).astype(np.float32))
    zi = rng.integers(0, 16, size=(4, 4), dtype=np.uint8)
    zf = zi.astype(np.float16).view(np.uint16)
    assert np.array_equal(O.dequant("int4zpf_g128", codes, s, None, zf), O.dequant("int4zp_g128", codes, s, None, zi))


def test_dequant_asymmetric_int4_with_zero_point_8_is_uint4b8():
    # uint4b8 is the asymmetric format with every zero point at 8
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 256, size=(4, 128), dtype=np.uint8)
    s = W._to_bf16_bits(rng.uniform(0.002, 0.02, (4, 2)).astype(np.float32))
    a = O.dequant("int4zp_g128", codes, s, None, np.full((4, 2), 8, np.uint8))
    b = O.dequant("int4_g128", codes, s)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------------- activations
def test_silu_mul_hand_values():
    g = np.array([1.0, -2.0, 0.0, 3.5])
    u = np.array([2.0, 0.5, 7.0, -1.0])
    want = [_silu(a) * b for a, b in zip(g, u)]
    assert np.allclose(O.act_silu_mul(g, u), want, rtol=1e-15)


def test_swiglu_alpha_hand_values():
    g = np.array([1.75, -0.5, 4.0, 12.0])
    u = np.array([0.375, -1.0, -9.0, 2.0])
    a, lim = 1.702, 7.0
    want = [min(x, lim) * _sig(a * min(x, lim)) * (max(-lim, min(y, lim)) + 1) for x, y in zip(g, u)]
    assert np.allclose(O.act_swiglu_alpha(g, u, a, lim), want, rtol=1e-15)
    # up = -1 zeroes the output, gate = 0 zeroes it; no clamp with an infinite limit
    assert O.act_swiglu_alpha(np.array([3.0]), np.array([-1.0]), a, math.inf)[0] == 0.0
    assert O.act_swiglu_alpha(np.array([0.0]), np.array([5.0]), a, math.inf)[0] == 0.0
    assert O.act_swiglu_alpha(np.array([12.0]), np.array([9.0]), a, math.inf)[0] == pytest.approx(
        12.0 * _sig(a * 12.0) * 10.0, rel=1e-15)


def test_relu2_hand_values():
    h = np.array([-2.0, -0.5, 0.0, 0.5, 3.0, -0.0])
    assert list(O.act_relu2(h)) == [0.0, 0.0, 0.0, 0.25, 9.0, 0.0]
    assert not O.GATED["relu2"] and O.GATED["silu_mul"] and O.GATED["swiglu_alpha"]


def test_split_gate_up_golden():
    g = json.load(open(os.path.join(GOLDEN, "deinterleave_small.json")))
    rows = np.array(g["rows_in"], dtype=object)
    gate, up = O.split_gate_up(rows, interleaved=True)
    assert list(gate) == g["gate_rows"] and list(up) == g["up_rows"]
    gate, up = O.split_gate_up(np.array(g["gate_rows"] + g["up_rows"], dtype=object), interleaved=False)
    assert list(gate) == g["gate_rows"] and list(up) == g["up_rows"]


# ----------------------------------------------------------------------------- combine
def test_combine_norm_weight_first_and_eps_placement():
    # H = 2, one live slot, one dead slot (its row is NaN and must not leak)
    Y = np.array([[3e-4, 4e-4], [np.nan, np.nan]])
    g = np.array([[0.6, 0.4]])
    loc = np.array([[0, -1]])
    nw = np.array([2.0, 0.5])
    out = O.combine(Y, g, loc, nw, 1e-8)
    z = [6e-4, 2e-4]
    inv = 1 / math.sqrt((z[0] ** 2 + z[1] ** 2) / 2 + 1e-8)
    assert np.allclose(out[0], [0.6 * inv * z[0], 0.6 * inv * z[1]], rtol=1e-14)


def test_combine_reduces_to_rmsnorm_and_weighted_sum():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((1, 64))
    out = O.combine(y, np.array([[1.0]]), np.array([[0]]), np.ones(64), 1e-8)
    rms = np.sqrt(np.mean(y ** 2) + 1e-8)
    assert np.allclose(out, y / rms, rtol=1e-14)
    Y = rng.standard_normal((6, 64))
    g = rng.random((2, 3))
    loc = np.array([[0, 1, -1], [2, -1, 0]])
    out = O.combine(Y, g, loc, None, 1e-8)
    assert np.allclose(out[0], g[0, 0] * Y[0] + g[0, 1] * Y[1], rtol=1e-14)
    assert np.allclose(out[1], g[1, 0] * Y[3] + g[1, 2] * Y[5], rtol=1e-14)


def test_combine_routed_scaling_factor():
    Y = np.array([[1.0, -2.0], [0.5, 4.0]])
    g = np.array([[0.25, 0.75]])
    loc = np.array([[0, 3]])
    out = O.combine(Y, g, loc, None, 1e-8, routed_scaling_factor=2.5)
    assert np.allclose(out[0], [2.5 * (0.25 * 1.0 + 0.75 * 0.5), 2.5 * (0.25 * -2.0 + 0.75 * 4.0)], rtol=1e-15)
    nw = np.array([1.0, 1.0])
    a = O.combine(Y, g, loc, nw, 1e-8, routed_scaling_factor=1.0)
    b = O.combine(Y, g, loc, nw, 1e-8, routed_scaling_factor=-3.0)
    assert np.allclose(b, -3.0 * a, rtol=1e-15)


def test_norm_weight_rounds_one_plus_w_to_bf16():
    w = np.array([_bf16(0.0), _bf16(2.0 ** -9), _bf16(-0.25), _bf16(3 * 2.0 ** -9)], dtype=np.uint16)
    nw = O.norm_weight(w)
    # 1 + 2^-9 is below half an ulp (2^-8) of 1 -> 1 ; 1 + 3*2^-9 -> 1 + 2^-7 (nearest)
    assert list(nw) == [1.0, 1.0, 0.75, 1 + 2.0 ** -7]


# ----------------------------------------------------------------------------- whole layer
def test_layer_int4_one_token_one_expert_closed_form():
    H = I = 128
    x0 = 0.5
    w13 = _const_proj([10] * I + [5] * I, H, _bf16(2.0 ** -7), np.uint16, 128)   # gate 2, up -3
    w2 = _const_proj([12] * H, I, _bf16(2.0 ** -6), np.uint16, 128)              # 4
    x = np.full((1, H), _bf16(x0), np.uint16)
    out = O.moe_layer("int4_g128", x, np.array([[0]], np.int32), np.array([[0.75]], np.float32),
                      w13, w2, expert_start=0, n_local=1, bf16_intermediates=False)
    hg, hu = 2 * 2.0 ** -7 * H * x0, -3 * 2.0 ** -7 * H * x0
    y = 4 * 2.0 ** -6 * I * (_silu(hg) * hu)
    assert np.allclose(out, 0.75 * y, rtol=1e-14)


def test_layer_nvfp4_norm_closed_form_with_dead_slot():
    H = I = 32
    x0 = 0.125
    w13 = _const_proj([2] * I + [11] * I, H, 0x40, np.uint8, 16, gs=0.25)        # 1.0 / -1.5, scale 2
    w2 = _const_proj([4] * H, I, 0x40, np.uint8, 16, gs=0.5)                     # 2.0 * 2 * 0.5
    x = np.full((1, H), _bf16(x0), np.uint16)
    ids = np.array([[5, 0]], np.int32)   # expert 5 is outside the single-expert slice
    gw = np.array([[0.3, 0.7]], np.float32)
    nwb = np.full(H, _bf16(0.0), np.uint16)
    out = O.moe_layer("nvfp4_g16", x, ids, gw, w13, w2, expert_start=0, n_local=1,
                      norm_w_bits=nwb, eps=1e-8, bf16_intermediates=False)
    hg, hu = 0.5 * H * x0, -0.75 * H * x0
    y = 2.0 * I * _silu(hg) * hu
    want = float(gw[0, 1]) * y / math.sqrt(y * y + 1e-8)
    assert np.allclose(out, want, rtol=1e-14)


@pytest.mark.parametrize("limit", [math.inf, 1.0])
def test_layer_mxfp4_swiglu_interleaved_bias_closed_form(limit):
    H = I = 32
    x0 = 0.0625
    b13 = [_bf16(0.25), _bf16(-0.125)] * I                 # interleaved gate/up bias
    w13 = _const_proj([3, 1] * I, H, 126, np.uint8, 32, bias=b13)   # gate 1.5, up 0.5, scale 0.5
    w2 = _const_proj([2] * H, I, 125, np.uint8, 32, bias=[_bf16(0.5)] * H)  # 1.0 * 0.25
    x = np.full((1, H), _bf16(x0), np.uint16)
    out = O.moe_layer("mxfp4_g32", x, np.array([[0]], np.int32), np.array([[0.875]], np.float32),
                      w13, w2, expert_start=0, n_local=1, act="swiglu_alpha", alpha=1.702,
                      limit=limit, interleaved_w13=True, bf16_intermediates=False)
    hg = 1.5 * 0.5 * H * x0 + 0.25
    hu = 0.5 * 0.5 * H * x0 - 0.125
    g, u = min(hg, limit), max(-limit, min(hu, limit))
    a = g * _sig(1.702 * g) * (u + 1)
    y = 0.25 * I * a + 0.5
    assert np.allclose(out, 0.875 * y, rtol=1e-14)


def test_layer_int4_relu2_non_gated_bias_closed_form():
    # non-gated GEMM1 (I rows), relu(h)^2 with a negative row that relu zeroes, routed scaling
    H, I = 128, 128
    x0 = 0.25
    b13 = [_bf16(0.25)] * I
    w13 = _const_proj([11] * (I // 2) + [6] * (I // 2), H, _bf16(2.0 ** -7), np.uint16, 128, bias=b13)  # 3, -2
    w2 = _const_proj([9] * H, I, _bf16(2.0 ** -5), np.uint16, 128, bias=[_bf16(-0.25)] * H)            # 1
    x = np.full((1, H), _bf16(x0), np.uint16)
    out = O.moe_layer("int4_g128", x, np.array([[0]], np.int32), np.array([[0.625]], np.float32),
                      w13, w2, expert_start=0, n_local=1, act="relu2", routed_scaling_factor=1.5,
                      bf16_intermediates=False)
    hp = 3 * 2.0 ** -7 * H * x0 + 0.25           # = 1.0, relu keeps it
    hn = -2 * 2.0 ** -7 * H * x0 + 0.25          # = -0.25, relu zeroes it
    y = 2.0 ** -5 * ((I // 2) * hp ** 2 + (I // 2) * max(hn, 0.0) ** 2) - 0.25
    assert np.allclose(out, 1.5 * 0.625 * y, rtol=1e-14)


def _rne_bf16(v):
    """Nearest value with 8 significant bits (bf16), ties to the even one -- written from the
    format's definition with frexp (Python's round() breaks ties to even), independently of
    the oracle's rounding routine.  Normal magnitudes only."""
    if v == 0.0:
        return 0.0
    m, e = math.frexp(v)            # v = m * 2^e, 0.5 <= |m| < 1
    return math.ldexp(round(m * 256), e - 8)


def test_layer_int4_bf16_intermediates_closed_form():
    # The tensors stored between the experiment's kernels (cache1 = h, cache2 = a, cache13 = y)
    # are bf16; with bf16_intermediates=True the oracle rounds there.  One token, one expert,
    # H = I = 128 (one int4 group), constant codes, chosen so that each of the three roundings
    # moves the output:
    #   gate row code 12 -> 4, up row code 5 -> -3, scale 2^-7, x = 0.5:
    #   h_gate = 4 * 2^-7 * 128 * 0.5 + 7 * 2^-9 = 2.013671875 = 128.875 ulps of 2^-6 -> 2.015625
    #   h_up   = -1.5 - 6 * 2^-9 = -1.51171875 = -193.5 ulps of 2^-7, a tie -> even -194 -> -1.515625
    #   a = silu(2.015625) * -1.515625 = -2.69575681 = -172.53 ulps of 2^-6 -> -2.703125
    #   down row code 11 -> 3, scale 2^-6: y = 3 * 2^-6 * 128 * a + 2^-5 = 6a + 2^-5
    #     = -16.1875 = -129.5 ulps of 2^-3, a tie -> even -130 -> -16.25
    #   out = 0.75 * y = -12.1875
    H = I = 128
    w13 = _const_proj([12] * I + [5] * I, H, _bf16(2.0 ** -7), np.uint16, 128,
                      bias=[_bf16(7 * 2.0 ** -9)] * I + [_bf16(-6 * 2.0 ** -9)] * I)
    w2 = _const_proj([11] * H, I, _bf16(2.0 ** -6), np.uint16, 128, bias=[_bf16(2.0 ** -5)] * H)
    x = np.full((1, H), _bf16(0.5), np.uint16)
    out = O.moe_layer("int4_g128", x, np.array([[0]], np.int32), np.array([[0.75]], np.float32),
                      w13, w2, expert_start=0, n_local=1, bf16_intermediates=True)
    assert np.all(out == -12.1875)
    # the same chain evaluated with math and the frexp rounding gives that value, and leaving out
    # any one rounding (or rounding h before its bias) gives another one
    hg, hu = 4 * 2.0 ** -7 * H * 0.5 + 7 * 2.0 ** -9, -3 * 2.0 ** -7 * H * 0.5 - 6 * 2.0 ** -9

    def chain(rh=True, ra=True, ry=True, h_before_bias=False):
        g = _rne_bf16(hg) if rh else hg
        u = _rne_bf16(hu) if rh else hu
        if h_before_bias:
            g, u = _rne_bf16(hg - 7 * 2.0 ** -9) + 7 * 2.0 ** -9, _rne_bf16(hu + 6 * 2.0 ** -9) - 6 * 2.0 ** -9
        a = _silu(g) * u
        a = _rne_bf16(a) if ra else a
        y = 6 * a + 2.0 ** -5
        return 0.75 * (_rne_bf16(y) if ry else y)
    assert chain() == -12.1875
    for alt in (chain(rh=False), chain(ra=False), chain(ry=False), chain(h_before_bias=True)):
        assert abs(alt - chain()) > 0.04


def test_layer_relu2_bf16_intermediates_closed_form():
    # non-gated relu2 with stored bf16 intermediates: a = bf16(relu(bf16(h))^2), y = bf16(W2 a + b2)
    #   code 12 -> 4, scale 2^-7, x = 0.25: h = 4 * 2^-7 * 128 * 0.25 + 5 * 2^-9 = 1.009765625
    #     = 129.25 ulps of 2^-7 -> 1.0078125
    #   a = 1.0078125^2 = 1.01568603515625 = 130.008 ulps of 2^-7 -> 1.015625
    #   down code 9 -> 1, scale 2^-5: y = 4a - 6 * 2^-7 = 4.015625 = 128.5 ulps of 2^-5, a tie
    #     -> even 128 -> 4.0
    #   out = 1.5 (routed scaling) * 0.625 * y = 3.75
    H = I = 128
    w13 = _const_proj([12] * I, H, _bf16(2.0 ** -7), np.uint16, 128, bias=[_bf16(5 * 2.0 ** -9)] * I)
    w2 = _const_proj([9] * H, I, _bf16(2.0 ** -5), np.uint16, 128, bias=[_bf16(-6 * 2.0 ** -7)] * H)
    x = np.full((1, H), _bf16(0.25), np.uint16)
    out = O.moe_layer("int4_g128", x, np.array([[0]], np.int32), np.array([[0.625]], np.float32),
                      w13, w2, expert_start=0, n_local=1, act="relu2", routed_scaling_factor=1.5,
                      bf16_intermediates=True)
    assert np.all(out == 3.75)
    h = 4 * 2.0 ** -7 * H * 0.25 + 5 * 2.0 ** -9

    def chain(rh=True, ra=True, ry=True):
        v = _rne_bf16(h) if rh else h
        a = _rne_bf16(v * v) if ra else v * v
        y = 4 * a - 6 * 2.0 ** -7
        return 1.5 * 0.625 * (_rne_bf16(y) if ry else y)
    assert chain() == 3.75
    for alt in (chain(rh=False), chain(ra=False), chain(ry=False)):
        assert abs(alt - chain()) > 0.01


def _small(qtype, M=None, **kw):
    wl = W.small_workload(qtype, **kw)
    lw = W.make_weights(wl)
    inp = W.make_inputs(wl, M or wl.Ms[0])
    return wl, lw, inp


def _run(wl, lw, inp, ids=None, gw=None, **kw):
    args = dict(expert_start=wl.expert_start, n_local=wl.n_local, act=wl.act, alpha=wl.alpha,
                limit=wl.limit, norm_w_bits=lw.norm_w, eps=wl.eps,
                interleaved_w13=wl.interleaved_w13)
    args.update(kw)
    return O.moe_layer(wl.qtype, inp.x, inp.topk_ids if ids is None else ids,
                       inp.topk_weights if gw is None else gw, lw.w13, lw.w2, **args)


@pytest.mark.parametrize("qtype", W.QTYPES)
def test_layer_linear_in_topk_weights(qtype):
    wl, lw, inp = _small(qtype)
    rng = np.random.default_rng(11)
    g1 = rng.random(inp.topk_weights.shape)
    g2 = rng.random(inp.topk_weights.shape)
    o1 = _run(wl, lw, inp, gw=g1, bf16_intermediates=False)
    o2 = _run(wl, lw, inp, gw=g2, bf16_intermediates=False)
    o12 = _run(wl, lw, inp, gw=g1 + g2, bf16_intermediates=False)
    assert np.allclose(o12, o1 + o2, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("qtype", W.QTYPES)
def test_layer_token_permutation_invariance(qtype):
    wl, lw, inp = _small(qtype)
    perm = np.random.default_rng(12).permutation(inp.M)
    base = _run(wl, lw, inp)
    pin = W.LayerInputs(inp.x[perm], inp.topk_ids[perm], inp.topk_weights[perm], inp.M)
    other = _run(wl, lw, pin)
    assert np.allclose(other, base[perm], rtol=1e-12, atol=1e-12)


def test_layer_zero_for_off_slice_tokens():
    wl, lw, inp = _small("nvfp4_g16")
    ids = inp.topk_ids.copy()
    ids[::3] = (ids[::3] % 8) + 40         # all of every third token's slots outside [8, 24)
    out = _run(wl, lw, inp, ids=ids)
    assert np.all(out[::3] == 0.0)
    assert np.any(out[1::3] != 0.0)


def test_layer_token_subset_matches_full():
    wl, lw, inp = _small("mxfp4_g32")
    full = _run(wl, lw, inp)
    sub = [5, 0, 17, 40]
    part = _run(wl, lw, inp, tokens=sub)
    assert np.array_equal(part, full[sub])


def test_layer_zero_padding_of_intermediate_is_neutral():
    wl, lw, inp = _small("int4_g128", I=256)
    base = _run(wl, lw, inp)
    I, P = 256, 128
    E = wl.n_local
    zero = 0x88                            # int4 nibble 8 is the value 0

    def pad_rows(a, fill, axis):
        shape = list(a.shape)
        shape[axis] = P
        return np.full(shape, fill, a.dtype)
    w13 = lw.w13
    c = np.concatenate([w13.codes[:, :I], pad_rows(w13.codes, zero, 1)[:, :P],
                        w13.codes[:, I:], pad_rows(w13.codes, zero, 1)[:, :P]], axis=1)
    s = np.concatenate([w13.scales[:, :I], pad_rows(w13.scales, _bf16(1.0), 1),
                        w13.scales[:, I:], pad_rows(w13.scales, _bf16(1.0), 1)], axis=1)
    w2 = lw.w2
    c2 = np.concatenate([w2.codes, np.full((E, w2.codes.shape[1], P // 2), zero, np.uint8)], axis=2)
    s2 = np.concatenate([w2.scales, np.full((E, w2.scales.shape[1], P // 128), _bf16(1.0), np.uint16)], axis=2)
    lp = W.LayerWeights(NS(codes=c, scales=s, gs=None, bias=None), NS(codes=c2, scales=s2, gs=None, bias=None), None)
    padded = _run(wl, lp, inp)
    assert np.allclose(padded, base, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("qtype", W.QTYPES)
def test_bf16_intermediates_stay_within_layer_tolerance(qtype):
    wl, lw, inp = _small(qtype)
    a = _run(wl, lw, inp, bf16_intermediates=True)
    b = _run(wl, lw, inp, bf16_intermediates=False)
    assert np.all(np.abs(a - b) <= 0.06 + 0.04 * np.abs(b))
    assert np.abs(a - b).max() < 0.05 * np.abs(b).max()


def test_intermediates_route_to_slot_rows():
    wl, lw, inp = _small("int4_g128")
    out, inter = _run(wl, lw, inp, return_intermediates=True)
    loc = O.route_local(inp.topk_ids, wl.expert_start, wl.n_local).reshape(-1)
    assert sorted(inter["y"].keys()) == [i for i in range(loc.size) if loc[i] >= 0]
    assert all(v.shape == (wl.H,) for v in inter["y"].values())
