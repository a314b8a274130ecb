"""Pins of the requant oracle (CPU only): its float8 encoder against torch's float32 ->
float8_e4m3fn cast and hand-computed cases, the requant against closed forms, an element-wise
torch computation and its masked-row contract; then planted mistakes in the oracle that one
of those pins must catch."""
import numpy as np
import pytest
import torch

import oracle.requant as R
from oracle.formats import decode_e4m3fn


def _torch_encode(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _finite_codes():
    c = np.arange(256)
    return c[(c & 0x7F) != 0x7F]


def test_encode_matches_torch_cast_on_representables_midpoints_and_random():
    pos = decode_e4m3fn(np.arange(0x7F))
    mids = (pos[1:] + pos[:-1]) / 2                           # every tie (exact in float32)
    rng = np.random.default_rng(11)
    rnd = np.exp2(rng.uniform(-12, np.log2(448.0), 20000)) * rng.choice([-1.0, 1.0], 20000)
    v = np.concatenate([pos, -pos, mids, -mids, rnd, [0.0, -0.0]]).astype(np.float32)
    assert np.abs(v).max() <= 448.0
    got = R.encode_e4m3fn_sat(v)
    assert np.array_equal(got, _torch_encode(v))
    assert got[len(pos) * 2 + 3] == 0x04 and got[len(pos) * 2 + 4] == 0x04   # ties to even


def test_encode_saturation_nan_and_zero_by_hand():
    v = np.array([448.0, 449.0, 464.0, 1e30, np.inf, -np.inf, -500.0, np.nan, -np.nan,
                  0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -11, 2.0 ** -9, 1.0, -1.5, 2.0 ** -12])
    want = [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x7F,
            0x00, 0x80, 0x00, 0x80, 0x01, 0x01, 0x38, 0xBC, 0x00]
    assert R.encode_e4m3fn_sat(v).tolist() == want


def _codes_batch(E, max_m, K, seed):
    rng = np.random.default_rng(seed)
    return rng.choice(_finite_codes(), size=(E, max_m, K)).astype(np.uint8)


@pytest.mark.parametrize("s", [1.0, 3.7, 0.0123])
def test_scales_that_cancel_return_every_code(s):
    # each row holds all 256 codes once; s = tensor_scale, so v = x up to float32 rounding
    x = np.stack([np.stack([np.roll(np.arange(256), 17 * (e + m)) for m in range(3)])
                  for e in range(2)]).astype(np.uint8)
    scales = np.full((2, 3, 2), s, dtype=np.float32)
    out, live = R.requant(x, scales, [3, 2], np.float32(s))
    assert live.tolist() == [[True] * 3, [True, True, False]]
    want = np.where((x & 0x7F) == 0x7F, 0x7F, x)
    assert np.array_equal(out[live], want[live])
    assert not out[~live].any()


def test_power_of_two_scales_shift_the_exponent_field():
    # normal codes with exponent field 5..10; scale 2^a (a distinct per expert, row and group),
    # tensor scale 2^b: the code keeps sign and mantissa and its exponent field moves by a - b
    rng = np.random.default_rng(5)
    E, max_m, G, gs = 3, 4, 5, 128
    exp = rng.integers(5, 11, size=(E, max_m, G * gs))
    man = rng.integers(0, 8, size=exp.shape)
    sgn = rng.integers(0, 2, size=exp.shape)
    x = (sgn << 7 | exp << 3 | man).astype(np.uint8)
    a = (np.arange(E)[:, None, None] + 2 * np.arange(max_m)[None, :, None]
         + 3 * np.arange(G)[None, None, :]) % 9 - 4 + 1          # in -3 .. 5, varies with e, m, g
    b = 1
    scales = np.exp2(a).astype(np.float32)
    out, live = R.requant(x, scales, [4, 4, 4], np.float32(2.0 ** b))
    shift = np.repeat(a - b, gs, axis=-1)
    want = (sgn << 7 | (exp + shift) << 3 | man).astype(np.uint8)
    assert live.all() and np.array_equal(out, want)


def test_matches_elementwise_torch_computation():
    rng = np.random.default_rng(7)
    E, max_m, K = 3, 5, 384
    x = rng.integers(0, 256, size=(E, max_m, K)).astype(np.uint8)     # NaN codes included
    scales = np.exp2(rng.uniform(-8, 8, size=(E, max_m, K // 128))).astype(np.float32)
    ts = np.float32(0.37)                                              # saturates many values
    out, live = R.requant(x, scales, [5, 0, 3], ts)
    xt = torch.from_numpy(x).view(torch.float8_e4m3fn).to(torch.float32)
    st = torch.from_numpy(scales).repeat_interleave(128, dim=-1)
    r = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(ts)
    v = (xt * st) * r
    nan = torch.isnan(v)
    v = torch.where(nan, torch.zeros_like(v), v.clamp(-448.0, 448.0))
    ref = v.to(torch.float8_e4m3fn).view(torch.uint8)
    ref = torch.where(nan, torch.full_like(ref, 0x7F), ref).numpy()
    assert (out[live] == 0x7E).any() and (out[live] == 0x7F).any()
    assert np.array_equal(out[live], ref[live])


def test_float32_products_decide_ties():
    # x * s lands within half a float32 ulp above an e4m3 midpoint: float32 arithmetic rounds it
    # onto the midpoint (then ties to even), the exact product would round up
    pos = decode_e4m3fn(np.arange(0x7F))
    mids = ((pos[1:] + pos[:-1]) / 2)[8:100]
    xs = pos[40:90]
    cand = []
    for xv in xs:
        for mv in mids:
            s32 = np.float32(mv / xv)
            if np.float32(xv) * s32 == np.float32(mv) and np.float64(xv) * np.float64(s32) > mv:
                cand.append((xv, s32))
    assert len(cand) >= 64
    cand = cand[:128]
    x = R.encode_e4m3fn_sat(np.array([c[0] for c in cand]))
    x = np.repeat(x[:, None], 128, axis=1)[None]                 # [1, n, 128]
    scales = np.array([c[1] for c in cand], dtype=np.float32)[None, :, None]
    out, _ = R.requant(x, scales, [len(cand)], np.float32(1.0))
    v32 = np.float32(decode_e4m3fn(x[0, :, 0])) * scales[0, :, 0]
    assert np.array_equal(out[0, :, 0], _torch_encode(v32))
    exact = decode_e4m3fn(x[0, :, 0]) * scales[0, :, 0].astype(np.float64)
    assert (R.encode_e4m3fn_sat(exact) != out[0, :, 0]).sum() >= 16


def test_live_rows_contract():
    live = R.live_rows([-3, 0, 2, 4, 99], 4)
    assert live.sum(axis=1).tolist() == [0, 0, 2, 4, 4]
    assert live[2].tolist() == [True, True, False, False]


PINS = [
    (test_encode_matches_torch_cast_on_representables_midpoints_and_random, {}),
    (test_encode_saturation_nan_and_zero_by_hand, {}),
    (test_scales_that_cancel_return_every_code, dict(s=3.7)),
    (test_power_of_two_scales_shift_the_exponent_field, {}),
    (test_matches_elementwise_torch_computation, {}),
    (test_float32_products_decide_ties, {}),
    (test_live_rows_contract, {}),
]

_ENC, _VAL, _LIVE = R.encode_e4m3fn_sat, R.requant_values, R.live_rows


def _enc_ties_away(v):
    v = np.asarray(v, dtype=np.float64)
    pos = decode_e4m3fn(np.arange(0x7F))
    a = np.minimum(np.abs(v), 448.0)
    idx = np.argmin(np.abs(pos[None, :] - np.nan_to_num(a).reshape(-1, 1))[:, ::-1], axis=1)
    code = (0x7E - idx).reshape(a.shape)                    # ties resolved to the larger value
    code = code | np.where(np.signbit(v), 0x80, 0)
    return np.where(np.isnan(v), 0x7F, code).astype(np.uint8)


MUTATIONS = {
    "ties away from zero": ("encode_e4m3fn_sat", lambda: _enc_ties_away),
    "no saturation (overflow to NaN)": ("encode_e4m3fn_sat", lambda: (
        lambda v: np.where(np.abs(np.asarray(v, dtype=np.float64)) > 448.0, 0x7F, _ENC(v)).astype(np.uint8))),
    "sign of zero dropped": ("encode_e4m3fn_sat", lambda: (
        lambda v: np.where(np.asarray(v, dtype=np.float64) == 0.0, 0x00, _ENC(v)).astype(np.uint8))),
    "NaN keeps its sign": ("encode_e4m3fn_sat", lambda: (
        lambda v: np.where(np.isnan(v) & np.signbit(v), 0xFF, _ENC(v)).astype(np.uint8))),
    "scale of the wrong group": ("requant_values", lambda: (
        lambda x, s, ts, gs=128: _VAL(x, np.asarray(s)[..., ::-1], ts, gs))),
    "tensor scale multiplied": ("requant_values", lambda: (
        lambda x, s, ts, gs=128: _VAL(x, s, np.float32(1.0) / np.float32(ts), gs))),
    "one multiply in float64": ("requant_values", lambda: (
        lambda x, s, ts, gs=128: (decode_e4m3fn(x) * np.repeat(np.asarray(s, np.float64), gs, axis=-1)
                                  / np.float64(ts)))),
    "row beyond masked_m kept": ("live_rows", lambda: (
        lambda n, max_m: np.arange(max_m)[None, :] <= np.clip(np.asarray(n), 0, max_m)[:, None])),
}


def _failing_pins():
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
    monkeypatch.setattr(R, attr, make())
    assert _failing_pins(), f"no pin catches: {name}"
