"""Pins of the oracle's number formats against library routines and bit-field
definitions (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import formats as F


def _torch_table(dtype):
    return torch.arange(256, dtype=torch.uint8).view(dtype).to(torch.float64).numpy()


def test_e4m3fn_all_codes_match_torch():
    ref = _torch_table(torch.float8_e4m3fn)
    got = F.decode_e4m3fn(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def test_e8m0_all_codes_match_torch():
    ref = _torch_table(torch.float8_e8m0fnu)
    got = F.decode_e8m0(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127


def test_e2m1_table_matches_bitfield_definition():
    # OCP MX E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
    # exponent 0 is subnormal: m * 2^(1 - bias) * 2^-1.
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        want = -mag if s else mag
        got = F.decode_e2m1(np.array([code]))[0]
        assert got == want and math.copysign(1, got) == math.copysign(1, want if want else (-1 if s else 1))


def test_e2m1_values_are_e4m3_representable():
    # every fp4 value survives a round trip through float8 e4m3 (torch cast)
    v = torch.tensor(F.E2M1_VALUES, dtype=torch.float32)
    assert torch.equal(v.to(torch.float8_e4m3fn).to(torch.float32), v)


def test_uint4b8_is_offset_binary():
    got = F.decode_uint4b8(np.arange(16))
    assert list(got) == list(range(-8, 8))


def test_fp16_decode_matches_numpy_for_all_codes():
    # every binary16 pattern: normals, subnormals, signed zeros, infinities and NaNs
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = F.decode_fp16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # hand values: 0x3C00 = 1, 0x4780 = 7.5, 0x0001 = 2^-24 (smallest subnormal), 0x7BFF = 65504
    assert list(F.decode_fp16(np.array([0x3C00, 0x4780, 0x0001, 0x7BFF], np.uint16))) == [1.0, 7.5, 2.0 ** -24, 65504.0]


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = F.decode_bf16(bits)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_round_to_bf16_matches_torch_cast_of_float32():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        (rng.standard_normal(2000) * 1e-36).astype(np.float32),   # bf16 subnormals
        np.array([3.3895314e38, -3.3895314e38, 1e-45], dtype=np.float32),
    ])
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = F.round_to_bf16(vals.astype(np.float64))
    assert np.array_equal(ref, got)


def test_round_to_bf16_ties_and_overflow():
    r = F.round_to_bf16(np.array([
        1 + 2.0 ** -8,               # tie between 1 and 1+2^-7 -> even (1)
        1 + 3 * 2.0 ** -8,           # tie between 1+2^-7 and 1+2^-6 -> even (1+2^-6)
        1 + 2.0 ** -8 + 2.0 ** -30,  # just above the tie -> up (no double rounding)
        -(1 + 2.0 ** -8),
        (2 - 2.0 ** -9) * 2.0 ** 127,  # above the largest bf16 midpoint -> inf
        0.0, -0.0,
    ]))
    assert r[0] == 1.0 and r[1] == 1 + 2.0 ** -6 and r[2] == 1 + 2.0 ** -7
    assert r[3] == -1.0 and r[4] == math.inf
    assert r[5] == 0.0 and math.copysign(1, r[6]) == -1


def test_bf16_bits_roundtrip():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 0x7F80, size=1000).astype(np.uint16)
    assert np.array_equal(F.bf16_bits_of(F.decode_bf16(bits)), bits)
