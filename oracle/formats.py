"""Number formats of the oracle: explicit decode tables in float64.

Test infrastructure only (see the package docstring).

* E2M1 (OCP MX fp4): 1 sign, 2 exponent bits with bias 1, 1 mantissa bit.
  The packed-weight dtype of the NVFP4 and MXFP4 paths ("packed E2M1" in the
  Muse Spark experiment's ``Weights``; ``float4_e2m1f`` as ``b_q_type``).
* uint4b8 (int4): the stored nibble ``u`` means ``u - 8`` (the
  ``scalar_types.uint4b8`` quant type of the sglang PR 31552 unit test).
* float8 e4m3fn: the NVFP4 per-16 block scale (``w13_sf`` in ``Weights``).
* E8M0: the MXFP4 per-32 block scale, ``2^(e - 127)``.
* bf16: activations, biases, int4 scales and every stored intermediate.
* float16 (IEEE binary16): the zero points of the asymmetric int4 format with
  float zero points (the Marlin template's ``is_zp_float`` case).

Pins: e4m3fn and E8M0 against torch's ``float8_e4m3fn`` / ``float8_e8m0fnu``
views for all 256 codes; E2M1 against its bit-field definition; bf16
decode/rounding against torch's float32 casts plus hand-built ties; float16
against numpy's ``float16`` view for all 65536 codes.
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes for codes 0..7; codes 8..15 are the same values negated.
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)


def decode_e2m1(nibbles: np.ndarray) -> np.ndarray:
    return E2M1_VALUES[np.asarray(nibbles, dtype=np.int64)]


def decode_uint4b8(nibbles: np.ndarray) -> np.ndarray:
    return np.asarray(nibbles, dtype=np.float64) - 8.0


def decode_uint4(nibbles: np.ndarray) -> np.ndarray:
    """Plain unsigned 4-bit value 0..15 (the asymmetric int4 format, whose zero point is separate)."""
    return np.asarray(nibbles, dtype=np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """float8 e4m3fn: bias 7, subnormals at exponent 0, S.1111.111 is NaN, no inf."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """E8M0: a bare exponent, 2^(e - 127); code 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.exp2(c.astype(np.float64) - 127.0))


def decode_fp16(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64: 1 sign, 5 exponent bits with bias 15,
    10 mantissa bits; exponent 0 holds the subnormals m * 2^-24, exponent 31 infinities (m = 0)
    and NaN."""
    c = np.asarray(bits).astype(np.int64)
    sign = np.where(c >> 15, -1.0, 1.0)
    e = (c >> 10) & 0x1F
    m = (c & 0x3FF).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -24, (1.0 + m / 1024.0) * np.exp2(e.astype(np.float64) - 15.0))
    mag = np.where(e == 0x1F, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # NaN payloads stay NaN
        return b.view(np.float32).astype(np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even (a single
    rounding, no intermediate float32).  Keeps NaN, overflows to +-inf."""
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, copy=True)
    fin = np.isfinite(v) & (v != 0)
    if np.any(fin):
        a = v[fin]
        _, e = np.frexp(a)                      # a = f * 2^e, 0.5 <= |f| < 1
        q = np.exp2(np.maximum(e, -125) - 8.0)  # spacing of 8 significant bits
        r = np.rint(a / q) * q                  # np.rint rounds half to even
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
        out[fin] = r
    return out


def bf16_bits_of(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values that are already bf16-representable."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
