"""CPU oracle of the W4AFP8 activation requant (test infrastructure only).

Like the rest of ``oracle/``, this module exists to check the HIP library: only the tests,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import it, it shares
no code with the HIP path and imports nothing from it.

Source: the "sglang PR 35760" summary on prhub.com.cn (W4AFP8 requant launch geometry),
sections "Feature and motivation" and "Implementation breakdown" items 1-2.  After the
low-latency dispatch the activations of expert ``e`` sit in a masked layout: ``max_m`` row
slots of ``K`` float8 e4m3fn values, of which the first ``masked_m[e]`` are live, with one
float32 scale per row and 128-wide group of ``K`` (per-token-group quantisation; the scale
array may be row- or column-major).  The requant turns them into float8 values for one
per-tensor scale.  The page fixes the arithmetic only as "two multiplies per element, two
bytes moved" and the scale as one load per group; the readings taken here:

* element (e, m, k) of a live row: ``v = float32(float32(x * s) * r)`` with ``x`` the decoded
  code, ``s = scales[e, m, k // group_size]`` and ``r = float32(1 / tensor_scale)`` (one
  reciprocal per launch, then the two multiplies the page names, in that order);
* ``v`` becomes a float8 e4m3fn code with saturation: NaN -> 0x7F, otherwise clamped to
  [-448, 448] and rounded to the nearest value, ties to the even code; the sign of zero
  is kept (-0.0 -> 0x80);
* rows ``m >= masked_m[e]`` (after clamping ``masked_m`` to ``[0, max_m]``) are neither read
  nor written.

The result does not depend on the launch geometry (tile width, programs per expert, row cap,
overflow sharing): every output byte is a function of its own input byte and scale.

Pins (``tests/test_oracle_requant.py``): the encoder against torch's float32 ->
``float8_e4m3fn`` cast on every representable value, every midpoint and random values,
plus hand-computed saturation / NaN / zero cases; the requant against closed forms (scales
that cancel return every input code; power-of-two scales shift the exponent field by a known,
per-row and per-group distinct amount), against an element-by-element torch computation on a
small input, and against its masked-row contract.  Planted mistakes in this module must fail
one of those pins (the same test file).
"""
from __future__ import annotations

import numpy as np

from .formats import decode_e4m3fn

E4M3_MAX = 448.0
E4M3_NAN = 0x7F

# the 127 non-negative finite e4m3fn values, increasing with the code (0x00 .. 0x7E)
_POS_VALUES = decode_e4m3fn(np.arange(0x7F))


def encode_e4m3fn_sat(v) -> np.ndarray:
    """Real values -> float8 e4m3fn codes (uint8): NaN -> 0x7F; otherwise the magnitude is
    clamped to 448 and rounded to the nearest representable value, a tie going to the code
    whose last (mantissa) bit is 0; the sign bit is the value's sign bit (so -0.0 -> 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    with np.errstate(invalid="ignore"):
        hi = np.clip(np.searchsorted(_POS_VALUES, np.nan_to_num(a), side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.int64)
    code |= np.where(np.signbit(v), 0x80, 0)
    code = np.where(np.isnan(v), E4M3_NAN, code)
    return code.astype(np.uint8)


def live_rows(masked_m, max_m: int) -> np.ndarray:
    """bool [E, max_m]: row m of expert e is live iff m < clamp(masked_m[e], 0, max_m)."""
    n = np.clip(np.asarray(masked_m, dtype=np.int64), 0, max_m)
    return np.arange(max_m)[None, :] < n[:, None]


def requant_values(x_codes, scales, tensor_scale, group_size: int = 128) -> np.ndarray:
    """float32 [..., K] values ``(x * s) * r`` before the conversion back to float8.
    x_codes uint8 [..., K]; scales float32 [..., K / group_size] (same leading shape)."""
    x = decode_e4m3fn(x_codes).astype(np.float32)            # exact: e4m3 fits in float32
    s = np.repeat(np.asarray(scales, dtype=np.float32), group_size, axis=-1)
    assert s.shape == x.shape, (s.shape, x.shape)
    r = np.float32(1.0) / np.float32(tensor_scale)            # correctly rounded float32
    with np.errstate(invalid="ignore", over="ignore"):
        return (x * s) * r                                    # two float32 multiplies


def requant(x_codes, scales, masked_m, tensor_scale, group_size: int = 128):
    """The requant of a masked ``[E, max_m, K]`` batch.

    Returns ``(out, live)``: ``out`` uint8 ``[E, max_m, K]`` holds the new codes in live rows and
    zeros elsewhere (the kernel leaves those bytes untouched), ``live`` is ``live_rows``."""
    x_codes = np.asarray(x_codes, dtype=np.uint8)
    E, max_m, K = x_codes.shape
    assert K % group_size == 0
    scales = np.asarray(scales, dtype=np.float32)
    assert scales.shape == (E, max_m, K // group_size), scales.shape
    live = live_rows(masked_m, max_m)
    out = np.zeros_like(x_codes)
    if live.any():
        out[live] = encode_e4m3fn_sat(requant_values(x_codes[live], scales[live], tensor_scale,
                                                     group_size))
    return out, live
