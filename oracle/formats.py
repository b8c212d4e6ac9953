"""Number formats, written out from their definitions (oracle; test infrastructure).

bf16: the upper 16 bits of an IEEE-754 binary32 value.

OCP 8-bit floating point, E4M3FN flavour (the FP8 type the pages quantise K, V and
Q to; FlashMLA PR #54 "Functionality", FlashInfer PR #869 item 2, where the P scale
is the format's largest finite value): 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits; exponent field 0 encodes subnormals 2^-6 * m/8; the pattern
S.1111.111 is NaN; there are no infinities; the largest finite magnitude is
1.75 * 2^8 = 448.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16/int16) -> float64, exactly."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_code_to_f64(codes: np.ndarray) -> np.ndarray:
    """E4M3FN codes (uint8) -> float64, from the bit fields (NaN for S.1111.111)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m / 8.0, -6)
    mag = np.where(e == 0, sub, normal)
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def _e4m3_positive_table():
    codes = np.arange(0, 0x7F, dtype=np.int64)          # 0x00..0x7E: all finite non-negative
    vals = e4m3_code_to_f64(codes)
    assert np.all(np.diff(vals) > 0)
    return codes, vals


_POS_CODES, _POS_VALS = _e4m3_positive_table()


def f64_to_e4m3_rne(x: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3FN value, ties to the code with an even last
    mantissa bit.  Inputs must already be finite and within [-448, 448] (the
    quantiser clamps first).  The sign of zero is kept (-0.0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("f64_to_e4m3_rne: input outside the finite E4M3 range")
    a = np.abs(x)
    hi = np.searchsorted(_POS_VALS, a, side="left")      # first table value >= a
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(_POS_VALS[hi] == a, _POS_CODES[hi], code)   # exact hits
    neg = np.signbit(x)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest, ties to even (the upper 16
    bits of the float32 after adding 0x7FFF plus the lowest kept bit); NaN stays a
    quiet NaN."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    return np.where(nan, (u >> 16) | 0x40, rounded).astype(np.uint16)
