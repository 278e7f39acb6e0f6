"""Number formats used by the oracle, written from their definitions.

bf16: the top 16 bits of an IEEE-754 binary32; fp32 -> bf16 rounds to nearest,
ties to even.  e4m3 (OCP 8-bit float, "fn" variant): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent 0 encodes subnormals m/8 * 2^-6;
there is no infinity and S.1111.111 is NaN, so the largest finite value is
1.75 * 2^8 = 448.  The pages say only that an FP8 checkpoint exists (Reflection
Beam 1.0 overview, section "Mixture of Experts"); the OCP e4m3 reading is the
one this layer adopts.

Test infrastructure only: never imported by the product path.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    u = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32(a) -> np.ndarray:
    """Round to nearest-even binary32 (NumPy's float64 -> float32 cast is IEEE RNE)."""
    return np.asarray(a, np.float64).astype(np.float32)


def bf16_round_bits(a) -> np.ndarray:
    """float32 values -> bf16 bit patterns, round to nearest, ties to even.

    Inputs are rounded to float32 first (callers pass float32 already).
    NaN maps to a quiet NaN with the same sign; infinities are preserved.
    """
    x = np.asarray(a, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint32)
        r = np.where(nan, sign | np.uint32(0x7FC0), r)
    return r.astype(np.uint16)


def bf16_round(a) -> np.ndarray:
    """float32 -> bf16 -> float64 (the value after rounding)."""
    return bf16_to_f64(bf16_round_bits(a))


def _e4m3_table() -> np.ndarray:
    t = np.empty(256, np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            t[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_VALUES = _e4m3_table()


def e4m3_decode(codes) -> np.ndarray:
    """e4m3 bytes (uint8) -> exact float64 values."""
    return E4M3_VALUES[np.asarray(codes, np.uint8)]
