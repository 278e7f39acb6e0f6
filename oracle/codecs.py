"""Number formats used by the oracle, written from their definitions.

bf16: the top 16 bits of an IEEE-754 binary32; fp32 -> bf16 rounds to nearest,
ties to even.  e4m3 (OCP 8-bit float, "fn" variant): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent 0 encodes subnormals m/8 * 2^-6;
there is no infinity and S.1111.111 is NaN, so the largest finite value is
1.75 * 2^8 = 448.  The pages say only that an FP8 checkpoint exists (Reflection
Beam 1.0 overview, section "Mixture of Experts"); the OCP e4m3 reading is the
one this layer adopts.

MXFP4 (OCP Microscaling, the MI355X analogue of the pages' NVFP4 checkpoint:
Reflection Beam 1.0 overview, section "Mixture of Experts" lists BF16, FP8 and
NVFP4 checkpoints): blocks of 32 consecutive values along the reduction share
one E8M0 scale 2^(e-127) (e = 255 is NaN); each value is FP4 E2M1: 1 sign bit,
2 exponent bits with bias 1, 1 mantissa bit; exponent 0 is subnormal (m * 0.5),
so the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Two codes per byte, the
lower-indexed value in the low nibble.  Quantisation (the format's conversion
rule): shared exponent = floor(log2(max |v| of the block)) - 2 (2 = E2M1's
largest exponent), clamped to the scale's range; each value v / 2^shared is
rounded to the nearest E2M1 value, ties to even mantissa, magnitudes past 6
saturate to 6; an all-zero block takes e = 0.

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


def _e2m1_table() -> np.ndarray:
    """All 16 E2M1 codes decoded from the bit-field definition."""
    out = np.zeros(16, np.float64)
    for c in range(16):
        sign = -1.0 if c & 8 else 1.0
        e = (c >> 1) & 3
        m = c & 1
        mag = (m * 0.5) if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
        out[c] = sign * mag
    return out


_E2M1 = _e2m1_table()


def e2m1_decode(codes) -> np.ndarray:
    """4-bit E2M1 codes (0..15) -> float64 values."""
    return _E2M1[np.asarray(codes, np.uint8) & 15]


def e8m0_scale(e) -> np.ndarray:
    """E8M0 scale bytes -> float64 2^(e-127); 255 -> NaN."""
    e = np.asarray(e, np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, (e - 127).astype(np.int64)))


def mxfp4_unpack(packed) -> np.ndarray:
    """[..., n/2] bytes -> [..., n] codes, the lower-indexed value from the low nibble."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def mxfp4_dequant(packed, scales) -> np.ndarray:
    """Packed E2M1 codes [rows, n/2] and E8M0 scales [rows, n/32] -> float64 [rows, n] (exact)."""
    v = e2m1_decode(mxfp4_unpack(packed))
    s = e8m0_scale(scales)
    return v * np.repeat(s, 32, axis=-1)


def _e2m1_round(u: np.ndarray) -> np.ndarray:
    """|v| / 2^shared (exact, < 8) -> E2M1 magnitude code 0..7, nearest, ties to even mantissa, saturating."""
    grid = _E2M1[:8]
    code = np.zeros(u.shape, np.uint8)
    # midpoints between consecutive grid values; at a midpoint the even code (mantissa 0) wins
    for c in range(1, 8):
        mid = 0.5 * (grid[c - 1] + grid[c])
        above = (u > mid) | ((u == mid) & (c % 2 == 0))
        code = np.where(above, c, code).astype(np.uint8)
    return code


def mxfp4_quantize(v_bits):
    """bf16 bits [rows, n] (n % 32 == 0) -> (packed codes [rows, n/2] uint8, E8M0 scales [rows, n/32] uint8)."""
    v = bf16_to_f64(np.asarray(v_bits, np.uint16))
    rows, n = v.shape
    blocks = v.reshape(rows, n // 32, 32)
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        ex = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))), 0.0).astype(np.int64)
    shared = np.clip(ex - 2, -127, 127)
    e = np.where(amax > 0, shared + 127, 0).astype(np.uint8)
    u = np.abs(blocks) / np.ldexp(1.0, (e.astype(np.int64) - 127))[..., None]
    mag = _e2m1_round(u)
    codes = (mag | np.where(blocks < 0, 8, 0).astype(np.uint8)).reshape(rows, n)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, e
