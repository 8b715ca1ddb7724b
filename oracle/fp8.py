"""Oracle: OCP 8-bit floating point E4M3 codec and the FP8 KV write — test infrastructure only.

Definitions followed
  * E4M3 (the OCP 8-bit floating point format, "E4M3FN"): 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits. Exponent field 0 holds subnormals m * 2^-9; fields 1..15 hold
    normals 2^(e-7) * (1 + m/8); the one pattern S.1111.111 is NaN and there is no infinity,
    so the largest finite magnitude is 2^8 * 1.75 = 448.
  * Encoding a float32 value rounds to the nearest finite E4M3 value with ties to the even
    mantissa, keeps the sign (also of zero), and saturates magnitudes beyond 448 to 448.
  * FP8 KV with per-tensor scales: a pool stores code = encode(x * inv_scale) per element,
    where inv_scale = 1 / scale is rounded to float32 once and the product is one float32
    multiply; a read dequantises to decode(code) * scale ("P3: native paged-KV
    continuous-batching sampler", quantised KV is one of its lossy modes; "Finish RL Training
    Faster: Bitwise-Consistent ...", FP8 KV at about 57 % of the BF16 bytes).
Nothing here depends on the HIP path.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (exact); NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = s * mag
    out = np.where((e == 15) & (m == 7), np.nan, out)
    return out


# the 127 finite non-negative magnitudes, ascending with their codes 0x00 .. 0x7E
_MAG_CODES = np.arange(0x7F, dtype=np.uint8)
_MAG_VALUES = e4m3_decode(_MAG_CODES)


def e4m3_encode(x) -> np.ndarray:
    """float32 values -> uint8 codes: nearest finite E4M3 value, ties to the even mantissa,
    sign kept, magnitudes beyond 448 saturated to 448. NaN inputs are refused."""
    xs = np.asarray(x, dtype=np.float32)
    if np.isnan(xs).any():
        raise ValueError("e4m3_encode: NaN input")
    a = np.abs(xs.astype(np.float64))
    neg = np.signbit(xs)
    a = np.minimum(a, E4M3_MAX)
    # index of the largest grid value <= a, and its upper neighbour
    lo = np.searchsorted(_MAG_VALUES, a, side="right") - 1
    lo = np.clip(lo, 0, len(_MAG_VALUES) - 1)
    hi = np.minimum(lo + 1, len(_MAG_VALUES) - 1)
    dlo = a - _MAG_VALUES[lo]
    dhi = _MAG_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & (_MAG_CODES[hi] % 2 == 0))
    mag = np.where(pick_hi, _MAG_CODES[hi], _MAG_CODES[lo]).astype(np.uint8)
    return np.where(neg, mag | np.uint8(0x80), mag).astype(np.uint8)


def inv_scale_f32(scale: float) -> np.float32:
    """1 / scale rounded to float32 (the factor every element is multiplied by)."""
    return np.float32(np.float32(1.0) / np.float32(scale))


def quantize_rows(x, scale: float) -> np.ndarray:
    """float32 (or bfloat16-valued float32) rows -> E4M3 codes with one float32 multiply each."""
    xf = np.asarray(x, dtype=np.float32)
    return e4m3_encode(xf * inv_scale_f32(scale))


def dequantize(codes, scale: float) -> np.ndarray:
    """E4M3 codes -> float64 values times the per-tensor scale."""
    return e4m3_decode(codes) * np.float64(np.float32(scale))
