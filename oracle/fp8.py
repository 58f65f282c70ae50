"""FP8 E4M3 (the OCP "E4M3FN" layout) for the oracle's fp8 KV cache
-- TEST INFRASTRUCTURE ONLY.

[Blog] "vLLM engineering details" (the serving configuration stores the KV
cache in fp8). A code is 1 sign bit, 4 exponent bits (bias 7) and 3 mantissa
bits: exponent field 0 encodes subnormals m * 2^-9, fields 1..15 encode
(1 + m/8) * 2^(e-7), except S.1111.111 which is NaN; there is no infinity,
and the largest finite magnitude is 448 (S.1111.110).

Readings: values are stored as x / scale (a per-layer scale for K and one
for V, given with the model) rounded to the nearest code, ties to the even
mantissa, and saturated to +-448 (a cache never holds NaN); reading a code
gives its value times the scale.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Values (float64) of E4M3 codes (uint8)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code (ties to even mantissa), saturating at +-448.
    NaN inputs are not expected (the cache never stores them)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # the spacing of the codes around a: 2^(e-3) for binades e >= -6, 2^-9 below
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = np.exp2(e - 3.0)
    q = a / step                               # exact: a power-of-two division
    lo = np.floor(q)
    frac = q - lo
    up = (frac > 0.5) | ((frac == 0.5) & (lo % 2 == 1))
    n = (lo + up) * step                       # the rounded magnitude, on the code grid
    n = np.minimum(n, E4M3_MAX)
    # back to fields: subnormal below 2^-6, else exponent and mantissa
    sub = n < 2.0 ** -6
    mant_sub = np.round(n / 2.0 ** -9)
    en = np.floor(np.log2(np.where(n > 0, n, 1.0)))
    mant = np.round((n / np.exp2(en) - 1.0) * 8.0)
    code = np.where(sub, mant_sub, (en + 7) * 8 + mant).astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)   # the sign bit, -0 included
    return code.astype(np.uint8)


def fp8_roundtrip(x, scale: float) -> np.ndarray:
    """What the cache holds for x: the code of x / scale, read back times scale."""
    return e4m3_decode(e4m3_encode(np.asarray(x, np.float64) / scale)) * scale
