"""OCP FP8 E4M3 ("E4M3FN") codes for the quantised KV cache.

"KV cache: la memoria de trabajo ..." (blog.lo0.es), "Trucos para que el
cuaderno sea mas fino": the cache can be stored in 8 bits, which halves its
size and the bytes each decode step reads; "PagedAttention por dentro"
(blog.lo0.es), "Trampas y mitos comunes": an FP8 cache is described as safe
almost always.  The pages fix
neither the 8-bit format nor how values are scaled.  Readings:
  - the format is OCP 8-bit floating point E4M3: 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 holds the
    subnormals m * 2^-9; the all-ones exponent with mantissa 7 is NaN;
    there is no infinity, so the largest finite magnitude is 448;
  - one scale per tensor (K and V separately): a stored code c stands for
    decode(c) * scale;
  - a value x is quantised as y = float32(x) * float32(1 / scale) (one
    float32 multiply) and then rounded to the nearest E4M3 value, ties to the
    code with the even mantissa; magnitudes beyond 448 are clamped to 448,
    and NaN becomes the NaN code with the input's sign.

Written from that definition: every code is decoded by its fields, and
encoding is a nearest search over the 127 non-negative finite values (in
float64, where y is exact; the two neighbours of y are compared).
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e.astype(np.float64) - 10))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


# the non-negative finite codes 0x00 .. 0x7E and their values, increasing
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = decode(_POS_CODES)


def encode_f32(y) -> np.ndarray:
    """float32 values -> uint8 codes: nearest E4M3 value, ties to the even
    mantissa (the even code), clamped to +-448, NaN -> NaN code."""
    y = np.asarray(y, dtype=np.float32)
    nan = np.isnan(y)
    a = np.minimum(np.abs(np.where(nan, 0, y).astype(np.float64)), MAX_FINITE)
    hi = np.minimum(np.searchsorted(_POS_VALUES, a), len(_POS_VALUES) - 1)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    code = np.where(dhi == 0, hi,
                    np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi))))
    code = np.where(nan, NAN_CODE, code).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << 7)


def quantize(x, scale: float) -> np.ndarray:
    """Stored codes for values x (float32, or anything widened to it)."""
    inv = np.float32(1.0) / np.float32(scale)
    y = np.asarray(x, dtype=np.float32) * inv
    return encode_f32(y)
