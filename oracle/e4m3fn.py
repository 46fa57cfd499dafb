"""OCP fp8 e4m3fn decoding, written out from the format's definition.

TEST INFRASTRUCTURE: part of the CPU oracle. Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import it.

The fp8 KV cache stores e4m3fn codes, the OCP variant that gfx950 decodes
natively: the fp8 path of "[ROCm] Add FlyDSL paged-attention decode backend
(dense + fp8) with benchmark" (Other changes: the Triton decode had decoded
gfx950 caches with the fnuz grid and was switched to OCP e4m3fn).

Format of one byte ``s eeee mmm``:

* exponent bias 7;
* e = 0 is subnormal: (-1)^s * (m / 8) * 2^(1 - 7);
* 0 < e < 15, and e = 15 with m < 7, are normal: (-1)^s * (1 + m / 8) * 2^(e - 7);
* e = 15 with m = 7 is NaN (both signs); there is no infinity.

So the largest finite magnitude is 1.75 * 2^8 = 448 and the smallest
positive value is 2^-9.
"""

from __future__ import annotations

import math

import numpy as np

BIAS = 7


def decode_code(code: int) -> float:
    """Value of one e4m3fn byte, as a Python float (exact)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - BIAS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - BIAS)


# All 256 values, built once from decode_code.
DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 e4m3fn codes to float64 (exact)."""
    codes = np.asarray(codes)
    assert codes.dtype == np.uint8, "e4m3fn codes are bytes"
    return DECODE_TABLE[codes]


def dequantise(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Symmetric per-row dequantisation: decode(codes) * scale[..., None].

    ``codes`` has shape [..., D]; ``scale`` has shape [...] (one scale per
    token and kv head). Float64 holds the product exactly: a 4-bit mantissa
    times a 24-bit mantissa needs at most 28 bits.
    """
    return decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


# Finite non-negative values in code order (codes 0x00 .. 0x7E increase with
# the value), for the nearest-value search of ``encode``.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = DECODE_TABLE[:0x7F]


def encode(y: np.ndarray) -> np.ndarray:
    """e4m3fn codes of finite values |y| <= 448, rounded to nearest, ties to even.

    Each |y| lies between two adjacent finite magnitudes (or equals one); the
    nearer one wins and a tie goes to the even code (the code whose mantissa
    LSB is 0, which is how adjacent magnitudes alternate). The sign bit is the
    sign of y, including that of -0.0.
    """
    y = np.asarray(y, dtype=np.float64)
    assert np.all(np.isfinite(y)) and np.all(np.abs(y) <= 448.0), "encode takes |y| <= 448"
    a = np.abs(y)
    hi = np.searchsorted(_POS_VALUES, a, side="left")      # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    exact = _POS_VALUES[hi] == a
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    mag = np.where(exact, _POS_CODES[hi], np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]))
    sign = np.where(np.signbit(y), 0x80, 0x00)
    return (mag | sign).astype(np.uint8)
