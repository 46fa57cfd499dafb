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
