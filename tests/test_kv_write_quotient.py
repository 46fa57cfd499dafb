"""The fp8 KV write's quotient method, emulated exactly on the CPU.

The write kernel computes x / scale for a whole row from one correctly
rounded reciprocal r = RN(1/scale): q = RN(x * r), e = fma(-q, scale, x),
y = fma(e, r, q) (Markstein's correction step), with x itself for zero and
infinite x. This test replays that arithmetic in binary32 with every fma
rounded once (products of two binary32 values are exact in binary64, the
residual is exact by Sterbenz's lemma, and a sum that lands on a binary32
midpoint in binary64 is redone in exact rational arithmetic) and requires
y == RN(x / scale), the IEEE quotient the oracle's quantiser uses, for every
bf16 and f16 input (both signs, zeros, subnormals) against a set of scales:
random ones over the whole range the write allows on this path (2^-64 up),
the row scales of powers of two and of all-ones significands, and the f16
storage of such scales. The kernel's own search was exhaustive over every
scale; this CPU test samples them so the suite stays fast.
"""

from fractions import Fraction

import numpy as np
import pytest

E4M3_MAX = np.float32(448.0)


def _all_inputs(kind):
    if kind == "bf16":
        bits = np.arange(0, 0x7F80, dtype=np.uint32)
        pos = (bits << 16).view(np.float32)
    else:
        bits = np.arange(0, 0x7C00, dtype=np.uint16)
        pos = bits.view(np.float16).astype(np.float32)
    return np.concatenate([pos, -pos, np.array([np.inf, -np.inf], dtype=np.float32)])


def _scales(rng, kind_scale):
    absmax = np.concatenate([
        np.exp2(rng.uniform(-60, 127, 300)),
        np.exp2(np.arange(-50, 120, 7, dtype=np.float64)),
        (2.0 - 2.0 ** -7) * np.exp2(np.arange(-50, 120, 9, dtype=np.float64)),  # bf16 all ones
    ]).astype(np.float32)
    s = (absmax / E4M3_MAX).astype(np.float32)
    if kind_scale == "f16":
        s = np.minimum(s, np.float32(65504.0)).astype(np.float16).astype(np.float32)
    s = s[(s >= np.float32(2.0 ** -64)) & np.isfinite(s)]
    return np.unique(s)


def _round_sum_f32(q, e, r):
    """RN_binary32(q + e * r) with one rounding (q, e, r binary32 values)."""
    s64 = q.astype(np.float64) + e.astype(np.float64) * np.float64(r)
    y = s64.astype(np.float32)
    up = np.nextafter(y, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(y, np.float32(-np.inf)).astype(np.float64)
    mid = (s64 == (y.astype(np.float64) + up) / 2) | (s64 == (y.astype(np.float64) + dn) / 2)
    for i in np.nonzero(mid & np.isfinite(s64))[0]:
        exact = Fraction(float(q[i])) + Fraction(float(e[i])) * Fraction(float(r))
        c = np.float32(float(exact))
        cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
        y[i] = min(cands, key=lambda v: (abs(Fraction(float(v)) - exact),
                                         int(np.array(v).view(np.uint32)) & 1))
    return y


def _kernel_quotient(x, b):
    r = np.float32(np.float32(1.0) / b)
    with np.errstate(over="ignore", invalid="ignore"):
        q = (x.astype(np.float64) * np.float64(r)).astype(np.float32)
        e = (x.astype(np.float64) - q.astype(np.float64) * np.float64(b)).astype(np.float32)
        y = _round_sum_f32(q, e, r)
    self = (x == 0) | np.isinf(x)
    return np.where(self, x, y)


@pytest.mark.parametrize("inputs", ["bf16", "f16"])
@pytest.mark.parametrize("scale_kind", ["f32", "f16"])
def test_quotient_from_the_row_reciprocal_is_the_ieee_quotient(inputs, scale_kind):
    rng = np.random.default_rng(7 + (inputs == "f16") + 2 * (scale_kind == "f16"))
    x = _all_inputs(inputs)
    checked = 0
    for b in _scales(rng, scale_kind):
        b = np.float32(b)
        with np.errstate(over="ignore"):
            want = (x / b).astype(np.float32)
        # Quotients whose e4m3 code depends on the exact rounding; outside
        # this band both give code 0 or clamp to +-448.
        band = (np.abs(want) >= np.float32(2.0 ** -11)) & \
               (np.abs(want) <= np.float32(448.0 * (1 + 2.0 ** -8)))
        band |= (x == 0) | np.isinf(x)
        got = _kernel_quotient(x[band], b)
        w = want[band]
        same = (got.view(np.uint32) == w.view(np.uint32))
        assert same.all(), (float(b), x[band][~same][:4], got[~same][:4], w[~same][:4])
        checked += int(band.sum())
    assert checked > 100_000


def test_emulation_catches_a_planted_error():
    """Without the zero case the method gives +0 for -0 / scale: the check must see it."""
    x = np.array([-0.0, 3.0, -5.5], dtype=np.float32)
    b = np.float32(0.0078125)
    r = np.float32(np.float32(1.0) / b)
    q = (x.astype(np.float64) * np.float64(r)).astype(np.float32)
    e = (x.astype(np.float64) - q.astype(np.float64) * np.float64(b)).astype(np.float32)
    raw = _round_sum_f32(q, e, r)
    want = (x / b).astype(np.float32)
    assert raw.view(np.uint32)[0] != want.view(np.uint32)[0]   # +0 vs -0
    assert (_kernel_quotient(x, b).view(np.uint32) == want.view(np.uint32)).all()
