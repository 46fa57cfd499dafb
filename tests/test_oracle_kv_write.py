"""The oracle's KV-write step (e4m3fn encoding, per-row quantisation, slot
writes) pinned to things other than itself (CPU only)."""

import numpy as np
import pytest
import torch

from oracle import e4m3fn, kv_write
from workloads import fp8_quantise_per_token


def _torch_codes(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_encode_matches_torch_on_every_value_midpoint_and_random_value():
    vals = e4m3fn.DECODE_TABLE[:0x7F]                      # finite magnitudes
    mids = (vals[:-1] + vals[1:]) / 2                      # exact ties in f32
    rng = np.random.default_rng(1)
    ys = np.concatenate([vals, -vals, mids, -mids, rng.uniform(-448, 448, 50000),
                         rng.uniform(-2.0 ** -8, 2.0 ** -8, 5000), [0.0, -0.0]])
    ys = ys.astype(np.float32)
    assert np.array_equal(e4m3fn.encode(ys), _torch_codes(ys))


def test_encode_then_decode_is_the_identity_on_representable_values():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3fn.decode(codes)
    assert np.array_equal(e4m3fn.encode(vals), codes)


def test_ties_go_to_the_even_code():
    # 1.0 (0x38) and 1.125 (0x39): the midpoint goes down to the even 0x38;
    # 1.125 and 1.25 (0x3A): the midpoint goes up to 0x3A.
    assert e4m3fn.encode(np.array([1.0625]))[0] == 0x38
    assert e4m3fn.encode(np.array([1.1875]))[0] == 0x3A
    # Half the smallest subnormal rounds to zero; just above it rounds up.
    assert e4m3fn.encode(np.array([2.0 ** -10]))[0] == 0x00
    assert e4m3fn.encode(np.array([2.0 ** -10 * 1.01]))[0] == 0x01


def test_row_quantisation_matches_the_independent_torch_quantiser():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 3, 128)).astype(np.float32)
    x[7, 1] = 0.0                                          # zero row: scale 0, codes 0
    x[9, 2, 5] = 1e-30                                     # one tiny row
    x[9, 2, :5] = 0.0
    x[9, 2, 6:] = 0.0
    codes_t, scale_t = fp8_quantise_per_token(torch.from_numpy(x))
    for i in range(x.shape[0]):
        for h in range(x.shape[1]):
            c, s = kv_write.quantise_row(x[i, h])
            assert s == scale_t[i, h].item(), (i, h)
            assert np.array_equal(c, codes_t[i, h].numpy()), (i, h)


def test_row_quantisation_error_bound():
    rng = np.random.default_rng(3)
    for _ in range(200):
        x = (rng.standard_normal(256) * rng.uniform(1e-3, 1e3)).astype(np.float32)
        c, s = kv_write.quantise_row(x)
        deq = e4m3fn.decode(c) * np.float64(s)
        y = np.abs(x.astype(np.float64) / np.float64(s))
        # half an e4m3 ulp at |y| (2^-9 below the normal range), times the scale
        e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
        half_ulp = np.exp2(e - 3) / 2
        assert np.all(np.abs(deq - x) <= (half_ulp + 1e-6 * np.abs(y)) * s)
        assert np.max(np.abs(e4m3fn.decode(c))) == 448.0    # the absmax lands on 448


@pytest.mark.parametrize("fmt", ["dense", "fp8"])
def test_write_kv_lands_in_the_named_slots_only(fmt):
    rng = np.random.default_rng(4)
    P, bs, H, D, N = 6, 4, 2, 8, 7
    if fmt == "fp8":
        kp = rng.integers(0, 120, (P, bs, H, D)).astype(np.uint8)
        ks = rng.uniform(0.1, 1, (P, bs, H)).astype(np.float32)
    else:
        kp = rng.standard_normal((P, bs, H, D)).astype(np.float32)
        ks = None
    vp, vs = kp.copy(), None if ks is None else ks.copy()
    nk = rng.standard_normal((N, H, D)).astype(np.float32)
    nv = rng.standard_normal((N, H, D)).astype(np.float32)
    slots = np.array([5, 0, -1, 23, 12, -7, 9])
    k2, v2, ks2, vs2 = kv_write.write_kv(kp, vp, nk, nv, slots, kv_format=fmt,
                                         k_scale=ks, v_scale=vs)
    touched = np.zeros((P, bs), bool)
    for i, sl in enumerate(slots):
        if sl < 0:
            continue
        p, o = sl // bs, sl % bs
        touched[p, o] = True
        if fmt == "dense":
            assert np.array_equal(k2[p, o], nk[i]) and np.array_equal(v2[p, o], nv[i])
        else:
            for h in range(H):
                back = e4m3fn.decode(k2[p, o, h]) * np.float64(ks2[p, o, h])
                assert np.allclose(back, nk[i, h], rtol=0.07, atol=1e-6)
    assert np.array_equal(k2[~touched], kp[~touched]) and np.array_equal(v2[~touched], vp[~touched])
    if fmt == "fp8":
        assert np.array_equal(ks2[~touched], ks[~touched])


def test_head_major_write_is_the_transposed_token_major_write():
    rng = np.random.default_rng(91)
    P, bs, H, D, N = 5, 4, 3, 16, 14
    kp = rng.integers(0, 126, (P, bs, H, D)).astype(np.uint8)
    vp = rng.integers(0, 126, (P, bs, H, D)).astype(np.uint8)
    ks = rng.random((P, bs, H)).astype(np.float32)
    vs = rng.random((P, bs, H)).astype(np.float32)
    nk = rng.standard_normal((N, H, D)).astype(np.float32)
    nv = rng.standard_normal((N, H, D)).astype(np.float32)
    slots = rng.permutation(P * bs)[:N].astype(np.int64)
    slots[3] = -1
    tok = kv_write.write_kv(kp, vp, nk, nv, slots, kv_format="fp8", k_scale=ks, v_scale=vs)
    t = lambda a: np.ascontiguousarray(np.swapaxes(a, 1, 2))  # noqa: E731
    head = kv_write.write_kv(t(kp), t(vp), nk, nv, slots, kv_format="fp8", k_scale=t(ks),
                             v_scale=t(vs), kv_layout="head")
    for a, b in zip(tok, head):
        assert np.array_equal(t(a), b)


def test_f16_scale_rounding_is_nearest_even_as_in_torch():
    """The oracle's f32 -> f16 scale rounding (numpy's cast) against torch's
    independent cast, on every f16 midpoint (exact ties), subnormal-range
    values and values past the largest finite f16 (capped first)."""
    f16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((f16[:-1] + f16[1:]) / 2).astype(np.float32)     # exact in f32
    rng = np.random.default_rng(11)
    vals = np.concatenate([mids, np.exp2(rng.uniform(-30, 20, 20000)),
                           [65504.0, 65519.0, 65520.0, 1e9, 0.0]]).astype(np.float32)
    capped = np.minimum(vals, kv_write.F16_MAX)
    ours = capped.astype(np.float16)
    theirs = torch.from_numpy(capped).to(torch.float16).numpy()
    assert np.array_equal(ours.view(np.uint16), theirs.view(np.uint16))
    # ties go to the even f16 code
    codes = mids.astype(np.float16).view(np.uint16)
    assert np.all(codes % 2 == 0)


def test_f16_scale_quantisation_matches_the_generator():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((200, 2, 64)).astype(np.float32)
    x *= np.exp2(rng.uniform(-40, 30, (200, 2, 1))).astype(np.float32)  # subnormal..capped scales
    x[3, 0] = 0.0
    codes_t, scale_t = fp8_quantise_per_token(torch.from_numpy(x), "f16")
    assert scale_t.dtype == torch.float16
    for i in range(x.shape[0]):
        for h in range(x.shape[1]):
            c, s = kv_write.quantise_row(x[i, h], "f16")
            assert np.float16(s) == s and s == np.float32(scale_t[i, h].item()), (i, h)
            assert np.array_equal(c, codes_t[i, h].numpy()), (i, h)


def test_f16_scale_write_stores_half_precision_scales():
    rng = np.random.default_rng(13)
    P, bs, H, D, N = 4, 4, 2, 16, 9
    kp = np.zeros((P, bs, H, D), np.uint8)
    ks = np.zeros((P, bs, H), np.float16)
    nk = (rng.standard_normal((N, H, D)) * 1e-3).astype(np.float32)
    slots = rng.permutation(P * bs)[:N].astype(np.int64)
    rk, _, rks, _ = kv_write.write_kv(kp, kp, nk, nk, slots, kv_format="fp8", k_scale=ks,
                                      v_scale=ks)
    assert rks.dtype == np.float16
    for i, sl in enumerate(slots):
        for h in range(H):
            c, s = kv_write.quantise_row(nk[i, h], "f16")
            assert rks[sl // bs, sl % bs, h] == s
            assert np.array_equal(rk[sl // bs, sl % bs, h], c)
