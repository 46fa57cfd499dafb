"""Planted mistakes in the oracle must trip at least one pin (CPU only).

Each test swaps one helper of the oracle for a plausibly wrong version (a
wrong GQA head mapping, a dropped softmax scale, an off-by-one page, a wrong
split partition, a base-2 LSE, a flipped fp8 exponent bias, causal-mask
slips, round-half-up encoding, ignored per-sequence counts, head-major pages
read with token-major axes, truncated f16 scales) and checks that the pins
report a deviation far above their tolerance, or fail. This shows the pins
can see the kinds of mistakes they are meant to catch.
"""

import math

import numpy as np

import oracle
import oracle_pins as pins
from oracle import e4m3fn
from oracle import paged_decode as pa

TOL = 1e-12


def _case(**kw):
    return pins.random_contiguous_case(3, **kw)


def test_wrong_gqa_head_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(pa, "kv_head_of", lambda h, hq, hkv: h % hkv)
    assert pins.check_against_sdpa(_case(Hq=8, Hkv=2)) > 1e-3


def test_dropped_scale_is_caught(monkeypatch):
    real = pa.attend
    monkeypatch.setattr(pa, "attend", lambda q, K, V, scale: real(q, K, V, 1.0))
    assert pins.check_against_sdpa(_case()) > 1e-3
    assert pins.check_identical_keys() > 1e-3


def test_off_by_one_page_is_caught(monkeypatch):
    real = pa._token_rows

    def shifted(pages, scale, row, ctx, bs, h_kv, fmt, layout="token"):
        row = np.asarray(row).copy()
        if len(row) > 1:
            row[1:] = row[:-1].copy()
        return real(pages, scale, row, ctx, bs, h_kv, fmt, layout)

    monkeypatch.setattr(pa, "_token_rows", shifted)
    assert pins.check_needle() > 1e-3
    assert pins.check_against_sdpa(_case(lens=(9, 17, 33))) > 1e-3


def test_wrong_split_partition_is_caught(monkeypatch):
    def overlapping(ctx, bs, S):
        return [(0, ctx)] * S          # every split sees the whole context

    monkeypatch.setattr(pa, "split_token_ranges", overlapping)
    assert pins.check_split_combine(_case(lens=(5, 9, 33)), splits=(2, 3)) > 1e-3


def test_scratch_in_the_first_split_is_caught(monkeypatch):
    # The combined result does not see where the scratch tokens go; the
    # per-split brute force does.
    monkeypatch.setattr(pa, "owns_scratch", lambda s, S: s == 0)
    c = pins.random_contiguous_case(3, B=3, Tq=2, Hq=4, Hkv=2, D=8, bs=4,
                                    lens=(1, 13, 30), scratch=3)
    assert pins.check_split_combine(c, splits=(2, 3)) <= TOL   # invisible there
    assert pins.check_partials_brute_force(c, splits=(2, 3)) > 1e-3


def test_split_partition_off_by_one_page_is_caught(monkeypatch):
    # Pages shifted one split later: the combination is unchanged (every page
    # still counted once), the partials are not.
    real = pa.split_token_ranges

    def shifted(ctx, bs, S):
        r = real(ctx, bs, S)
        if S > 1 and r[0][1] - r[0][0] > bs:
            lo0, hi0 = r[0]
            lo1, hi1 = r[1]
            r[0] = (lo0, hi0 - bs)
            r[1] = (hi0 - bs, hi1 if hi1 > lo1 else hi0)
        return r

    monkeypatch.setattr(pa, "split_token_ranges", shifted)
    c = pins.random_contiguous_case(4, B=3, Tq=1, Hq=4, Hkv=2, D=8, bs=4,
                                    lens=(9, 30, 40), scratch=0)
    assert pins.check_partials_brute_force(c, splits=(2, 3)) > 1e-3


def test_base2_lse_is_caught(monkeypatch):
    real = pa.attend

    def base2(q, K, V, scale):
        O, lse = real(q, K, V, scale)
        return O, lse / math.log(2.0)

    monkeypatch.setattr(pa, "attend", base2)
    assert pins.check_zero_keys_count() > 1e-3


def test_missing_scratch_tokens_is_caught(monkeypatch):
    real = pa.logical_kv

    def no_scratch(*a, **kw):
        kw["with_scratch"] = False
        return real(*a, **kw)

    monkeypatch.setattr(pa, "logical_kv", no_scratch)
    assert pins.check_zero_keys_count() > 1e-3


def test_wrong_fp8_bias_is_caught(monkeypatch):
    import torch
    wrong = np.array([e4m3fn.decode_code(c) * 2.0 for c in range(256)])
    monkeypatch.setattr(e4m3fn, "DECODE_TABLE", wrong)
    codes = np.arange(256, dtype=np.uint8)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    mine = e4m3fn.decode(codes)
    ok = ~np.isnan(theirs)
    assert np.abs(mine[ok] - theirs[ok]).max() > 1.0


def test_off_by_one_causal_scratch_mask_is_caught(monkeypatch):
    real = pa.visible_scratch
    monkeypatch.setattr(pa, "visible_scratch",
                        lambda t, tq, s, m: max(0, real(t, tq, s, m) - 1) if m == "causal" else s)
    c = pins.random_contiguous_case(31, B=2, Tq=2, Hq=4, Hkv=2, D=6, bs=4, lens=(5, 0), scratch=2)
    assert pins.check_causal_brute_force(c) > 1e-3
    c = pins.random_contiguous_case(34, Tq=4, Hq=8, Hkv=2, bs=4, lens=(3, 0, 31), scratch=4)
    assert pins.check_causal_against_masked_sdpa(c) > 1e-3


def test_causal_mask_on_the_wrong_side_is_caught(monkeypatch):
    # Query token t seeing the scratch tokens from its position onward.
    def suffix(t, tq, s, m):
        return s if m == "none" else max(0, min(s, s - (t + (s - tq)) ))
    monkeypatch.setattr(pa, "visible_scratch", suffix)
    c = pins.random_contiguous_case(38, Tq=3, Hq=4, Hkv=2, bs=4, lens=(0, 7, 20), scratch=5)
    assert pins.check_causal_invariants(c) > 1e-3


def test_round_half_up_encoding_is_caught(monkeypatch):
    real_vals = e4m3fn.DECODE_TABLE[:0x7F]

    def half_up(y):
        y = np.asarray(y, dtype=np.float64)
        a = np.abs(y)
        hi = np.minimum(np.searchsorted(real_vals, a, side="left"), 0x7E)
        lo = np.maximum(hi - 1, 0)
        pick = (real_vals[hi] - a) <= (a - real_vals[lo])
        mag = np.where(pick, hi, lo)
        return (mag | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)

    monkeypatch.setattr(e4m3fn, "encode", half_up)
    import test_oracle_kv_write as t
    import pytest
    with pytest.raises(AssertionError):
        t.test_encode_matches_torch_on_every_value_midpoint_and_random_value()


def test_ignored_scratch_counts_are_caught(monkeypatch):
    real = pa._seq_counts
    monkeypatch.setattr(pa, "_seq_counts",
                        lambda b, tq, n, ql, sl: (real(b, tq, n, ql, sl)[0], n))
    c = pins.random_contiguous_case(41, B=4, Tq=4, Hq=4, Hkv=2, D=6, bs=4,
                                    lens=(0, 5, 9, 2), scratch=5)
    assert pins.check_seq_counts_brute_force(c, np.array([4, 1, 0, 3]), np.array([5, 2, 3, 0]),
                                             "none") > 1e-3


def test_head_major_pages_read_with_token_major_axes_are_caught(monkeypatch):
    real = pa._token_rows

    def wrong_axes(pages, scale, row, ctx, bs, h_kv, fmt, layout="token"):
        if layout == "head":      # treat the [P, Hkv, bs, D] pool as [P, bs, Hkv, D]
            pages = np.ascontiguousarray(pages).reshape(pages.shape[0], pages.shape[2],
                                                         pages.shape[1], pages.shape[3])
            if scale is not None:
                scale = np.ascontiguousarray(scale).reshape(scale.shape[0], scale.shape[2],
                                                            scale.shape[1])
            return real(pages, scale, row, ctx, bs, h_kv, fmt, "token")
        return real(pages, scale, row, ctx, bs, h_kv, fmt, layout)

    monkeypatch.setattr(pa, "_token_rows", wrong_axes)
    import test_oracle_pins as t
    import pytest
    with pytest.raises(AssertionError):
        t.test_head_major_pool_gives_bit_identical_results(
            dict(kv_dtype="bf16", head_dim=64, block_size=4, scratch_tokens=3))


def test_truncated_f16_scales_are_caught(monkeypatch):
    from oracle import kv_write
    real = kv_write.quantise_row

    def truncating(x, scale_dtype="f32"):
        if scale_dtype != "f16":
            return real(x, scale_dtype)
        x = np.asarray(x, dtype=np.float32)
        s = np.float32(np.max(np.abs(x)) / np.float32(448.0)) if x.size else np.float32(0.0)
        s = min(s, np.float32(65504.0))
        # round toward zero to f16: drop the low 13 mantissa bits (normal range)
        bits = np.array([s], dtype=np.float32).view(np.uint32) & np.uint32(0xFFFFE000)
        s16 = np.float32(np.float16(bits.view(np.float32)[0]))
        if s16 == 0.0:
            return np.zeros(x.shape, dtype=np.uint8), np.float32(0.0)
        y = np.clip((x / s16).astype(np.float32), -448.0, 448.0)
        return e4m3fn.encode(y), s16

    monkeypatch.setattr(kv_write, "quantise_row", truncating)
    import test_oracle_kv_write as t
    import pytest
    with pytest.raises(AssertionError):
        t.test_f16_scale_quantisation_matches_the_generator()
