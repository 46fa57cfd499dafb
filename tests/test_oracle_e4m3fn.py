"""The oracle's e4m3fn decoder and fp8 dequantisation (CPU only)."""

import math

import numpy as np
import torch

import oracle
from oracle import e4m3fn
from workloads import fp8_quantise_per_token, make_case


def test_all_256_codes_match_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    mine = e4m3fn.decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_mine, nan_theirs = np.isnan(mine), np.isnan(theirs)
    assert np.array_equal(nan_mine, nan_theirs)
    assert np.array_equal(mine[~nan_mine], theirs[~nan_theirs])
    # Signed zeros agree too.
    assert np.array_equal(np.signbit(mine[~nan_mine]), np.signbit(theirs[~nan_theirs]))


def test_format_landmarks():
    d = e4m3fn.decode_code
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0          # largest finite
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))     # the only NaNs
    assert d(0x08) == 2.0 ** -6                            # smallest normal
    assert d(0x01) == 2.0 ** -9                            # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9                        # largest subnormal
    assert d(0x38) == 1.0 and d(0xB8) == -1.0              # exponent = bias
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert np.count_nonzero(np.isnan(e4m3fn.DECODE_TABLE)) == 2   # no infinities


def test_quantisation_round_trip_error_is_half_an_ulp_of_the_grid():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(257, 64, generator=g) * torch.logspace(-3, 3, 257)[:, None]
    x[3] = 0.0
    codes, scale = fp8_quantise_per_token(x)
    deq = e4m3fn.dequantise(codes.numpy(), scale.numpy().astype(np.float64))
    xs = x.double().numpy()
    y = np.abs(xs) / np.where(scale.numpy() > 0, scale.numpy(), 1.0)[:, None]
    # Grid spacing of e4m3fn at |y|: 2^(floor(log2 y) - 3) for normals, 2^-9 below 2^-6.
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    spacing = 2.0 ** (e - 3)
    bound = 0.5 * spacing * scale.numpy().astype(np.float64)[:, None]
    # x / scale is itself rounded to float32 before the cast: allow that too.
    bound = bound + np.abs(xs) * 2.0 ** -23
    assert np.all(np.abs(deq - xs) <= bound)
    assert np.all(deq[3] == 0.0) and scale[3] == 0.0


def test_fp8_oracle_equals_dense_oracle_on_dequantised_pages():
    case = make_case(batch=3, q_tokens=2, num_q_heads=4, num_kv_heads=2, head_dim=32,
                     block_size=4, ctx=(1, 9, 22), seed=41, kv_dtype="fp8",
                     poison=True)
    O8, L8 = oracle.run_case(case)
    kd = e4m3fn.dequantise(case.k_pages.numpy(), case.k_scale.numpy())
    vd = e4m3fn.dequantise(case.v_pages.numpy(), case.v_scale.numpy())
    O, L = oracle.paged_attention(case.q.double().numpy(), kd, vd,
                                  case.block_table.numpy(), case.context_lens.numpy(),
                                  case.scale)
    assert np.array_equal(O8, O) and np.array_equal(L8, L)
    assert np.all(np.isfinite(O8))
