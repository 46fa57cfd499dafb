"""The CPU oracle pinned to things other than itself (CPU only).

Tolerances: 1e-12 where the oracle and the pin round differently (library
kernels, fsum, split combine); bit-exact where the computation is the same
sequence of float operations on the same numbers (page moves, page size).
"""

import math
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import oracle_pins as pins
from workloads import make_case

TOL = 1e-12


@pytest.mark.parametrize("seed,kw", [
    (1, dict()),
    (2, dict(Hq=8, Hkv=8, bs=1, lens=(0, 2, 9))),
    (3, dict(Hq=16, Hkv=1, Tq=1, bs=16, lens=(16, 17, 64))),
    (4, dict(Tq=4, Hq=8, Hkv=2, bs=2, lens=(3, 0, 31), scratch=4)),
    (5, dict(B=2, Hq=6, Hkv=3, D=32, bs=8, lens=(40, 1), scratch=1)),
])
def test_oracle_matches_torch_sdpa_and_logsumexp(seed, kw):
    c = pins.random_contiguous_case(seed, **kw)
    assert pins.check_against_sdpa(c) <= TOL


@pytest.mark.parametrize("seed,kw", [
    (7, dict(B=2, Tq=1, Hq=4, Hkv=2, D=4, bs=2, lens=(5, 3))),
    (8, dict(B=3, Tq=2, Hq=2, Hkv=1, D=6, bs=4, lens=(0, 9, 4), scratch=2)),
    (9, dict(B=1, Tq=1, Hq=3, Hkv=3, D=5, bs=1, lens=(7,))),
    (10, dict(B=2, Tq=1, Hq=4, Hkv=1, D=8, bs=16, lens=(16, 18))),
])
def test_oracle_matches_scalar_brute_force(seed, kw):
    c = pins.random_contiguous_case(seed, **kw)
    assert pins.check_brute_force(c) <= TOL


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_split_partials_combine_to_the_unsplit_result(seed):
    c = pins.random_contiguous_case(seed, scratch=2 if seed % 2 else 0,
                                    lens=(0, 5, 33))
    assert pins.check_split_combine(c) <= TOL


@pytest.mark.parametrize("seed,mask", [(31, "none"), (32, "none"), (33, "causal")])
def test_each_split_partial_matches_scalar_brute_force(seed, mask):
    # Every split's own (O_s, LSE_s), not only their combination: the scratch
    # tokens must sit in the last split, and every page in exactly one split.
    # Lengths include an empty context, one token, a partial last page, and
    # contexts with fewer pages than splits (empty splits).
    c = pins.random_contiguous_case(seed, B=4, Tq=2, Hq=4, Hkv=2, D=8, bs=4,
                                    lens=(0, 1, 13, 30), scratch=3)
    assert pins.check_partials_brute_force(c, scratch_mask=mask) <= TOL


def test_zero_keys_give_lse_equal_to_log_token_count():
    assert pins.check_zero_keys_count() <= TOL


def test_needle_returns_that_tokens_value():
    assert pins.check_needle() <= 1e-14


def test_identical_keys_give_mean_of_values():
    assert pins.check_identical_keys() <= TOL


def test_single_token_returns_its_value():
    assert pins.check_single_token() <= TOL


def test_gqa_equals_mha_with_repeated_kv():
    assert pins.check_gqa_equals_repeated_mha() <= TOL


def test_query_tokens_are_independent():
    assert pins.check_query_token_separability() <= TOL


def test_scratch_tokens_equal_extra_context_pages():
    assert pins.check_scratch_as_pages() <= TOL


def test_page_pool_permutation_is_bit_exact():
    assert pins.check_pool_permutation_bitexact()


def test_page_size_is_bit_exact():
    assert pins.check_page_size_bitexact()


def test_empty_context_without_scratch():
    case = make_case(batch=2, q_tokens=1, num_q_heads=4, num_kv_heads=1, head_dim=8,
                     block_size=4, ctx=(0, 3), seed=3)
    O, L = oracle.run_case(case)
    assert np.all(O[0] == 0.0) and np.all(np.isneginf(L[0]))
    assert np.all(np.isfinite(L[1]))
    Op, Lp = oracle.run_case(case, num_splits=3)
    assert np.all(Op[0] == 0.0) and np.all(np.isneginf(Lp[0]))


def test_split_ranges_follow_the_page_partition():
    # npages = 5, S = 4 -> pps = 2: pages [0,2) [2,4) [4,5) and an empty split.
    r = oracle.split_token_ranges(ctx=70, block_size=16, num_splits=4)
    assert r == [(0, 32), (32, 64), (64, 70), (70, 70)]
    assert oracle.split_token_ranges(0, 16, 3) == [(0, 0)] * 3
    r = oracle.split_token_ranges(ctx=100, block_size=16, num_splits=3)
    assert r == [(0, 48), (48, 96), (96, 100)]
    # Ranges tile the context exactly, for many shapes.
    for ctx in range(0, 90, 7):
        for S in (1, 2, 3, 5, 64):
            rr = oracle.split_token_ranges(ctx, 8, S)
            assert rr[0][0] == 0 and rr[-1][1] == ctx
            assert all(a[1] == b[0] for a, b in zip(rr, rr[1:]))


def test_all_splits_empty_combine_gives_zero_and_neg_inf():
    Op = np.zeros((1, 1, 2, 3, 4))
    Lp = np.full((1, 1, 2, 3), -np.inf)
    O, L = oracle.combine_partials(Op, Lp)
    assert np.all(O == 0.0) and np.all(np.isneginf(L))


def test_combine_weights_by_exp_lse():
    # Two splits, LSEs ln 1 and ln 3: weights 1/4 and 3/4.
    Op = np.array([[[[[1.0, 0.0], [0.0, 1.0]]]]])
    Lp = np.array([[[[0.0, math.log(3.0)]]]])
    O, L = oracle.combine_partials(Op, Lp)
    assert np.allclose(O[0, 0, 0], [0.25, 0.75], rtol=0, atol=1e-15)
    assert abs(L[0, 0, 0] - math.log(4.0)) <= 1e-15


@pytest.mark.parametrize("seed,kw", [
    (31, dict(B=2, Tq=2, Hq=4, Hkv=2, D=6, bs=4, lens=(5, 0), scratch=2)),   # S_tok = Tq
    (32, dict(B=2, Tq=3, Hq=2, Hkv=1, D=4, bs=2, lens=(0, 6), scratch=5)),   # S_tok > Tq
    (33, dict(B=2, Tq=4, Hq=2, Hkv=2, D=5, bs=1, lens=(0, 3), scratch=2)),   # S_tok < Tq
])
def test_causal_scratch_mask_matches_scalar_brute_force(seed, kw):
    c = pins.random_contiguous_case(seed, **kw)
    assert pins.check_causal_brute_force(c) <= TOL


@pytest.mark.parametrize("seed,kw", [
    (34, dict(Tq=4, Hq=8, Hkv=2, bs=4, lens=(3, 0, 31), scratch=4)),
    (35, dict(Tq=2, Hq=8, Hkv=4, bs=8, lens=(0, 12, 40), scratch=6)),
    (36, dict(Tq=4, Hq=4, Hkv=1, bs=2, lens=(0, 1, 9), scratch=2)),
])
def test_causal_scratch_mask_matches_masked_sdpa(seed, kw):
    c = pins.random_contiguous_case(seed, **kw)
    assert pins.check_causal_against_masked_sdpa(c) <= TOL


@pytest.mark.parametrize("seed", [37, 38])
def test_causal_scratch_invariants_and_split_combine(seed):
    c = pins.random_contiguous_case(seed, Tq=3, Hq=4, Hkv=2, bs=4, lens=(0, 7, 20),
                                    scratch=5)
    assert pins.check_causal_invariants(c) <= TOL
    assert pins.check_causal_split_combine(c) <= TOL


def test_visible_scratch_counts():
    # Four drafts over four scratch slots: 1, 2, 3, 4 visible; fewer slots than
    # drafts: the first drafts see none.
    assert [oracle.visible_scratch(t, 4, 4, "causal") for t in range(4)] == [1, 2, 3, 4]
    assert [oracle.visible_scratch(t, 4, 2, "causal") for t in range(4)] == [0, 0, 1, 2]
    assert [oracle.visible_scratch(t, 2, 5, "causal") for t in range(2)] == [4, 5]
    assert [oracle.visible_scratch(t, 3, 5, "none") for t in range(3)] == [5, 5, 5]


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_per_sequence_query_and_scratch_counts(mask):
    c = pins.random_contiguous_case(41, B=4, Tq=4, Hq=4, Hkv=2, D=6, bs=4,
                                    lens=(0, 5, 9, 2), scratch=5)
    q_lens = np.array([4, 1, 0, 3])
    scratch_lens = np.array([5, 2, 3, 0])
    assert pins.check_seq_counts_as_separate_problems(c, q_lens, scratch_lens, mask) <= TOL
    assert pins.check_seq_counts_brute_force(c, q_lens, scratch_lens, mask) <= TOL
    # Split partials still combine to the unsplit result.
    O, L = oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["ctx"], c["scale"],
                                  scratch_k=c["sk"], scratch_v=c["sv"], scratch_mask=mask,
                                  q_lens=q_lens, scratch_lens=scratch_lens)
    for S in (2, 3):
        Op, Lp = oracle.paged_attention_partials(
            c["q"], c["kp"], c["vp"], c["table"], c["ctx"], c["scale"], S,
            scratch_k=c["sk"], scratch_v=c["sv"], scratch_mask=mask,
            q_lens=q_lens, scratch_lens=scratch_lens)
        Oc, Lc = oracle.combine_partials(Op, Lp)
        assert pins._max_dev(Oc, Lc, O, L) <= TOL


@pytest.mark.parametrize("kw", [
    dict(kv_dtype="bf16", head_dim=64, block_size=4, scratch_tokens=3),
    dict(kv_dtype="fp8", head_dim=64, block_size=16),
])
def test_head_major_pool_gives_bit_identical_results(kw):
    """The same draws stored head-major ([P, Hkv, bs, D]) give the same
    logical K/V, hence bit-identical outputs and partials."""
    base = dict(batch=3, q_tokens=2, num_q_heads=4, num_kv_heads=2, ctx=(0, 9, 40), seed=77)
    tok = make_case(**base, **kw)
    head = make_case(**base, **kw, kv_layout="head")
    assert tuple(head.k_pages.shape) == (tok.num_pages, 2, tok.block_size, kw["head_dim"])
    O1, L1 = oracle.run_case(tok)
    O2, L2 = oracle.run_case(head)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    P1 = oracle.run_case(tok, num_splits=3)
    P2 = oracle.run_case(head, num_splits=3)
    assert np.array_equal(P1[0], P2[0]) and np.array_equal(P1[1], P2[1])


def test_f16_scale_storage_reads_as_its_f32_value():
    """A case drawn with f16 scales gives bit-identical results to the same
    codes with those scales widened to f32 storage."""
    case = make_case(batch=2, q_tokens=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                     block_size=8, ctx=(5, 33), seed=91, kv_dtype="fp8", scale_dtype="f16")
    assert case.k_scale.dtype == torch.float16 and case.scale_dtype == "f16"
    wide = replace(case, k_scale=case.k_scale.float(), v_scale=case.v_scale.float())
    O1, L1 = oracle.run_case(case)
    O2, L2 = oracle.run_case(wide)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
