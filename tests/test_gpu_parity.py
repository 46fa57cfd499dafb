"""HIP path vs the CPU oracle, through the C ABI (GPU only).

Sizes: every workload's shapes at a batch the oracle finishes in seconds
(several tiles and a ragged tail per sequence), then the full workloads,
every output row and every split partial (the long-context one at each of
its split counts). Inputs are NaN-poisoned
wherever the method must not read (page tails, unused pages, block-table
entries past the context), so a stray read shows up as a non-finite output.
"""

import functools
import math
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (compare, decoder_for, oracle_rows, partials_from_workspace, run_gpu,
                         to_device)
from workloads import CONFIGS, make_case, make_config_case, permute_pool

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def _full_case(name):
    # Full size, NaN-poisoned like the small cases: page tails, the spare page
    # and block-table entries past each context hold NaN at the real widths.
    return make_config_case(name, poison=True)


@functools.lru_cache(maxsize=1)
def _full_oracle(name):
    return oracle.run_case(_full_case(name))


def _kind(case):
    return "fp8" if case.kv_dtype == "fp8" else "dense"


def _check_full(case, num_splits, what):
    dec = decoder_for(case, max_num_splits=max(64, num_splits))
    out, lse, ws, S = run_gpu(case, num_splits, dec=dec, keep_workspace=True)
    O, L = oracle.run_case(case)
    what = f"{what} S={S}"
    summary = compare(out, lse, O, L, _kind(case), what=what)
    if S > 1:
        Op_ref, Lp_ref = oracle.run_case(case, num_splits=S)
        Op, Lp = partials_from_workspace(ws, dec, case.batch, case.q_tokens, case.num_q_heads,
                                         S, case.head_dim)
        B, Tq, Hq, _, D = Op_ref.shape
        compare(Op.permute(0, 1, 2, 3, 4).reshape(B, Tq, Hq * S, D),
                Lp.reshape(B, Tq, Hq * S), Op_ref.reshape(B, Tq, Hq * S, D),
                Lp_ref.reshape(B, Tq, Hq * S), _kind(case), what=f"{what} partials")
    dec.close()
    return summary, S


@pytest.mark.parametrize("splits", [1, 3, 0])
def test_tiny_gqa8(splits):
    case = make_config_case("tiny_gqa8", poison=True)
    print(f"tiny_gqa8 splits={splits}", flush=True)
    _check_full(case, splits, "tiny_gqa8")


@pytest.mark.parametrize("name,batch,splits", [
    ("llama3_8b_decode", 5, 0),
    ("llama3_8b_decode", 3, 4),
    ("long_context_splitk", 1, 8),
    ("fp8_mqa_d256", 6, 0),
    ("fp8_mqa_d256", 3, 5),
    ("diffusion_multitoken", 3, 0),
    ("diffusion_multitoken", 2, 3),
])
def test_workload_shapes_small_batch(name, batch, splits):
    case = make_config_case(name, batch=batch, poison=True)
    print(f"{name} batch={batch} splits={splits} ctx={case.context_lens.tolist()}", flush=True)
    _check_full(case, splits, name)


@pytest.mark.parametrize("name,splits", [
    ("llama3_8b_decode", 0),
    ("fp8_mqa_d256", 0),
    ("diffusion_multitoken", 0),
    ("long_context_splitk", 0),
    ("long_context_splitk", 8),
    ("long_context_splitk", 16),
    ("long_context_splitk", 32),
    ("long_context_splitk", 64),
])
def test_full_workload(name, splits):
    """Every output row and every split partial of the full workload against
    the oracle, with the inputs poisoned where nothing may be read."""
    case = _full_case(name)
    print(f"{name} full batch={case.batch} splits={splits} poisoned", flush=True)
    dec = decoder_for(case, max_num_splits=max(64, splits))
    out, lse, ws, S = run_gpu(case, splits, dec=dec, keep_workspace=True)
    O, L = _full_oracle(name)
    compare(out, lse, O, L, _kind(case), what=f"{name} full S={S}")
    if S > 1:
        Op_ref, Lp_ref = oracle.run_case(case, num_splits=S)
        Op, Lp = partials_from_workspace(ws, dec, case.batch, case.q_tokens, case.num_q_heads,
                                         S, case.head_dim)
        B, Tq, Hq, _, D = Op_ref.shape
        compare(Op.reshape(B, Tq, Hq * S, D), Lp.reshape(B, Tq, Hq * S),
                Op_ref.reshape(B, Tq, Hq * S, D), Lp_ref.reshape(B, Tq, Hq * S), _kind(case),
                what=f"{name} full S={S} partials")
    dec.close()


def test_long_context_split_sweep_is_consistent():
    case = make_config_case("long_context_splitk", batch=2)
    outs = {}
    for S in CONFIGS["long_context_splitk"].splits:
        out, lse, _, _ = run_gpu(case, S)
        outs[S] = (out.float().cpu(), lse.cpu())
    ref = oracle_rows(case, [(0, 2), (1, 4)])
    for S, (out, lse) in outs.items():
        for (b, hk), (O, L) in ref.items():
            compare(out[b, :, hk * 8:(hk + 1) * 8], lse[b, :, hk * 8:(hk + 1) * 8], O, L,
                    what=f"long_context split {S} b={b} hk={hk}")


@pytest.mark.parametrize("bs,lens,splits", [
    (1, (1, 31, 32, 33), 0),
    (2, (0, 5, 64, 65), 2),
    (4, (17, 3, 100), 7),
    (8, (250, 1), 3),
    (32, (32, 31, 95, 96, 97), 0),
    (64, (1, 63, 64, 65, 200), 2),
    (128, (129, 5), 1),
    (256, (300,), 2),
])
def test_page_sizes_and_ragged_lengths(bs, lens, splits):
    case = make_case(batch=len(lens), q_tokens=1, num_q_heads=8, num_kv_heads=2,
                     head_dim=128, block_size=bs, ctx=lens, seed=700 + bs, poison=True)
    _check_full(case, splits, f"bs={bs} lens={lens}")


@pytest.mark.parametrize("D,kv,q_dtype,g,tq", [
    (64, "bf16", "bf16", 4, 1),
    (256, "bf16", "bf16", 2, 2),
    (128, "f16", "f16", 8, 2),
    (128, "fp8", "bf16", 4, 1),
    (64, "fp8", "f16", 16, 1),
    (256, "fp8", "f16", 1, 3),
    (128, "bf16", "bf16", 1, 1),
    (128, "bf16", "bf16", 16, 1),
])
def test_dtypes_head_dims_and_groups(D, kv, q_dtype, g, tq):
    hkv = 2
    case = make_case(batch=3, q_tokens=tq, num_q_heads=g * hkv, num_kv_heads=hkv,
                     head_dim=D, block_size=16, ctx=(7, 130, 300), seed=800 + D + g,
                     kv_dtype=kv, q_dtype=q_dtype, poison=True)
    for S in (1, 4, 0):
        _check_full(case, S, f"D={D} kv={kv} q={q_dtype} g={g} tq={tq}")


@pytest.mark.parametrize("stok,lens", [(1, (0, 9, 40)), (4, (0, 1, 33)), (16, (5, 64, 0)),
                                       (64, (3, 100, 17))])
def test_scratch_tokens(stok, lens):
    case = make_case(batch=len(lens), q_tokens=4, num_q_heads=16, num_kv_heads=4,
                     head_dim=128, block_size=16, ctx=lens, seed=900 + stok,
                     scratch_tokens=stok, poison=True)
    for S in (1, 2, 5, 0):
        _check_full(case, S, f"scratch={stok}")


def test_batch_beyond_the_ranking_limit():
    """1100 sequences: more than the kernel ranks by length (1024), so the
    items keep the natural sequence order; the results must not change."""
    rng = np.random.default_rng(5)
    lens = tuple(int(x) for x in rng.integers(0, 70, size=1100))
    case = make_case(batch=len(lens), q_tokens=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
                     block_size=16, ctx=lens, seed=1201, poison=True)
    for S in (1, 3):
        _check_full(case, S, "B=1100")


@pytest.mark.parametrize("batch,D", [(12, 128), (40, 128), (64, 128), (200, 64), (64, 256),
                                     (700, 64)])
def test_length_ranking_with_many_ties(batch, D):
    """Batches whose context lengths repeat (ties are ranked by sequence
    index), including empty ones, at sizes that take either ranking path
    (one thread per sequence; from 64 sequences, comparisons spread over the
    workgroup and counted in LDS): every sequence is processed exactly once."""
    rng = np.random.default_rng(batch)
    lens = tuple(int(x) for x in rng.choice([0, 1, 17, 33, 64, 100], size=batch))
    case = make_case(batch=batch, q_tokens=1, num_q_heads=4, num_kv_heads=2, head_dim=D,
                     block_size=16, ctx=lens, seed=1300 + batch, poison=True)
    for S in (1, 3):
        _check_full(case, S, f"B={batch} D={D} tied lengths")


def test_block_table_rows_with_padding():
    """Block-table rows wider than the pages they name (row stride > width),
    the padding holding a NaN page's index: only the first ceil(ctx/bs)
    entries of a row may be read."""
    case = make_case(batch=3, q_tokens=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                     block_size=16, ctx=(40, 300, 17), seed=1202, poison=True)
    W = case.block_table.shape[1]
    wide = torch.full((case.batch, W + 37), int(case.block_table.max()), dtype=torch.int32)
    wide[:, :W] = case.block_table
    view = wide[:, :W]
    assert view.stride(0) == W + 37
    dec = decoder_for(case)
    dev = to_device(case)
    dev["block_table"] = wide.cuda()[:, :W]
    O, L = oracle.run_case(case)
    for S in (1, 4):
        out, lse = dec(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                       dev["context_lens"], softmax_scale=case.scale, num_splits=S)
        torch.cuda.synchronize()
        compare(out, lse, O, L, "dense", what=f"padded block table S={S}")
    dec.close()


@pytest.mark.parametrize("stok,tq,g,lens", [
    (4, 4, 4, (0, 1, 33, 200)),      # one scratch slot per draft token
    (6, 2, 8, (0, 17, 64)),          # more scratch tokens than queries
    (2, 4, 2, (0, 5, 48)),           # fewer: the first drafts of an empty context see nothing
    (40, 3, 4, (0, 3, 100)),         # two scratch tiles
])
def test_causal_scratch_mask(stok, tq, g, lens):
    case = make_case(batch=len(lens), q_tokens=tq, num_q_heads=2 * g, num_kv_heads=2,
                     head_dim=128, block_size=16, ctx=lens, seed=1300 + stok + tq,
                     scratch_tokens=stok, poison=True, scratch_mask="causal")
    for S in (1, 2, 5, 0):
        _check_full(case, S, f"causal stok={stok} tq={tq} g={g}")


def test_causal_mask_multitoken_workload():
    """The full multi-token workload with the causal scratch mask, every row."""
    case = replace(_full_case("diffusion_multitoken"), scratch_mask="causal")
    out, lse, _, S = run_gpu(case, 0)
    O, L = oracle.run_case(case)
    compare(out, lse, O, L, what=f"causal multitoken full S={S}")


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_per_sequence_query_and_scratch_counts(mask):
    """Sequences with fewer draft (query) tokens and scratch tokens than the
    arrays hold; padding query rows must come out as (0, -inf)."""
    lens = (0, 7, 33, 130, 16, 64)
    case = make_case(batch=len(lens), q_tokens=4, num_q_heads=16, num_kv_heads=4,
                     head_dim=128, block_size=16, ctx=lens, seed=1500, scratch_tokens=6,
                     poison=True, scratch_mask=mask)
    case.q_lens = torch.tensor([4, 1, 0, 3, 2, 4], dtype=torch.int32)
    case.scratch_lens = torch.tensor([6, 2, 3, 0, 6, 1], dtype=torch.int32)
    for S in (1, 3, 0):
        _check_full(case, S, f"per-sequence counts mask={mask}")


@pytest.mark.parametrize("kw", [
    dict(head_dim=128, block_size=16, kv_dtype="bf16", num_kv_heads=2, num_q_heads=8),
    dict(head_dim=128, block_size=64, kv_dtype="bf16", num_kv_heads=8, num_q_heads=64),
    dict(head_dim=256, block_size=16, kv_dtype="fp8", num_kv_heads=1, num_q_heads=16),
    dict(head_dim=64, block_size=4, kv_dtype="f16", q_dtype="f16", num_kv_heads=2,
         num_q_heads=4),
    dict(head_dim=128, block_size=32, kv_dtype="bf16", num_kv_heads=4, num_q_heads=16,
         q_tokens=4, scratch_tokens=4, scratch_mask="causal"),
])
def test_head_major_page_layout(kw):
    kw = dict(kw)
    case = make_case(batch=4, q_tokens=kw.pop("q_tokens", 1), ctx=(0, 17, 130, 301),
                     seed=1600, poison=True, kv_layout="head", **kw)
    for S in (1, 3, 0):
        _check_full(case, S, f"head-major {kw}")


@pytest.mark.parametrize("kw", [
    dict(head_dim=256, block_size=16, num_kv_heads=1, num_q_heads=16),
    dict(head_dim=128, block_size=32, num_kv_heads=4, num_q_heads=16, kv_layout="head"),
    dict(head_dim=64, block_size=8, num_kv_heads=2, num_q_heads=8, q_dtype="f16"),
])
def test_fp8_with_f16_scales(kw):
    case = make_case(batch=4, q_tokens=1, ctx=(1, 40, 129, 700), seed=1700, poison=True,
                     kv_dtype="fp8", scale_dtype="f16", **kw)
    assert case.k_scale.dtype == torch.float16
    for S in (1, 4, 0):
        _check_full(case, S, f"f16 scales {kw}")


@pytest.mark.parametrize("kw", [
    dict(num_q_heads=64, num_kv_heads=2, head_dim=128, block_size=16),        # GQA 32: 2 groups
    dict(num_q_heads=40, num_kv_heads=1, head_dim=128, block_size=32),        # 16 + 16 + 8 rows
    dict(num_q_heads=48, num_kv_heads=1, head_dim=256, block_size=16, kv_dtype="fp8"),
    dict(num_q_heads=20, num_kv_heads=1, head_dim=64, block_size=8, kv_dtype="fp8"),
    dict(num_q_heads=32, num_kv_heads=4, head_dim=128, block_size=16, q_tokens=4,
         scratch_tokens=4, scratch_mask="causal"),                             # 8 x 4 = 32 rows
    dict(num_q_heads=128, num_kv_heads=1, head_dim=64, block_size=16),        # 8 groups
    dict(num_q_heads=48, num_kv_heads=2, head_dim=128, block_size=16, kv_layout="head",
         q_dtype="f16", kv_dtype="f16"),                                      # 16 + 8 rows
    dict(num_q_heads=32, num_kv_heads=1, head_dim=128, block_size=16, kv_dtype="fp8"),
    dict(num_q_heads=64, num_kv_heads=1, head_dim=128, block_size=64, kv_dtype="fp8",
         scale_dtype="f16", kv_layout="head"),                                # 4 groups, 2 passes
    dict(num_q_heads=36, num_kv_heads=3, head_dim=64, block_size=32, q_dtype="f16",
         kv_dtype="f16"),                                                     # 12 rows: one group
])
def test_row_groups_beyond_16_packed_rows(kw):
    kw = dict(kw)
    case = make_case(batch=3, q_tokens=kw.pop("q_tokens", 1), ctx=(5, 77, 300), seed=1800,
                     poison=True, **kw)
    for S in (1, 3, 0):
        _check_full(case, S, f"row groups {kw}")


@pytest.mark.parametrize("splits", [0, 8])
def test_row_groups_long_context_full(splits):
    """GQA 32 at long context (two row groups read together): every row and
    split partial of the full, poisoned workload."""
    case = make_config_case("gqa32_long_context", poison=True)
    print(f"gqa32_long_context full splits={splits}", flush=True)
    _check_full(case, splits, "gqa32 long context")


def test_row_groups_with_per_sequence_query_counts():
    """Padding query rows inside the second row group come out as (0, -inf)."""
    case = make_case(batch=4, q_tokens=4, num_q_heads=48, num_kv_heads=4, head_dim=128,
                     block_size=16, ctx=(9, 70, 200, 33), seed=1810, scratch_tokens=3,
                     poison=True, scratch_mask="causal")
    case.q_lens = torch.tensor([4, 2, 3, 1], dtype=torch.int32)
    case.scratch_lens = torch.tensor([3, 1, 0, 3], dtype=torch.int32)
    for S in (1, 2, 0):
        _check_full(case, S, "row groups, per-sequence counts")


def test_maximum_split_count_and_page_size():
    """S = 256 (the largest allowed) over one 131072-token context in
    256-token pages, and S = 256 over short contexts (most splits empty)."""
    case = make_case(batch=1, q_tokens=1, num_q_heads=8, num_kv_heads=1, head_dim=128,
                     block_size=256, ctx=(131072,), seed=1900, poison=True)
    dec = decoder_for(case, max_num_splits=256)
    out, lse, _, S = run_gpu(case, 256, dec=dec)
    assert S == 256
    O, L = oracle.run_case(case)
    compare(out, lse, O, L, "dense", what="S=256 over 131072 tokens")
    dec.close()
    short = make_case(batch=3, q_tokens=1, num_q_heads=8, num_kv_heads=1, head_dim=128,
                      block_size=16, ctx=(1, 100, 0), seed=1901, poison=True)
    _check_full(short, 256, "S=256 over short contexts")


def test_largest_row_count_with_most_scratch_tokens():
    """128 packed rows (16 draft tokens x GQA 8: eight row groups) with 64
    scratch tokens under the causal mask."""
    case = make_case(batch=2, q_tokens=16, num_q_heads=16, num_kv_heads=2, head_dim=64,
                     block_size=16, ctx=(0, 45), seed=1910, scratch_tokens=64, poison=True,
                     scratch_mask="causal")
    for S in (1, 2):
        _check_full(case, S, "128 rows, 64 scratch tokens")


@pytest.mark.parametrize("kw", [
    dict(head_dim=128, block_size=16, num_kv_heads=2, num_q_heads=8),            # UPG path
    dict(head_dim=256, block_size=2, num_kv_heads=1, num_q_heads=4, kv_layout="head",
         scale_dtype="f16"),                                                       # generic path
])
def test_fp8_multi_token_with_per_sequence_query_counts(kw):
    """fp8 KV with 4 query tokens per sequence, some of them padding."""
    case = make_case(batch=5, q_tokens=4, ctx=(0, 1, 30, 77, 513), seed=1950, poison=True,
                     kv_dtype="fp8", **kw)
    case.q_lens = torch.tensor([4, 0, 1, 3, 2], dtype=torch.int32)
    for S in (1, 3, 0):
        _check_full(case, S, f"fp8 multi-token counts {kw}")


def test_unranked_batch_with_fp8_and_head_major_pages():
    """A batch past the longest-first ranking limit (natural order) on the
    fp8 path with head-major pages and f16 scales."""
    rng = np.random.default_rng(1960)
    lens = tuple(int(x) for x in rng.integers(0, 40, size=1030))
    case = make_case(batch=1030, q_tokens=1, num_q_heads=8, num_kv_heads=2, head_dim=64,
                     block_size=16, ctx=lens, seed=1961, kv_dtype="fp8", kv_layout="head",
                     scale_dtype="f16")
    for S in (1, 2):
        _check_full(case, S, "unranked fp8 head-major")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_out_of_range_context_lengths_are_clamped(kv):
    """A context length past the block-table width (or negative) is clamped
    to [0, max_blocks_per_seq * block_size]: no read past the table row, and
    the result is that of the clamped length."""
    case = make_case(batch=4, q_tokens=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                     block_size=16, ctx=(64, 0, 40, 64), seed=1970, table_width=4,
                     kv_dtype=kv, poison=True)
    dev = to_device(case)
    bad = torch.tensor([10 ** 6, -5, 40, 2 ** 31 - 1], dtype=torch.int32).cuda()
    O, L = oracle.run_case(case)
    for S in (1, 3):
        dec = decoder_for(case, max_num_splits=8)
        out, lse = dec(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], bad,
                       softmax_scale=case.scale, num_splits=S, k_scale=dev["k_scale"],
                       v_scale=dev["v_scale"])
        torch.cuda.synchronize()
        compare(out, lse, O, L, _kind(case), what=f"clamped ctx S={S}")
        dec.close()
    # Past the ranking limit the kernel reads the lengths directly: same clamp.
    lens = [32 if i % 97 == 0 else i % 20 for i in range(1030)]
    big = make_case(batch=1030, q_tokens=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                    block_size=16, ctx=tuple(lens), seed=1971, table_width=2, kv_dtype=kv)
    dev = to_device(big)
    bad = big.context_lens.clone()
    bad[::97] = 1000
    bad[1] = -3
    ref = big.context_lens.clone()
    ref[1] = 0
    Ob, Lb = oracle.run_case(replace(big, context_lens=ref))
    dec = decoder_for(big, max_num_splits=8)
    out, lse = dec(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], bad.cuda(),
                   softmax_scale=big.scale, num_splits=2, k_scale=dev["k_scale"],
                   v_scale=dev["v_scale"])
    torch.cuda.synchronize()
    compare(out, lse, Ob, Lb, _kind(big), what="clamped ctx, unranked batch")
    dec.close()


@pytest.mark.parametrize("kv,bs", [("bf16", 16), ("fp8", 16), ("bf16", 4)])
def test_out_of_range_block_table_entries_are_clamped(kv, bs):
    """With the pool size given, a block-table entry outside [0, P) reads page
    0 or P - 1 (the entry clamped) instead of memory outside the pools."""
    case = make_case(batch=3, q_tokens=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                     block_size=bs, ctx=(50, 97, 130), seed=1980, kv_dtype=kv)
    bt = case.block_table.clone()
    bt[0, 1] = 10 ** 6
    bt[1, 0] = -7
    bt[2, 2] = case.num_pages
    clipped = replace(case, block_table=torch.clamp(bt, 0, case.num_pages - 1))
    # Entries past each context stay -1 in the reference: they are never read.
    clipped.block_table[case.block_table < 0] = -1
    O, L = oracle.run_case(clipped)
    dev = to_device(case)
    for S in (1, 3):
        dec = decoder_for(case, max_num_splits=8)
        out, lse = dec(dev["q"], dev["k_pages"], dev["v_pages"], bt.cuda(), dev["context_lens"],
                       softmax_scale=case.scale, num_splits=S, k_scale=dev["k_scale"],
                       v_scale=dev["v_scale"])
        torch.cuda.synchronize()
        compare(out, lse, O, L, _kind(case), what=f"clamped block table S={S}")
        dec.close()


def test_empty_contexts_give_zero_and_neg_inf():
    case = make_case(batch=3, q_tokens=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
                     block_size=16, ctx=(0, 0, 5), seed=31, pool_pages=3, poison=True)
    for S in (1, 3):
        out, lse, _, _ = run_gpu(case, S)
        assert torch.all(out[:2].float() == 0)
        assert torch.all(torch.isneginf(lse[:2]))
        assert torch.all(torch.isfinite(lse[2]))


def test_needle_is_bit_exact():
    """K = 0 except one token whose key scores 40 for every head of its group."""
    D, bs, n = 128, 16, 149
    torch.manual_seed(3)
    for star in sorted({0, 1, 15, 16, 31, 32, 33, 63, 64, 127, 128, 147, 148}):
        case = make_case(batch=1, q_tokens=1, num_q_heads=4, num_kv_heads=1, head_dim=D,
                         block_size=bs, ctx=(n,), seed=1000 + star, poison=True)
        qdir = torch.randn(D).to(torch.bfloat16)
        case.q[:] = qdir
        bt = case.block_table
        page, slot = int(bt[0, star // bs]), star % bs
        case.k_pages.zero_()
        kq = qdir.double()
        key = (kq * (40.0 / (case.scale * float(kq @ kq)))).to(torch.bfloat16)
        case.k_pages[page, slot, 0] = key
        want = case.v_pages[page, slot, 0].clone()
        for S in (1, 4):
            out, lse, _, _ = run_gpu(case, S)
            got = out[0, 0].cpu()
            assert torch.equal(got, want.expand_as(got)), f"needle at {star}, S={S}"


@pytest.mark.parametrize("slope", [0.02, 0.3, -0.3])
def test_scores_that_rise_or_fall_along_the_context(slope):
    """Score of token t = slope * t: the running maximum rises by about 1 (base 2)
    every 9 tiles, by about 14 every tile, or never after the first token."""
    D, bs, lens = 128, 16, (700, 333)
    case = make_case(batch=2, q_tokens=1, num_q_heads=4, num_kv_heads=1, head_dim=D,
                     block_size=bs, ctx=lens, seed=61, poison=True)
    q = torch.zeros(D)
    q[0] = 1.0
    case.q[:] = q.to(case.q.dtype)
    case.scale = 1.0
    for b, n in enumerate(lens):
        t = torch.arange(n)
        pages = case.block_table[b, t // bs].long()
        case.k_pages[pages, t % bs, 0, 0] = (slope * t.double()).to(case.k_pages.dtype)
    for S in (1, 4):
        _check_full(case, S, f"ramp slope={slope}")


def test_zero_keys_count_tokens_exactly():
    """K = 0: LSE = ln(ctx + scratch) to well within half the gap to ln(n +- 1)."""
    lens = (1, 15, 16, 17, 333, 1000)
    case = make_case(batch=len(lens), q_tokens=2, num_q_heads=8, num_kv_heads=2,
                     head_dim=128, block_size=16, ctx=lens, seed=77, scratch_tokens=3,
                     poison=False)
    case.k_pages.zero_()
    case.scratch_k.zero_()
    for S in (1, 3, 8):
        _, lse, _, _ = run_gpu(case, S)
        for b, n in enumerate(lens):
            tot = n + 3
            tol = 0.5 * math.log((tot + 1) / tot)
            err = (lse[b].double().cpu() - math.log(tot)).abs().max().item()
            assert err < min(tol, 1e-4), (b, n, S, err)


def test_page_pool_permutation_is_bit_identical():
    case = make_config_case("llama3_8b_decode", batch=4, poison=True)
    out1, lse1, _, _ = run_gpu(case, 0)
    out2, lse2, _, _ = run_gpu(permute_pool(case, 5), 0)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_runs_are_deterministic():
    case = make_config_case("fp8_mqa_d256", batch=8, poison=True)
    dev = to_device(case)
    dec = decoder_for(case)
    a = run_gpu(case, 0, dec=dec, dev=dev)
    b = run_gpu(case, 0, dec=dec, dev=dev)
    dec.close()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("q_dtype", ["bf16", "f16"])
def test_fp8_value_path_decodes_every_code_exactly(q_dtype):
    """A needle selects one token whose V row holds every finite e4m3fn code.

    With v_scale = 1 the output must equal the decoded codes exactly (every
    e4m3fn value is a bf16 and an f16 value), so any decode error shows bit
    for bit.
    """
    D, bs, n = 256, 16, 40
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)] + [0x00, 0x80]
    case = make_case(batch=1, q_tokens=1, num_q_heads=2, num_kv_heads=1, head_dim=D,
                     block_size=bs, ctx=(n,), seed=55, kv_dtype="fp8", q_dtype=q_dtype,
                     poison=True)
    star = 21
    page, slot = int(case.block_table[0, star // bs]), star % bs
    qdir = torch.zeros(D, dtype=case.q.dtype)
    qdir[0] = 1.0
    case.q[:] = qdir
    case.k_pages.zero_()
    case.k_pages[page, slot, 0, 0] = 0x7E   # code of 448
    case.k_scale[page, slot, 0] = 1.0
    case.v_pages[page, slot, 0] = torch.tensor(codes, dtype=torch.uint8)
    case.v_scale[page, slot, 0] = 1.0
    case.scale = 1.0
    for S in (1, 2):
        out, _, _, _ = run_gpu(case, S)
        want = torch.from_numpy(oracle.e4m3fn.decode(np.array(codes, dtype=np.uint8))).float()
        got = out[0, 0].float().cpu()
        assert torch.equal(got, want.expand_as(got)), (got - want).abs().max()


@pytest.mark.parametrize("splits", [0, 3])
def test_graph_replay_matches_eager_bit_for_bit(splits):
    case = make_config_case("diffusion_multitoken", batch=4, poison=True)
    dev = to_device(case)
    dec = decoder_for(case)
    S = dec.num_splits(case.batch, splits)
    ws = dec.alloc_workspace(case.batch, splits)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:3], dtype=torch.float32, device="cuda")
    args = dec.make_args(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                         dev["context_lens"], out, softmax_scale=case.scale, lse=lse,
                         num_splits=splits, scratch_k=dev["scratch_k"],
                         scratch_v=dev["scratch_v"])
    dec.launch(args, ws)
    torch.cuda.synchronize()
    eager_out, eager_lse = out.clone(), lse.clone()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            dec.launch(args, ws)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        out.fill_(7.0)
        lse.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out) and torch.equal(lse, eager_lse), f"replay {i}"
        _ = (dev["q"].float() * 2).sum().item()  # unrelated eager work between replays
    # Inputs rewritten in place are seen by the next replay.
    dev["q"].mul_(-1)
    g.replay()
    torch.cuda.synchronize()
    dec.launch(args, ws)
    torch.cuda.synchronize()
    out2 = out.clone()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and not torch.equal(out2, eager_out)
    assert S >= 1 and (splits == 0 or S == splits)
    dec.close()
