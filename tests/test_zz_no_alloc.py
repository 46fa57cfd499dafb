"""paged_decode_run_noalloc: run + reduce with the library-owned workspace
(GPU only), checked against paged_decode_run + paged_decode_reduce with a
caller workspace on the same inputs.

Both go through the same kernels, so the outputs must agree bit for bit; the
oracle bound is checked as well. Two calls in a row, the second with a
smaller input (fewer sequences, a different split count), show that the
second call is not affected by the partials the first left in the array.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import compare, decoder_for, to_device
from paged_kv_attention_14_amd import _lib
from workloads import make_case, make_config_case

pytestmark = pytest.mark.gpu


def _with_workspace(dec, case, dev, splits):
    out = torch.full_like(dev["q"], float("nan"))
    lse = torch.full(dev["q"].shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    dec(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], dev["context_lens"],
        softmax_scale=case.scale, num_splits=splits, k_scale=dev["k_scale"],
        v_scale=dev["v_scale"], scratch_k=dev["scratch_k"], scratch_v=dev["scratch_v"],
        out=out, lse=lse, q_lens=dev["q_lens"], scratch_lens=dev["scratch_lens"])
    torch.cuda.synchronize()
    return out, lse


def _noalloc(dec, case, dev, splits):
    out = torch.full_like(dev["q"], float("nan"))
    lse = torch.full(dev["q"].shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    args = dec.make_args(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                         dev["context_lens"], out, softmax_scale=case.scale, lse=lse,
                         num_splits=splits, k_scale=dev["k_scale"], v_scale=dev["v_scale"],
                         scratch_k=dev["scratch_k"], scratch_v=dev["scratch_v"],
                         q_lens=dev["q_lens"], scratch_lens=dev["scratch_lens"])
    stream = torch.cuda.current_stream().cuda_stream
    _lib.check(_lib.paged_decode_run_noalloc(dec.handle, args, stream))
    torch.cuda.synchronize()
    return out, lse


def _same(a, b, what):
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), f"{what}: out differs"
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)), f"{what}: lse differs"


@pytest.mark.parametrize("name,batches,splits", [
    ("llama3_8b_decode", (32, 7), (0, 3)),
    ("fp8_mqa_d256", (64, 5), (0, 8)),
    ("diffusion_multitoken", (16, 3), (0, 2)),
    ("long_context_splitk", (4, 1), (32, 64)),
])
def test_noalloc_matches_caller_workspace_twice(name, batches, splits):
    for i, (B, S) in enumerate(zip(batches, splits)):
        case = make_config_case(name, batch=B, poison=True)
        print(f"noalloc {name} call {i} batch={B} splits={S}", flush=True)
        dec = decoder_for(case)
        dev = to_device(case)
        want = _with_workspace(dec, case, dev, S)
        got = _noalloc(dec, case, dev, S)
        _same(got, want, f"{name} call {i}")
        if i == 1 or B <= 8:
            O, L = oracle.run_case(case)
            compare(got[0], got[1], O, L, "fp8" if case.kv_dtype == "fp8" else "dense",
                    what=f"{name} call {i} vs oracle")
        dec.close()


def test_noalloc_second_smaller_call_same_handle():
    """One handle, two calls: a large split count first, then a smaller batch
    with fewer splits and shorter contexts; then S = 1 (no workspace)."""
    big = make_case(batch=6, q_tokens=2, num_q_heads=16, num_kv_heads=4, head_dim=128,
                    block_size=16, ctx=(900, 17, 0, 350, 64, 1000), seed=9101, poison=True,
                    table_width=64)
    small = make_case(batch=2, q_tokens=2, num_q_heads=16, num_kv_heads=4, head_dim=128,
                      block_size=16, ctx=(33, 5), seed=9102, poison=True, table_width=64)
    dec = decoder_for(big, max_batch=6)
    for case, S in ((big, 16), (small, 3), (small, 1)):
        dev = to_device(case)
        want = _with_workspace(dec, case, dev, S)
        got = _noalloc(dec, case, dev, S)
        _same(got, want, f"batch {case.batch} S={S}")
        O, L = oracle.run_case(case)
        compare(got[0], got[1], O, L, what=f"noalloc batch {case.batch} S={S}")
    dec.close()


def test_noalloc_rejects_a_workspace_beyond_its_maximum():
    """Rejected on the host before any launch, with the output untouched."""
    case = make_case(batch=64, q_tokens=4, num_q_heads=32, num_kv_heads=8, head_dim=256,
                     block_size=16, ctx=(16,) * 64, seed=9103, table_width=4)
    dec = decoder_for(case, max_num_splits=8)
    need = dec.workspace_size(64, 8)
    assert need > _lib.NOALLOC_WORKSPACE_BYTES
    assert dec.workspace_size(64, 1) == 0
    dev = to_device(case)
    out = torch.full_like(dev["q"], 7.0)
    args = dec.make_args(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                         dev["context_lens"], out, softmax_scale=case.scale, num_splits=8)
    st = _lib.paged_decode_run_noalloc(dec.handle, args, 0)
    assert st == _lib.PD_ERR_WORKSPACE_TOO_SMALL
    assert "maximum" in _lib.last_error()
    torch.cuda.synchronize()
    assert torch.all(out.float() == 7.0)
    # Within the maximum at S = 1 (no workspace at all), the call runs.
    args.num_splits = 1
    _lib.check(_lib.paged_decode_run_noalloc(dec.handle, args, 0))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    dec.close()
