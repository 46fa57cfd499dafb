"""C ABI argument checks on the GPU machine: status codes, and nothing launched.

Every call here is rejected on the host before any kernel starts, so the
output buffer keeps its sentinel value.
"""

import ctypes

import pytest
import torch

from paged_kv_attention_14_amd import _lib
from paged_kv_attention_14_amd.decode import DecodeConfig, PagedDecoder
from workloads import make_case

pytestmark = pytest.mark.gpu


def _cfg(**kw):
    base = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, q_tokens=1,
                scratch_tokens=0, q_dtype="bf16", kv_dtype="bf16", max_batch=4,
                max_blocks_per_seq=8, max_num_splits=8)
    base.update(kw)
    return DecodeConfig(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), _lib.PD_ERR_UNSUPPORTED),
    (dict(block_size=24), _lib.PD_ERR_UNSUPPORTED),
    (dict(num_kv_heads=3), _lib.PD_ERR_INVALID_ARG),
    (dict(num_q_heads=256, num_kv_heads=1), _lib.PD_ERR_UNSUPPORTED),  # 256 packed rows
    (dict(q_tokens=17, num_q_heads=8, num_kv_heads=1), _lib.PD_ERR_UNSUPPORTED),  # 136
    (dict(kv_dtype="fp8", scratch_tokens=2), _lib.PD_ERR_UNSUPPORTED),
    (dict(q_dtype="bf16", kv_dtype="f16"), _lib.PD_ERR_UNSUPPORTED),
    (dict(max_num_splits=0), _lib.PD_ERR_INVALID_ARG),
    (dict(max_batch=0), _lib.PD_ERR_INVALID_ARG),
    (dict(max_num_splits=257), _lib.PD_ERR_INVALID_ARG),
])
def test_create_rejects_bad_configs(kw, status):
    with pytest.raises(_lib.PagedDecodeError) as e:
        PagedDecoder(_cfg(**kw))
    assert e.value.status == status
    assert _lib.last_error()


def test_create_rejects_unknown_scratch_mask():
    c = _cfg().to_c()
    c.scratch_mask = 2
    with pytest.raises(_lib.PagedDecodeError) as e:
        _lib.paged_decode_create(c)
    assert e.value.status == _lib.PD_ERR_INVALID_ARG


def test_create_rejects_unknown_kv_layout():
    c = _cfg().to_c()
    c.kv_layout = 2
    with pytest.raises(_lib.PagedDecodeError) as e:
        _lib.paged_decode_create(c)
    assert e.value.status == _lib.PD_ERR_INVALID_ARG


def test_create_rejects_bad_scale_dtypes():
    c = _cfg(kv_dtype="fp8").to_c()
    c.scale_dtype = 2
    with pytest.raises(_lib.PagedDecodeError) as e:
        _lib.paged_decode_create(c)
    assert e.value.status == _lib.PD_ERR_INVALID_ARG
    with pytest.raises(_lib.PagedDecodeError) as e:        # f16 scales need an fp8 cache
        PagedDecoder(_cfg(scale_dtype="f16"))
    assert e.value.status == _lib.PD_ERR_INVALID_ARG


def _setup(kv="bf16", scratch=0):
    case = make_case(batch=2, q_tokens=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                     block_size=16, ctx=(20, 100), seed=1, kv_dtype=kv,
                     scratch_tokens=scratch, table_width=8)
    dec = PagedDecoder(_cfg(kv_dtype=kv, scratch_tokens=scratch))
    d = {k: (None if v is None else v.cuda()) for k, v in dict(
        q=case.q, k=case.k_pages, v=case.v_pages, bt=case.block_table,
        ctx=case.context_lens, ks=case.k_scale, vs=case.v_scale, sk=case.scratch_k,
        sv=case.scratch_v).items()}
    out = torch.full_like(d["q"], 3.0)
    return case, dec, d, out


def _args(dec, case, d, out, **over):
    a = dec.make_args(d["q"], d["k"], d["v"], d["bt"], d["ctx"], out,
                      softmax_scale=case.scale, k_scale=d["ks"], v_scale=d["vs"],
                      scratch_k=d["sk"], scratch_v=d["sv"], num_splits=over.pop("num_splits", 1))
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("q", None, _lib.PD_ERR_INVALID_ARG),
    ("block_table", None, _lib.PD_ERR_INVALID_ARG),
    ("context_lens", None, _lib.PD_ERR_INVALID_ARG),
    ("out", None, _lib.PD_ERR_INVALID_ARG),
    ("batch", 5, _lib.PD_ERR_INVALID_ARG),
    ("batch", -1, _lib.PD_ERR_INVALID_ARG),
    ("num_splits", 9, _lib.PD_ERR_INVALID_ARG),
    ("num_splits", -2, _lib.PD_ERR_INVALID_ARG),
    ("block_table_stride", 4, _lib.PD_ERR_INVALID_ARG),
    ("softmax_scale", float("nan"), _lib.PD_ERR_INVALID_ARG),
    ("num_pages", -1, _lib.PD_ERR_INVALID_ARG),
])
def test_run_rejects_bad_args_without_launching(field, value, status):
    case, dec, d, out = _setup()
    a = _args(dec, case, d, out)
    setattr(a, field, value)
    st = _lib.paged_decode_run(dec.handle, a, 0, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == status, _lib.last_error()
    assert torch.all(out.float() == 3.0)
    dec.close()


def test_fp8_without_scales_and_misaligned_q():
    case, dec, d, out = _setup(kv="fp8")
    a = _args(dec, case, d, out, k_scale=None)
    assert _lib.paged_decode_run(dec.handle, a, 0, 0, 0) == _lib.PD_ERR_INVALID_ARG
    a = _args(dec, case, d, out)
    a.q = d["q"].data_ptr() + 2
    assert _lib.paged_decode_run(dec.handle, a, 0, 0, 0) == _lib.PD_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(out.float() == 3.0)
    dec.close()


def test_workspace_too_small_is_reported():
    case, dec, d, out = _setup()
    need = dec.workspace_size(2, 4)
    assert need > 0 and dec.workspace_size(2, 1) == 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    a = _args(dec, case, d, out, num_splits=4)
    st = _lib.paged_decode_run(dec.handle, a, ws.data_ptr(), need - 1, 0)
    assert st == _lib.PD_ERR_WORKSPACE_TOO_SMALL
    st = _lib.paged_decode_reduce(dec.handle, a, 0, 0, 0)
    assert st == _lib.PD_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(out.float() == 3.0)
    dec.close()


def test_misaligned_workspace_is_rejected_by_run_and_reduce():
    case, dec, d, out = _setup()
    need = dec.workspace_size(2, 4)
    ws = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    a = _args(dec, case, d, out, num_splits=4)
    base = ws.data_ptr()
    assert base % 256 == 0
    st = _lib.paged_decode_run(dec.handle, a, base + 16, need, 0)
    assert st == _lib.PD_ERR_INVALID_ARG
    st = _lib.paged_decode_reduce(dec.handle, a, base + 16, need, 0)
    assert st == _lib.PD_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(out.float() == 3.0)
    dec.close()


def test_scratch_pointer_rules():
    case, dec, d, out = _setup(scratch=2)
    a = _args(dec, case, d, out, scratch_v=None)
    assert _lib.paged_decode_run(dec.handle, a, 0, 0, 0) == _lib.PD_ERR_INVALID_ARG
    dec.close()
    case, dec, d, out = _setup()
    a = _args(dec, case, d, out)
    a.scratch_k = d["q"].data_ptr()
    assert _lib.paged_decode_run(dec.handle, a, 0, 0, 0) == _lib.PD_ERR_INVALID_ARG
    dec.close()


def test_split_resolution_is_pure_and_bounded():
    dec = PagedDecoder(_cfg(max_blocks_per_seq=4096, max_num_splits=64, max_batch=64))
    a = dec.num_splits(4, 0)
    assert a == dec.num_splits(4, 0) and 1 <= a <= 64
    assert dec.num_splits(4, 7) == 7
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert dec.workspace_size(4, 1) == 0
    assert dec.workspace_size(4, 3) == r256(r256(4 * 8 * 3 * 128 * 4) + 4 * 8 * 3 * 4)
    assert dec.workspace_offsets(4, 3) == (0, r256(4 * 8 * 3 * 128 * 4))
    with pytest.raises(_lib.PagedDecodeError):
        dec.num_splits(4, 65)
    dec.close()
    # Short maximum context: at least two tiles per wave per split.
    dec = PagedDecoder(_cfg(max_blocks_per_seq=2, max_num_splits=64, max_batch=64))
    assert dec.num_splits(1, 0) == 1
    dec.close()


def test_batch_zero_is_a_no_op():
    case, dec, d, out = _setup()
    a = _args(dec, case, d, out, batch=0)
    assert _lib.paged_decode_run(dec.handle, a, 0, 0, 0) == _lib.PD_OK
    assert _lib.paged_decode_reduce(dec.handle, a, 0, 0, 0) == _lib.PD_OK
    torch.cuda.synchronize()
    assert torch.all(out.float() == 3.0)
    dec.close()


def test_binding_rejects_strided_tensors():
    case, dec, d, out = _setup()
    qs = torch.empty(d["q"].shape[0], d["q"].shape[1], d["q"].shape[2], 2 * d["q"].shape[3],
                     dtype=d["q"].dtype, device="cuda")[..., ::2]
    with pytest.raises(ValueError):
        dec.make_args(qs, d["k"], d["v"], d["bt"], d["ctx"], out, softmax_scale=case.scale)
    with pytest.raises(ValueError):
        dec.make_args(d["q"], d["k"], d["v"], d["bt"].t(), d["ctx"], out, softmax_scale=case.scale)
    with pytest.raises(ValueError):
        dec.make_args(d["q"], d["k"], d["v"], d["bt"].long(), d["ctx"], out,
                      softmax_scale=case.scale)
    dec.close()
