"""The seeded input generator lays pages out as documented (CPU only)."""

import numpy as np
import torch

from workloads import CONFIGS, make_case, make_config_case


def test_block_tables_use_each_physical_page_once():
    case = make_case(batch=4, q_tokens=1, num_q_heads=4, num_kv_heads=2, head_dim=8,
                     block_size=16, ctx=("uniform", 1, 100), seed=5, poison=True)
    lens = case.context_lens.numpy()
    bt = case.block_table.numpy()
    used = []
    for b in range(case.batch):
        n = -(-int(lens[b]) // 16)
        used.extend(bt[b, :n].tolist())
    assert len(used) == len(set(used))
    assert all(0 <= p < case.num_pages for p in used)


def test_poison_marks_only_unread_slots():
    case = make_case(batch=3, q_tokens=1, num_q_heads=2, num_kv_heads=1, head_dim=4,
                     block_size=8, ctx=(5, 8, 17), seed=6, poison=True)
    k = case.k_pages.float()
    bt = case.block_table.numpy()
    for b, n in enumerate(case.context_lens.tolist()):
        np_ = -(-n // 8)
        for i in range(np_ * 8):
            page, slot = int(bt[b, i // 8]), i % 8
            assert torch.isnan(k[page, slot]).all().item() == (i >= n)
        # entries past the last page point at a page that is all NaN
        for p in bt[b, np_:]:
            assert torch.isnan(k[int(p)]).all()


def test_tiny_config_facts():
    case = make_config_case("tiny_gqa8")
    assert case.context_lens.tolist() == [37, 100]
    assert case.num_pages == 16 and case.table_width == 7
    assert tuple(case.q.shape) == (2, 1, 8, 128)
    assert abs(case.scale - 1 / np.sqrt(128)) < 1e-15


def test_generation_is_deterministic():
    a = make_config_case("diffusion_multitoken", batch=2)
    b = make_config_case("diffusion_multitoken", batch=2)
    assert torch.equal(a.q, b.q) and torch.equal(a.k_pages, b.k_pages)
    assert torch.equal(a.scratch_v, b.scratch_v)
    assert a.scratch_k.shape == (2, 4, 8, 128)


def test_fp8_config_has_codes_and_scales():
    case = make_config_case("fp8_mqa_d256", batch=2)
    assert case.k_pages.dtype == torch.uint8 and case.k_scale.dtype == torch.float32
    assert tuple(case.k_scale.shape) == tuple(case.k_pages.shape[:3])
    assert case.q.dtype == torch.bfloat16 and case.head_dim == 256


def test_config_table_widths():
    assert CONFIGS["long_context_splitk"].table_width == 2048
    assert CONFIGS["llama3_8b_decode"].table_width == 256
    assert CONFIGS["fp8_mqa_d256"].table_width == 512
    assert CONFIGS["diffusion_multitoken"].table_width == 512
