"""Shared helpers of the GPU tests: run the HIP path, compare with the oracle.

Tolerance (floating point), fixed here and applied element by element:

* output O: |O_gpu - O_ref| <= 1e-2 (bf16/f16 KV) or 3e-2 (fp8 KV, the
  oracle using the same dequantised codes) plus half a unit in the last
  place of the output type at |O_ref| (the final rounding to bf16/f16,
  which alone is 0.0156 for outputs between 4 and 8 in bf16), and for every
  (b, t, h) row the normwise error ||O_gpu - O_ref||_2 / ||O_ref||_2 <= 2e-2;
* LSE: the same rows are -inf, and |LSE_gpu - LSE_ref| <= 1e-3 elsewhere;
* split partials (float32 in the workspace): the same bounds.
The kernel rounds P to the 16-bit MFMA type (relative error 2^-9 for bf16)
and the output to bf16/f16 (2^-9 relative); scores and sums are float32.
Those errors sit two orders of magnitude below the bounds at every workload
here, so the bounds catch a missing token or page long before rounding
reaches them (the needle and zero-key tests check indexing exactly).
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from paged_kv_attention_14_amd import DecodeConfig, PagedDecoder

ATOL = {"dense": 1e-2, "fp8": 3e-2}
# Significand bits (with the implicit one) of the output types.
_SIG_BITS = {torch.bfloat16: 8, torch.float16: 11, torch.float32: 24}


def half_ulp(ref, dtype):
    """Half a unit in the last place of `dtype` at |ref| (normal range)."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - _SIG_BITS[dtype]), 0.0)
ROW_REL = 2e-2
LSE_ATOL = 1e-3


def to_device(case, device="cuda"):
    def mv(t):
        return None if t is None else t.to(device)
    return {
        "q": mv(case.q), "k_pages": mv(case.k_pages), "v_pages": mv(case.v_pages),
        "block_table": mv(case.block_table), "context_lens": mv(case.context_lens),
        "k_scale": mv(case.k_scale), "v_scale": mv(case.v_scale),
        "scratch_k": mv(case.scratch_k), "scratch_v": mv(case.scratch_v),
        "q_lens": mv(case.q_lens), "scratch_lens": mv(case.scratch_lens),
    }


def decoder_for(case, max_num_splits=64, max_batch=None):
    return PagedDecoder(DecodeConfig(
        num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
        head_dim=case.head_dim, block_size=case.block_size, q_tokens=case.q_tokens,
        scratch_tokens=case.scratch_tokens, q_dtype=case.q_dtype,
        kv_dtype=case.kv_dtype, max_batch=max_batch or max(1, case.batch),
        max_blocks_per_seq=case.table_width, max_num_splits=max_num_splits,
        scratch_mask=case.scratch_mask, kv_layout=case.kv_layout,
        scale_dtype=case.scale_dtype))


def run_gpu(case, num_splits=0, dec=None, dev=None, keep_workspace=False):
    """Run run + reduce through the C ABI. Returns (out, lse, workspace, S)."""
    own = dec is None
    dec = dec or decoder_for(case, max_num_splits=max(64, num_splits))
    dev = dev or to_device(case)
    S = dec.num_splits(case.batch, num_splits)
    ws = dec.alloc_workspace(case.batch, num_splits)
    out, lse = dec(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                   dev["context_lens"], softmax_scale=case.scale, num_splits=num_splits,
                   k_scale=dev["k_scale"], v_scale=dev["v_scale"],
                   scratch_k=dev["scratch_k"], scratch_v=dev["scratch_v"], workspace=ws,
                   q_lens=dev["q_lens"], scratch_lens=dev["scratch_lens"])
    torch.cuda.synchronize()
    if own:
        dec.close()
    return out, lse, (ws if keep_workspace else None), S


def partials_from_workspace(ws, dec, B, Tq, Hq, S, D):
    """View the workspace as (O_part [B,Tq,Hq,S,D], LSE_part [B,Tq,Hq,S]) float32."""
    o_off, l_off = dec.workspace_offsets(B, S)
    n = B * Tq * Hq * S
    raw = ws.view(torch.uint8)
    o = raw[o_off: o_off + n * D * 4].view(torch.float32).reshape(B, Tq, Hq, S, D)
    l = raw[l_off: l_off + n * 4].view(torch.float32).reshape(B, Tq, Hq, S)
    return o, l


def compare(o_gpu, lse_gpu, O_ref, L_ref, kind="dense", what=""):
    """Assert the tolerance above; returns the error summary."""
    o = o_gpu.detach().float().cpu().double().numpy()
    assert o.shape == O_ref.shape, (o.shape, O_ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - O_ref)
    max_abs = float(err.max(initial=0.0))
    # Error left after allowing the output type's own rounding of O_ref.
    excess = err - half_ulp(O_ref, o_gpu.dtype)
    max_excess = float(excess.max(initial=0.0))
    num = np.sqrt((err ** 2).sum(axis=-1))
    den = np.sqrt((O_ref ** 2).sum(axis=-1))
    zero = den == 0
    row_rel = np.where(zero, num, num / np.where(zero, 1.0, den))
    worst_row = float(row_rel.max(initial=0.0))
    summary = {"max_abs": max_abs, "max_abs_beyond_rounding": max_excess,
               "worst_row_rel": worst_row}
    assert max_excess <= ATOL[kind], (
        f"{what}: max abs {max_abs} exceeds {ATOL[kind]} + half an ulp of {o_gpu.dtype}")
    assert worst_row <= ROW_REL, f"{what}: row normwise {worst_row} > {ROW_REL}"
    if lse_gpu is not None:
        l = lse_gpu.detach().float().cpu().double().numpy()
        fin = np.isfinite(L_ref)
        assert np.array_equal(np.isfinite(l), fin), f"{what}: LSE -inf pattern differs"
        assert np.all(np.isneginf(l[~fin])), f"{what}: empty rows must be -inf"
        lerr = float(np.abs(l[fin] - L_ref[fin]).max(initial=0.0))
        summary["lse_max_abs"] = lerr
        assert lerr <= LSE_ATOL, f"{what}: LSE err {lerr} > {LSE_ATOL}"
    return summary


def oracle_rows(case, pairs):
    """Oracle (O, LSE) for selected (b, h_kv) pairs only, via the oracle's own steps.

    Returns dicts keyed by (b, h_kv): O [Tq, g, D], LSE [Tq, g].
    """
    fp8 = case.kv_dtype == "fp8"
    kp = case.k_pages.numpy() if fp8 else case.k_pages.float().numpy()
    vp = case.v_pages.numpy() if fp8 else case.v_pages.float().numpy()
    ks = None if case.k_scale is None else case.k_scale.numpy()
    vs = None if case.v_scale is None else case.v_scale.numpy()
    sk = None if case.scratch_k is None else case.scratch_k.double().numpy()
    sv = None if case.scratch_v is None else case.scratch_v.double().numpy()
    q = case.q.double().numpy()
    bt = case.block_table.numpy()
    ctx = case.context_lens.numpy().astype(np.int64)
    g = case.num_q_heads // case.num_kv_heads
    res = {}
    for b, hk in pairs:
        K, V = oracle.logical_kv(kp, vp, bt, ctx, b, hk, kv_format="fp8" if fp8 else "dense",
                                 k_scale=ks, v_scale=vs, scratch_k=sk, scratch_v=sv,
                                 kv_layout=case.kv_layout)
        Os, Ls = [], []
        n_ctx = int(ctx[b])
        nq = case.q_tokens if case.q_lens is None else int(case.q_lens[b])
        ns = case.scratch_tokens if case.scratch_lens is None else int(case.scratch_lens[b])
        for t in range(case.q_tokens):
            if t >= nq:
                Os.append(np.zeros((g, case.head_dim)))
                Ls.append(np.full((g,), -np.inf))
                continue
            n = n_ctx + oracle.visible_scratch(t, nq, ns, case.scratch_mask)
            o, l = oracle.attend(q[b, t, hk * g:(hk + 1) * g, :], K[:n], V[:n], case.scale)
            Os.append(o)
            Ls.append(l)
        res[(b, hk)] = (np.stack(Os), np.stack(Ls))
    return res
