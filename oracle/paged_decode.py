"""Paged-KV decode attention with split-K partials, in float64 on the CPU.

TEST INFRASTRUCTURE: this is the CPU oracle that the GPU path is checked
against. Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import it. It shares no code with the HIP path and imports nothing from
it. It is deliberately plain and slow: each step follows the definition,
with no blocking, fusion or reordering beyond what the definition states.

Sources (cited by page title and section):

* "Implementing a High-Performance Custom Diffusion Attention Kernel with
  FlyDSL" (AMD ROCm blog), introduction item 1: a paged KV cache plus scratch
  storage for speculatively generated tokens; introduction item 3: the
  computation is organised as FlashAttention with split-K; "Debug
  Systematically": the log-sum-exp (LSE) is the intermediate compared between
  implementations.
* "[ROCm] Add FlyDSL paged-attention decode backend (dense + fp8) with
  benchmark" (MSLK pull request), Kernels: head-packed GQA decode (ratio
  1..16), e4m3fn KV with a symmetric per-token scale, and a split-K partial
  combine kernel; review thread: ``num_splits: int = 0`` is the per-call
  knob and custom softmax scales are supported.

Readings where the pages are silent (each is also listed in the design notes):

* q head h reads kv head h // g with g = Hq / Hkv (contiguous groups);
* the page pool is [P, bs, Hkv, D] (token-major) or, as a layout option,
  [P, Hkv, bs, D] (head-major); logical token i of sequence b lives in page
  block_table[b, i // bs], slot i % bs; scales follow the pool's order;
* scratch tokens follow the paged context, and every query token of the
  sequence sees the whole context and all scratch tokens (mask "none");
* with the causal scratch mask, query token t of Tq sees scratch token j of
  S_tok iff j <= t + (S_tok - Tq): the query tokens are the last Tq of the
  speculative tokens the scratch area holds (blog, introduction item 1) and
  each sees those up to its own position (the order among draft tokens is
  this library's reading; the pages state none);
* a sequence may have fewer query and scratch tokens than the arrays hold
  (q_lens, scratch_lens): query tokens past its count are padding rows (O = 0,
  LSE = -inf) and scratch tokens past its count do not exist;
* split s of S covers the page range [s * pps, min((s + 1) * pps, npages))
  with pps = ceil(npages / S); the scratch tokens belong to the last split;
  an empty split contributes (O_s = 0, LSE_s = -inf);
* with nothing to attend to, O = 0 and LSE = -inf;
* LSE is a natural logarithm.
"""

from __future__ import annotations

import math
from typing import List, Optional, Tuple

import numpy as np

from . import e4m3fn


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """kv head read by q head h: groups of g = Hq / Hkv consecutive q heads."""
    g = num_q_heads // num_kv_heads
    return h // g


def _token_rows(pages, scale, block_table_row, ctx: int, bs: int, h_kv: int,
                kv_format: str, kv_layout: str = "token") -> np.ndarray:
    """Logical rows [ctx, D] of one kv head, gathered page by page."""
    rows = []
    for i in range(0, ctx, bs):
        page = int(block_table_row[i // bs])
        n = min(bs, ctx - i)
        if kv_layout == "head":
            codes, sc = pages[page, h_kv, :n, :], (None if scale is None else scale[page, h_kv, :n])
        else:
            codes, sc = pages[page, :n, h_kv, :], (None if scale is None else scale[page, :n, h_kv])
        if kv_format == "fp8":
            blk = e4m3fn.dequantise(codes, sc)
        else:
            blk = np.asarray(codes, dtype=np.float64)
        rows.append(blk)
    if not rows:
        return np.zeros((0, pages.shape[-1]), dtype=np.float64)
    return np.concatenate(rows, axis=0)


def logical_kv(k_pages, v_pages, block_table, context_lens, b: int, h_kv: int,
               *, kv_format: str = "dense", k_scale=None, v_scale=None,
               scratch_k=None, scratch_v=None,
               token_range: Optional[Tuple[int, int]] = None,
               with_scratch: bool = True,
               kv_layout: str = "token") -> Tuple[np.ndarray, np.ndarray]:
    """K and V rows of sequence b, kv head h_kv, in logical order, float64.

    Rows are the paged context tokens 0..ctx_b-1 (optionally restricted to
    ``token_range``), then the scratch tokens of sequence b. fp8 rows are
    dequantised as decode(code) * scale.
    """
    assert kv_layout in ("token", "head")
    bs = k_pages.shape[2] if kv_layout == "head" else k_pages.shape[1]
    ctx = int(context_lens[b])
    lo, hi = (0, ctx) if token_range is None else token_range
    assert 0 <= lo <= hi <= ctx
    assert lo % bs == 0 or lo == hi, "non-empty ranges start on a page boundary"
    row = np.asarray(block_table[b])[lo // bs:]
    K = _token_rows(k_pages, k_scale, row, hi - lo, bs, h_kv, kv_format, kv_layout)
    V = _token_rows(v_pages, v_scale, row, hi - lo, bs, h_kv, kv_format, kv_layout)
    if with_scratch and scratch_k is not None:
        K = np.concatenate([K, np.asarray(scratch_k[b, :, h_kv, :], np.float64)])
        V = np.concatenate([V, np.asarray(scratch_v[b, :, h_kv, :], np.float64)])
    return K, V


def visible_scratch(t: int, q_tokens: int, scratch_tokens: int, scratch_mask: str) -> int:
    """Number of scratch tokens query token t sees (a prefix of them)."""
    assert scratch_mask in ("none", "causal")
    if scratch_mask == "none":
        return scratch_tokens
    return max(0, min(scratch_tokens, t + (scratch_tokens - q_tokens) + 1))


def attend(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray,
           scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of query rows [r, D] over K, V [n, D], in float64.

    scores = scale * q K^T; m = max; w = exp(scores - m); l = sum w;
    O = (w V) / l; LSE = m + ln l. With n = 0: O = 0, LSE = -inf.
    """
    r, d = q_rows.shape
    if K.shape[0] == 0:
        return np.zeros((r, V.shape[1])), np.full((r,), -np.inf)
    s = scale * (q_rows @ K.T)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    O = (w @ V) / l
    lse = (m + np.log(l))[:, 0]
    return O, lse


def _as_np(x, dtype=np.float64):
    if x is None:
        return None
    return np.asarray(x) if dtype is None else np.asarray(x, dtype=dtype)


def _prepare(q, k_pages, v_pages, block_table, context_lens, kv_format,
             k_scale, v_scale, scratch_k, scratch_v):
    assert kv_format in ("dense", "fp8")
    q = _as_np(q)
    if kv_format == "fp8":
        k_pages = np.asarray(k_pages, dtype=np.uint8)
        v_pages = np.asarray(v_pages, dtype=np.uint8)
        k_scale = _as_np(k_scale)
        v_scale = _as_np(v_scale)
        assert k_scale is not None and v_scale is not None
    else:
        k_pages = np.asarray(k_pages)
        v_pages = np.asarray(v_pages)
    return (q, k_pages, v_pages, np.asarray(block_table), np.asarray(context_lens),
            k_scale, v_scale, _as_np(scratch_k), _as_np(scratch_v))


def _seq_counts(b: int, Tq: int, n_scr: int, q_lens, scratch_lens) -> Tuple[int, int]:
    """Query tokens and scratch tokens of sequence b (clamped to the arrays)."""
    nq = Tq if q_lens is None else min(max(int(q_lens[b]), 0), Tq)
    ns = n_scr if scratch_lens is None else min(max(int(scratch_lens[b]), 0), n_scr)
    return nq, ns


def paged_attention(q, k_pages, v_pages, block_table, context_lens, scale: float,
                    *, kv_format: str = "dense", k_scale=None, v_scale=None,
                    scratch_k=None, scratch_v=None, scratch_mask: str = "none",
                    q_lens=None, scratch_lens=None,
                    kv_layout: str = "token") -> Tuple[np.ndarray, np.ndarray]:
    """Decode attention over a paged KV cache, float64.

    q [B, Tq, Hq, D]; pages [P, bs, Hkv, D]; block_table [B, W];
    context_lens [B]; scratch [B, S_tok, Hkv, D] or None.
    Query token t attends the context and its visible scratch tokens
    (``visible_scratch``); optional q_lens / scratch_lens [B] give each
    sequence fewer query and scratch tokens. Returns O [B, Tq, Hq, D] and
    LSE [B, Tq, Hq] (natural log), float64.
    """
    (q, k_pages, v_pages, block_table, context_lens, k_scale, v_scale,
     scratch_k, scratch_v) = _prepare(q, k_pages, v_pages, block_table,
                                      context_lens, kv_format, k_scale, v_scale,
                                      scratch_k, scratch_v)
    B, Tq, Hq, D = q.shape
    Hkv = k_pages.shape[1] if kv_layout == "head" else k_pages.shape[2]
    O = np.zeros((B, Tq, Hq, D))
    LSE = np.zeros((B, Tq, Hq))
    n_scr = 0 if scratch_k is None else scratch_k.shape[1]
    for b in range(B):
        ctx = int(context_lens[b])
        nq, ns = _seq_counts(b, Tq, n_scr, q_lens, scratch_lens)
        for h_kv in range(Hkv):
            K, V = logical_kv(k_pages, v_pages, block_table, context_lens, b, h_kv,
                              kv_format=kv_format, k_scale=k_scale, v_scale=v_scale,
                              scratch_k=scratch_k, scratch_v=scratch_v, kv_layout=kv_layout)
            heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == h_kv]
            for t in range(Tq):
                if t >= nq:                      # padding query token
                    O[b, t, heads, :] = 0.0
                    LSE[b, t, heads] = -np.inf
                    continue
                n = ctx + visible_scratch(t, nq, ns, scratch_mask)
                o, lse = attend(q[b, t, heads, :], K[:n], V[:n], scale)
                O[b, t, heads, :] = o
                LSE[b, t, heads] = lse
    return O, LSE


def split_token_ranges(ctx: int, block_size: int, num_splits: int) -> List[Tuple[int, int]]:
    """Token range [lo, hi) of each split of one sequence's paged context.

    npages = ceil(ctx / bs); pps = ceil(npages / S); split s covers pages
    [s * pps, min((s + 1) * pps, npages)), clipped to the context. Later
    splits may be empty. Scratch tokens are not part of these ranges: they
    belong to the last split.
    """
    assert num_splits >= 1
    npages = -(-ctx // block_size)
    pps = -(-npages // num_splits) if npages else 0
    out = []
    for s in range(num_splits):
        p0 = min(s * pps, npages)
        p1 = min((s + 1) * pps, npages)
        out.append((min(p0 * block_size, ctx), min(p1 * block_size, ctx)))
    return out


def owns_scratch(s: int, num_splits: int) -> bool:
    """Whether split s of num_splits holds the sequence's scratch tokens.

    The pages leave the placement open; the scratch tokens follow the paged
    context in logical order, so they go with the split that ends it: the
    last one. The combined result does not depend on this choice, only the
    partials do.
    """
    return s == num_splits - 1


def paged_attention_partials(q, k_pages, v_pages, block_table, context_lens,
                             scale: float, num_splits: int, *,
                             kv_format: str = "dense", k_scale=None, v_scale=None,
                             scratch_k=None, scratch_v=None, scratch_mask: str = "none",
                             q_lens=None, scratch_lens=None, kv_layout: str = "token"):
    """Per-split partials (O_s, LSE_s) of the split-K decomposition, float64.

    Returns O_part [B, Tq, Hq, S, D] (each split normalised by its own
    softmax sum) and LSE_part [B, Tq, Hq, S] (natural log; -inf for an empty
    split, whose O_s is 0).
    """
    (q, k_pages, v_pages, block_table, context_lens, k_scale, v_scale,
     scratch_k, scratch_v) = _prepare(q, k_pages, v_pages, block_table,
                                      context_lens, kv_format, k_scale, v_scale,
                                      scratch_k, scratch_v)
    B, Tq, Hq, D = q.shape
    Hkv = k_pages.shape[1] if kv_layout == "head" else k_pages.shape[2]
    bs = k_pages.shape[2] if kv_layout == "head" else k_pages.shape[1]
    S = num_splits
    O_part = np.zeros((B, Tq, Hq, S, D))
    LSE_part = np.full((B, Tq, Hq, S), -np.inf)
    n_scr = 0 if scratch_k is None else scratch_k.shape[1]
    for b in range(B):
        ranges = split_token_ranges(int(context_lens[b]), bs, S)
        nq, ns = _seq_counts(b, Tq, n_scr, q_lens, scratch_lens)
        for h_kv in range(Hkv):
            heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == h_kv]
            for s, (lo, hi) in enumerate(ranges):
                K, V = logical_kv(k_pages, v_pages, block_table, context_lens, b, h_kv,
                                  kv_format=kv_format, k_scale=k_scale,
                                  v_scale=v_scale, scratch_k=scratch_k,
                                  scratch_v=scratch_v, token_range=(lo, hi),
                                  with_scratch=owns_scratch(s, S), kv_layout=kv_layout)
                for t in range(Tq):
                    if t >= nq:                  # padding query token: (0, -inf)
                        continue
                    n = hi - lo
                    if owns_scratch(s, S):
                        n += visible_scratch(t, nq, ns, scratch_mask)
                    o, lse = attend(q[b, t, heads, :], K[:n], V[:n], scale)
                    O_part[b, t, heads, s, :] = o
                    LSE_part[b, t, heads, s] = lse
    return O_part, LSE_part


def combine_partials(O_part: np.ndarray, LSE_part: np.ndarray):
    """Merge split partials into (O, LSE), float64.

    M = max_s LSE_s; w_s = exp(LSE_s - M); O = sum_s w_s O_s / sum_s w_s;
    LSE = M + ln sum_s w_s. If every split is empty (M = -inf): O = 0 and
    LSE = -inf.
    """
    O_part = np.asarray(O_part, dtype=np.float64)
    LSE_part = np.asarray(LSE_part, dtype=np.float64)
    M = LSE_part.max(axis=-1)
    empty = np.isneginf(M)
    Msafe = np.where(empty, 0.0, M)
    w = np.where(np.isneginf(LSE_part), 0.0, np.exp(LSE_part - Msafe[..., None]))
    wsum = w.sum(axis=-1)
    den = np.where(empty, 1.0, wsum)
    O = (w[..., None] * O_part).sum(axis=-2) / den[..., None]
    O = np.where(empty[..., None], 0.0, O)
    with np.errstate(divide="ignore"):
        LSE = np.where(empty, -np.inf, Msafe + np.log(np.where(empty, 1.0, wsum)))
    return O, LSE


def lse_log2e() -> float:
    """log2(e), exposed for tests that convert between bases."""
    return 1.0 / math.log(2.0)
