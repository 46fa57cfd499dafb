"""Seeded synthetic decode batches in the paged-KV layout.

Layouts (all contiguous, row-major):

* ``q``            [B, Tq, Hq, D]        bf16 or f16
* ``k_pages``      [P, bs, Hkv, D]       bf16/f16, or uint8 e4m3fn codes
* ``v_pages``      [P, bs, Hkv, D]       same as ``k_pages``
* ``k_scale``      [P, bs, Hkv]          f32, fp8 only (one scale per token
                                         and kv head)
* ``v_scale``      [P, bs, Hkv]          f32, fp8 only
* ``block_table``  [B, W]                int32, logical page -> physical page
* ``context_lens`` [B]                   int32, paged tokens per sequence
* ``scratch_k/v``  [B, S_tok, Hkv, D]    same dtype as q, or None

The paged cache with a per-sequence block table, plus a contiguous scratch
area for speculatively generated tokens, is the cache shape described in
"Implementing a High-Performance Custom Diffusion Attention Kernel with
FlyDSL" (introduction, item 1: flexible KV-cache layouts for vLLM's TiDAR
mode). The e4m3fn codes with one symmetric scale per token are the fp8 KV
format of "[ROCm] Add FlyDSL paged-attention decode backend (dense + fp8)
with benchmark" (Kernels).

Recipe (one ``numpy.random.default_rng(seed)`` stream, PCG64):

1. context lengths: uniform integers in [lo, hi] inclusive, unless fixed;
2. page permutation: ``rng.permutation(P)``; sequence b takes the b-th
   consecutive slice of it as its block-table row;
3. Q, then K, then V, then scratch K, then scratch V: float32 N(0, 1) draws,
   rounded to bf16/f16 with round-to-nearest-even;
4. fp8: K and V (float32 draws) are quantised per (token, kv head) with
   scale = absmax / 448 over the head dimension and codes
   RNE(clamp(x / scale, -448, 448)) in OCP e4m3fn.

``poison=True`` fills every slot that the method must never read with NaN:
the tail slots of each sequence's last page, every unused page, and the
block-table entries past each sequence's last page point at a NaN page.
With ``poison=False`` those entries are -1 and unused storage is zero.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

E4M3_MAX = 448.0

_TORCH_DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class WorkloadConfig:
    """One decode workload: shapes, dtypes, context-length draw and seed."""

    name: str
    batch: int
    q_tokens: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    ctx: Tuple[int, ...] | Tuple[str, int, int]
    kv_dtype: str = "bf16"
    q_dtype: str = "bf16"
    scratch_tokens: int = 0
    seed: int = 0
    pool_pages: Optional[int] = None
    splits: Tuple[int, ...] = (0,)
    description: str = ""

    @property
    def max_context(self) -> int:
        if self.ctx and self.ctx[0] == "uniform":
            return int(self.ctx[2])
        return int(max(self.ctx))

    @property
    def table_width(self) -> int:
        return max(1, -(-self.max_context // self.block_size))

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# The five decode workloads. Each is named by what it is, with its sizes.
CONFIGS = {
    "tiny_gqa8": WorkloadConfig(
        name="tiny_gqa8", batch=2, q_tokens=1, num_q_heads=8, num_kv_heads=1,
        head_dim=128, block_size=16, ctx=(37, 100), seed=101, pool_pages=16,
        splits=(1, 3),
        description="batch 2, 8 q heads / 1 kv head, D128, bs16, ctx {37,100}, "
                    "16-page pool, scale 1/sqrt(128), splits 1 and 3"),
    "llama3_8b_decode": WorkloadConfig(
        name="llama3_8b_decode", batch=32, q_tokens=1, num_q_heads=32,
        num_kv_heads=8, head_dim=128, block_size=16, ctx=("uniform", 512, 4096),
        seed=102, splits=(0,),
        description="batch 32, 32 q / 8 kv heads, D128, bs16, ctx U[512,4096], bf16"),
    "long_context_splitk": WorkloadConfig(
        name="long_context_splitk", batch=4, q_tokens=1, num_q_heads=64,
        num_kv_heads=8, head_dim=128, block_size=64,
        ctx=("uniform", 32768, 131072), seed=103, splits=(8, 16, 32, 64),
        description="batch 4, 64 q / 8 kv heads, D128, bs64, ctx U[32768,131072], "
                    "bf16, splits 8-64"),
    "fp8_mqa_d256": WorkloadConfig(
        name="fp8_mqa_d256", batch=64, q_tokens=1, num_q_heads=16, num_kv_heads=1,
        head_dim=256, block_size=16, ctx=("uniform", 1024, 8192), kv_dtype="fp8",
        seed=104, splits=(0,),
        description="batch 64, 16 q / 1 kv head, D256, bs16, ctx U[1024,8192], "
                    "e4m3fn KV with per-token scale, bf16 Q"),
    "diffusion_multitoken": WorkloadConfig(
        name="diffusion_multitoken", batch=16, q_tokens=4, num_q_heads=32,
        num_kv_heads=8, head_dim=128, block_size=16, ctx=("uniform", 2048, 8192),
        scratch_tokens=4, seed=105, splits=(0,),
        description="batch 16 x 4 draft tokens, 32 q / 8 kv heads, D128, bs16, "
                    "ctx U[2048,8192] + 4 scratch tokens, no mask, bf16"),
}

# Shapes beyond the five, for variants of the path (measured, not headline).
VARIANT_CONFIGS = {
    "gqa32_row_groups": WorkloadConfig(
        name="gqa32_row_groups", batch=32, q_tokens=1, num_q_heads=64, num_kv_heads=2,
        head_dim=128, block_size=16, ctx=("uniform", 512, 4096), seed=106, splits=(0,),
        description="batch 32, 64 q / 2 kv heads (32 packed rows: two 16-row groups), "
                    "D128, bs16, ctx U[512,4096], bf16"),
    "gqa32_long_context": WorkloadConfig(
        name="gqa32_long_context", batch=4, q_tokens=1, num_q_heads=64, num_kv_heads=2,
        head_dim=128, block_size=64, ctx=("uniform", 32768, 131072), seed=107, splits=(0,),
        description="batch 4, 64 q / 2 kv heads (32 packed rows: two 16-row groups), "
                    "D128, bs64, ctx U[32768,131072], bf16"),
}


@dataclass
class DecodeCase:
    """Host (CPU) tensors of one decode call, in the layouts listed above."""

    q: torch.Tensor
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    block_table: torch.Tensor
    context_lens: torch.Tensor
    scale: float
    kv_dtype: str
    q_dtype: str
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None
    scratch_k: Optional[torch.Tensor] = None
    scratch_v: Optional[torch.Tensor] = None
    scratch_mask: str = "none"   # which scratch tokens each query token sees
    kv_layout: str = "token"     # pools [P, bs, Hkv, D] ("token") or [P, Hkv, bs, D] ("head")
    q_lens: Optional[torch.Tensor] = None        # [B] int32 query tokens per sequence
    scratch_lens: Optional[torch.Tensor] = None  # [B] int32 scratch tokens per sequence
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def q_tokens(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[2])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[3])

    @property
    def num_pages(self) -> int:
        return int(self.k_pages.shape[0])

    @property
    def block_size(self) -> int:
        return int(self.k_pages.shape[2 if self.kv_layout == "head" else 1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_pages.shape[1 if self.kv_layout == "head" else 2])

    @property
    def table_width(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def scratch_tokens(self) -> int:
        return 0 if self.scratch_k is None else int(self.scratch_k.shape[1])

    @property
    def scale_dtype(self) -> str:
        """Storage type of the fp8 scales ("f32" or "f16"; "f32" when dense)."""
        return "f16" if self.k_scale is not None and self.k_scale.dtype == torch.float16 else "f32"

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one decode call must read.

        Every context token and every scratch token is read once per kv head
        for K and for V; fp8 adds the two scales of each (token, kv head), 4 or
        2 bytes each as stored.
        Page tails past the context, Q, the outputs, the block table and the
        split partials are not counted.
        """
        tokens = int(self.context_lens.to(torch.int64).sum())
        hkv, d = self.num_kv_heads, self.head_dim
        elem = 1 if self.kv_dtype == "fp8" else 2
        total = tokens * hkv * d * 2 * elem
        if self.kv_dtype == "fp8":
            total += tokens * hkv * 2 * (2 if self.scale_dtype == "f16" else 4)
        if self.scratch_k is not None:
            total += self.batch * self.scratch_tokens * hkv * d * 2 * 2
        return total


def _round_to(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(x).to(_TORCH_DTYPES[dtype])


def fp8_quantise_per_token(x: torch.Tensor,
                           scale_dtype: str = "f32") -> Tuple[torch.Tensor, torch.Tensor]:
    """Quantise float32 ``x`` [..., D] to e4m3fn codes with one scale per row.

    scale = absmax / 448 over the last axis (float32); codes are
    round-to-nearest-even of clamp(x / scale, -448, 448). The clamp is
    explicit because an unclamped cast maps out-of-range values to NaN. A row
    that is all zero gets scale 0 and codes 0. With ``scale_dtype`` "f16"
    the scale is rounded to f16 first (capped at the largest finite f16) and
    that value both divides x and is returned (as float16).
    """
    x = x.to(torch.float32)
    absmax = x.abs().amax(dim=-1)
    scale = absmax / E4M3_MAX
    if scale_dtype == "f16":
        scale = scale.clamp(max=65504.0).to(torch.float16).to(torch.float32)
    else:
        assert scale_dtype == "f32"
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    y = torch.where(scale[..., None] > 0, x / safe[..., None], torch.zeros_like(x))
    y = y.clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    if scale_dtype == "f16":
        scale = scale.to(torch.float16)
    return codes, scale.contiguous()


def _context_lengths(rng: np.random.Generator, cfg_ctx, batch: int) -> np.ndarray:
    if cfg_ctx and cfg_ctx[0] == "uniform":
        lo, hi = int(cfg_ctx[1]), int(cfg_ctx[2])
        return rng.integers(lo, hi + 1, size=batch).astype(np.int64)
    lens = np.asarray(cfg_ctx, dtype=np.int64)
    assert lens.shape == (batch,), "fixed context lengths must give one per sequence"
    return lens


def make_case(
    *,
    batch: int,
    q_tokens: int,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    ctx,
    seed: int,
    kv_dtype: str = "bf16",
    q_dtype: str = "bf16",
    scratch_tokens: int = 0,
    pool_pages: Optional[int] = None,
    table_width: Optional[int] = None,
    scale: Optional[float] = None,
    poison: bool = False,
    scratch_mask: str = "none",
    kv_layout: str = "token",
    scale_dtype: str = "f32",
) -> DecodeCase:
    """Draw one seeded decode batch (see the module docstring for the recipe).

    ``ctx`` is either a sequence of fixed lengths, or ("uniform", lo, hi).
    ``pool_pages`` defaults to the pages the contexts need (plus one NaN page
    when ``poison``); ``table_width`` defaults to the pages of the longest
    possible context.
    """
    assert num_q_heads % num_kv_heads == 0
    assert kv_dtype in ("bf16", "f16", "fp8") and q_dtype in ("bf16", "f16")
    if kv_dtype != "fp8":
        assert kv_dtype == q_dtype, "dense KV uses the query dtype"
    rng = np.random.default_rng(seed)
    lens = _context_lengths(rng, ctx, batch)
    npages = -(-lens // block_size)
    need = int(npages.sum())
    if table_width is None:
        if ctx and ctx[0] == "uniform":
            table_width = max(1, -(-int(ctx[2]) // block_size))
        else:
            table_width = max(1, int(npages.max()) if batch else 1)
    assert int(npages.max(initial=0)) <= table_width
    if pool_pages is None:
        pool_pages = need + (1 if poison else 0)
    assert pool_pages >= need, "the page pool must hold every context page"
    perm = rng.permutation(pool_pages)
    used = perm[:need]
    spare = perm[need:]

    table = np.full((batch, table_width), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        n = int(npages[b])
        table[b, :n] = used[off:off + n]
        off += n

    shape_q = (batch, q_tokens, num_q_heads, head_dim)
    shape_kv = (pool_pages, block_size, num_kv_heads, head_dim)
    q = _round_to(rng.standard_normal(shape_q, dtype=np.float32), q_dtype)
    k32 = torch.from_numpy(rng.standard_normal(shape_kv, dtype=np.float32))
    v32 = torch.from_numpy(rng.standard_normal(shape_kv, dtype=np.float32))
    k_scale = v_scale = None
    if kv_dtype == "fp8":
        k_pages, k_scale = fp8_quantise_per_token(k32, scale_dtype)
        v_pages, v_scale = fp8_quantise_per_token(v32, scale_dtype)
    else:
        k_pages = k32.to(_TORCH_DTYPES[kv_dtype])
        v_pages = v32.to(_TORCH_DTYPES[kv_dtype])
    del k32, v32

    scratch_k = scratch_v = None
    if scratch_tokens:
        shape_s = (batch, scratch_tokens, num_kv_heads, head_dim)
        scratch_k = _round_to(rng.standard_normal(shape_s, dtype=np.float32), q_dtype)
        scratch_v = _round_to(rng.standard_normal(shape_s, dtype=np.float32), q_dtype)

    if poison:
        _poison_unread(k_pages, v_pages, k_scale, v_scale, table, lens, spare,
                       block_size, kv_dtype)
    else:
        if spare.size:
            k_pages[torch.from_numpy(spare)] = 0
            v_pages[torch.from_numpy(spare)] = 0

    if kv_layout == "head":
        # Same draws, pages reordered to [P, Hkv, bs, D] (scales [P, Hkv, bs]).
        k_pages = k_pages.transpose(1, 2).contiguous()
        v_pages = v_pages.transpose(1, 2).contiguous()
        if k_scale is not None:
            k_scale = k_scale.transpose(1, 2).contiguous()
            v_scale = v_scale.transpose(1, 2).contiguous()
    else:
        assert kv_layout == "token"
    return DecodeCase(
        q=q, k_pages=k_pages, v_pages=v_pages,
        block_table=torch.from_numpy(table),
        context_lens=torch.from_numpy(lens.astype(np.int32)),
        scale=(1.0 / math.sqrt(head_dim)) if scale is None else float(scale),
        kv_dtype=kv_dtype, q_dtype=q_dtype,
        k_scale=k_scale, v_scale=v_scale,
        scratch_k=scratch_k, scratch_v=scratch_v, scratch_mask=scratch_mask,
        kv_layout=kv_layout, meta={"seed": seed, "poison": poison},
    )


def _poison_unread(k_pages, v_pages, k_scale, v_scale, table, lens, spare,
                   block_size, kv_dtype):
    """Fill every slot the method must not read with NaN (see module doc)."""
    nan_code = 0x7F
    fill = nan_code if kv_dtype == "fp8" else float("nan")
    if spare.size:
        idx = torch.from_numpy(spare)
        k_pages[idx] = fill
        v_pages[idx] = fill
        if k_scale is not None:
            k_scale[idx] = float("nan")
            v_scale[idx] = float("nan")
        poison_page = int(spare[0])
    else:
        poison_page = -1
    for b in range(table.shape[0]):
        n = -(-int(lens[b]) // block_size)
        tail = int(lens[b]) - (n - 1) * block_size if n else 0
        if n and tail < block_size:
            last = int(table[b, n - 1])
            k_pages[last, tail:] = fill
            v_pages[last, tail:] = fill
            if k_scale is not None:
                k_scale[last, tail:] = float("nan")
                v_scale[last, tail:] = float("nan")
        if poison_page >= 0:
            table[b, n:] = poison_page


def make_config_case(cfg: WorkloadConfig | str, *, poison: bool = False,
                     seed: Optional[int] = None,
                     batch: Optional[int] = None, kv_layout: str = "token",
                     scale_dtype: str = "f32") -> DecodeCase:
    """Draw the named workload (optionally with a reduced batch or new seed,
    or with head-major pages)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg] if cfg in CONFIGS else VARIANT_CONFIGS[cfg]
    pool = cfg.pool_pages  # None: sized to the context (+1 NaN page if poisoned)
    b = cfg.batch if batch is None else batch
    ctx = cfg.ctx
    if b != cfg.batch and ctx and ctx[0] != "uniform":
        ctx = tuple(ctx[:b])
    return make_case(
        batch=b, q_tokens=cfg.q_tokens, num_q_heads=cfg.num_q_heads,
        num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim,
        block_size=cfg.block_size, ctx=ctx,
        seed=cfg.seed if seed is None else seed, kv_dtype=cfg.kv_dtype,
        q_dtype=cfg.q_dtype, scratch_tokens=cfg.scratch_tokens,
        pool_pages=pool, table_width=cfg.table_width, scale=cfg.scale,
        poison=poison, kv_layout=kv_layout,
        scale_dtype=scale_dtype if cfg.kv_dtype == "fp8" else "f32",
    )


def repage(case: DecodeCase, *, block_size: int, seed: int,
           pool_extra: int = 0) -> DecodeCase:
    """Re-lay the same logical K/V into pages of another size.

    Logical token i of sequence b moves to a fresh random page assignment
    with ``block_size`` tokens per page. Token values, order and scales are
    unchanged, so the attention result must not change. Used to test that
    the page size is invisible to the method. Token-major pools only.
    """
    if case.kv_layout != "token":
        raise ValueError("repage expects a token-major pool")
    rng = np.random.default_rng(seed)
    B, bs0 = case.batch, case.block_size
    lens = case.context_lens.to(torch.int64).numpy()
    npages = -(-lens // block_size)
    need = int(npages.sum())
    P = need + pool_extra
    perm = rng.permutation(P)
    W = max(1, int(npages.max(initial=0)))
    table = np.full((B, W), -1, dtype=np.int32)
    hkv, d = case.num_kv_heads, case.head_dim
    kp = torch.zeros((P, block_size, hkv, d), dtype=case.k_pages.dtype)
    vp = torch.zeros_like(kp)
    ks = vs = None
    if case.k_scale is not None:
        ks = torch.zeros((P, block_size, hkv), dtype=torch.float32)
        vs = torch.zeros_like(ks)
    off = 0
    bt0 = case.block_table.numpy()
    for b in range(B):
        n = int(npages[b])
        table[b, :n] = perm[off:off + n]
        off += n
        for i in range(int(lens[b])):
            src_page, src_slot = int(bt0[b, i // bs0]), i % bs0
            dst_page, dst_slot = int(table[b, i // block_size]), i % block_size
            kp[dst_page, dst_slot] = case.k_pages[src_page, src_slot]
            vp[dst_page, dst_slot] = case.v_pages[src_page, src_slot]
            if ks is not None:
                ks[dst_page, dst_slot] = case.k_scale[src_page, src_slot]
                vs[dst_page, dst_slot] = case.v_scale[src_page, src_slot]
    return replace(case, k_pages=kp, v_pages=vp, k_scale=ks, v_scale=vs,
                   block_table=torch.from_numpy(table))


def permute_pool(case: DecodeCase, seed: int) -> DecodeCase:
    """Move every physical page to a new slot and remap the block table.

    The page index is the leading dimension in both pool layouts.
    """
    rng = np.random.default_rng(seed)
    P = case.num_pages
    new_of_old = rng.permutation(P)
    old_of_new = np.argsort(new_of_old)
    idx = torch.from_numpy(old_of_new)
    bt = case.block_table.numpy().copy()
    mask = bt >= 0
    bt[mask] = new_of_old[bt[mask]]
    return replace(
        case,
        k_pages=case.k_pages[idx].contiguous(),
        v_pages=case.v_pages[idx].contiguous(),
        k_scale=None if case.k_scale is None else case.k_scale[idx].contiguous(),
        v_scale=None if case.v_scale is None else case.v_scale[idx].contiguous(),
        block_table=torch.from_numpy(bt),
    )


def sequence_slices(sizes: Sequence[int]):
    """Offsets of consecutive slices of the given sizes (helper for tests)."""
    out, off = [], 0
    for s in sizes:
        out.append((off, off + s))
        off += s
    return out
