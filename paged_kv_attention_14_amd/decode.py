"""Torch-facing wrapper over the C ABI: device tensors in, device tensors out.

Torch supplies device memory (inputs, outputs, the split workspace) and the
current HIP stream; the library does all of the computation. Shapes and
layouts are those of include/paged_decode.h.
"""

from __future__ import annotations

import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _lib

_TORCH_TO_CODE = {torch.bfloat16: "bf16", torch.float16: "f16"}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dense(name: str, t: Optional[torch.Tensor]) -> None:
    """The C ABI takes packed arrays: reject strided views before launch."""
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (the C ABI takes packed arrays)")


_TORCH_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16}
# An e4m3fn cache is read as bytes: torch's own fp8 type or its uint8 view.
_FP8_POOL_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _expect(name: str, t: Optional[torch.Tensor], *, shape=None, min_shape=None, dtype=None,
            dtypes=None, device=None, required: bool = True, packed: bool = True) -> None:
    """Raise ValueError unless tensor ``t`` has this shape, dtype and device.

    ``shape`` must match exactly; ``min_shape`` fixes the rank and bounds every
    dimension from below (None = any size).
    """
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_shape is not None:
        if t.dim() != len(min_shape) or any(m is not None and n < m
                                            for n, m in zip(t.shape, min_shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected at least "
                             f"{tuple('*' if m is None else m for m in min_shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if packed:
        _dense(name, t)


def _pool_shapes(cfg: "DecodeConfig", k_pages: torch.Tensor, device):
    """Check the two page pools and return (P, expected scale shape)."""
    fp8 = cfg.kv_dtype == "fp8"
    _expect("k_pages", k_pages, min_shape=(None, None, None, None),
            dtypes=_FP8_POOL_DTYPES if fp8 else (_TORCH_DTYPE[cfg.kv_dtype],), device=device)
    P = int(k_pages.shape[0])
    if cfg.kv_layout == "head":
        shape = (P, cfg.num_kv_heads, cfg.block_size, cfg.head_dim)
        scale_shape = (P, cfg.num_kv_heads, cfg.block_size)
    else:
        shape = (P, cfg.block_size, cfg.num_kv_heads, cfg.head_dim)
        scale_shape = (P, cfg.block_size, cfg.num_kv_heads)
    if tuple(k_pages.shape) != shape:
        raise ValueError(f"k_pages has shape {tuple(k_pages.shape)}, expected {shape} "
                         f"({cfg.kv_layout}-major pages of the handle)")
    if P > 0x7FFFFFFF:
        raise ValueError(f"{P} pages exceed the 32-bit page count")
    return P, shape, scale_shape


def validate_decode_tensors(cfg: "DecodeConfig", device, q, k_pages, v_pages, block_table,
                            context_lens, out, *, lse=None, k_scale=None, v_scale=None,
                            scratch_k=None, scratch_v=None, q_lens=None,
                            scratch_lens=None) -> None:
    """Check every tensor of a decode call against the handle's config and
    each other before any pointer reaches the library.

    The C ABI sees only pointers, so a tensor that is too small, of the wrong
    type or on another device would make the kernels read or write outside
    it; every such mismatch raises ValueError here instead.
    """
    qdt = _TORCH_DTYPE[cfg.q_dtype]
    _expect("q", q, min_shape=(0, cfg.q_tokens, cfg.num_q_heads, cfg.head_dim), dtype=qdt,
            device=device)
    B = int(q.shape[0])
    want_q = (B, cfg.q_tokens, cfg.num_q_heads, cfg.head_dim)
    _expect("q", q, shape=want_q)
    if B > cfg.max_batch:
        raise ValueError(f"batch {B} exceeds the handle's max_batch {cfg.max_batch}")
    _expect("out", out, shape=want_q, dtype=qdt, device=device)
    _expect("lse", lse, shape=want_q[:3], dtype=torch.float32, device=device, required=False)
    P, pool_shape, scale_shape = _pool_shapes(cfg, k_pages, device)
    _expect("v_pages", v_pages, shape=pool_shape, dtype=k_pages.dtype, device=device)
    if cfg.kv_dtype == "fp8":
        sdt = torch.float16 if cfg.scale_dtype == "f16" else torch.float32
        _expect("k_scale", k_scale, shape=scale_shape, dtype=sdt, device=device)
        _expect("v_scale", v_scale, shape=scale_shape, dtype=sdt, device=device)
    elif k_scale is not None or v_scale is not None:
        raise ValueError("k_scale/v_scale are for an fp8 cache only")
    # Rows may sit at any stride (a view of a wider table); each row is packed.
    _expect("block_table", block_table, min_shape=(B, cfg.max_blocks_per_seq), dtype=torch.int32,
            device=device, packed=False)
    if block_table.stride(1) != 1 or block_table.stride(0) < cfg.max_blocks_per_seq:
        raise ValueError("block_table must be 2-D with contiguous rows")
    _expect("context_lens", context_lens, min_shape=(B,), dtype=torch.int32, device=device)
    if cfg.scratch_tokens > 0:
        sshape = (None, cfg.scratch_tokens, cfg.num_kv_heads, cfg.head_dim)
        for name, t in (("scratch_k", scratch_k), ("scratch_v", scratch_v)):
            _expect(name, t, min_shape=(B,) + sshape[1:], dtype=qdt, device=device)
            if tuple(t.shape[1:]) != sshape[1:]:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                                 f"[>= {B}, {cfg.scratch_tokens}, {cfg.num_kv_heads}, "
                                 f"{cfg.head_dim}]")
    elif scratch_k is not None or scratch_v is not None:
        raise ValueError("scratch_k/scratch_v given but the handle has no scratch tokens")
    for name, t in (("q_lens", q_lens), ("scratch_lens", scratch_lens)):
        _expect(name, t, min_shape=(B,), dtype=torch.int32, device=device, required=False)


def validate_write_tensors(cfg: "DecodeConfig", device, k, v, slot_mapping, k_pages, v_pages,
                           *, k_scale=None, v_scale=None) -> None:
    """Check the tensors of a KV-cache write against the handle's config."""
    _expect("slot_mapping", slot_mapping, min_shape=(0,), dtype=torch.int64, device=device)
    N = int(slot_mapping.shape[0])
    row_shape = (N, cfg.num_kv_heads, cfg.head_dim)
    qdt = _TORCH_DTYPE[cfg.q_dtype]
    _expect("k", k, shape=row_shape, dtype=qdt, device=device)
    _expect("v", v, shape=row_shape, dtype=qdt, device=device)
    _, pool_shape, scale_shape = _pool_shapes(cfg, k_pages, device)
    _expect("v_pages", v_pages, shape=pool_shape, dtype=k_pages.dtype, device=device)
    if cfg.kv_dtype == "fp8":
        sdt = torch.float16 if cfg.scale_dtype == "f16" else torch.float32
        _expect("k_scale", k_scale, shape=scale_shape, dtype=sdt, device=device)
        _expect("v_scale", v_scale, shape=scale_shape, dtype=sdt, device=device)
    elif k_scale is not None or v_scale is not None:
        raise ValueError("k_scale/v_scale are for an fp8 cache only")


@dataclass(frozen=True)
class DecodeConfig:
    """Values fixed for the life of a handle (see pd_config)."""

    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_tokens: int = 1
    scratch_tokens: int = 0
    q_dtype: str = "bf16"
    kv_dtype: str = "bf16"
    max_batch: int = 1
    max_blocks_per_seq: int = 1
    max_num_splits: int = 64
    scratch_mask: str = "none"   # "none" or "causal" (see pd_scratch_mask)
    kv_layout: str = "token"     # "token" ([P, bs, Hkv, D]) or "head" ([P, Hkv, bs, D])
    scale_dtype: str = "f32"     # fp8 scale storage: "f32" or "f16" (see pd_scale_dtype)

    def to_c(self) -> _lib.pd_config:
        return _lib.pd_config(
            self.num_q_heads, self.num_kv_heads, self.head_dim, self.block_size,
            self.q_tokens, self.scratch_tokens, _lib.DTYPE_CODES[self.q_dtype],
            _lib.DTYPE_CODES[self.kv_dtype], self.max_batch, self.max_blocks_per_seq,
            self.max_num_splits, _lib.MASK_CODES[self.scratch_mask],
            _lib.LAYOUT_CODES[self.kv_layout], _lib.SCALE_CODES[self.scale_dtype])


class PagedDecoder:
    """Owns one library handle; launches run + reduce on torch's current stream."""

    def __init__(self, cfg: DecodeConfig):
        self.cfg = cfg
        self._handle = _lib.paged_decode_create(cfg.to_c())
        self.device = torch.cuda.current_device()  # the device the handle is bound to
        self.torch_device = torch.device("cuda", self.device)

    def close(self) -> None:
        if self._handle:
            _lib.paged_decode_destroy(self._handle)
            self._handle = 0

    def __del__(self):  # pragma: no cover - interpreter teardown order varies
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self) -> int:
        return self._handle

    def num_splits(self, batch: int, requested: int = 0) -> int:
        return _lib.paged_decode_num_splits(self._handle, batch, requested)

    def workspace_size(self, batch: int, num_splits: int = 0) -> int:
        return _lib.paged_decode_workspace_size(self._handle, batch, num_splits)

    def alloc_workspace(self, batch: int, num_splits: int = 0,
                        device=None) -> Optional[torch.Tensor]:
        n = self.workspace_size(batch, num_splits)
        if n == 0:
            return None
        return torch.empty(n, dtype=torch.uint8, device=device or "cuda")

    def workspace_offsets(self, batch: int, num_splits: int) -> Tuple[int, int]:
        """Byte offsets of O_part and LSE_part in the workspace (S > 1)."""
        c = self.cfg
        S = self.num_splits(batch, num_splits)
        n = batch * c.q_tokens * c.num_q_heads * S
        return 0, (n * c.head_dim * 4 + 255) // 256 * 256

    def make_args(self, q, k_pages, v_pages, block_table, context_lens, out, *,
                  softmax_scale: float, lse=None, num_splits: int = 0, k_scale=None,
                  v_scale=None, scratch_k=None, scratch_v=None, q_lens=None,
                  scratch_lens=None) -> _lib.pd_args:
        validate_decode_tensors(self.cfg, self.torch_device, q, k_pages, v_pages, block_table,
                                context_lens, out, lse=lse, k_scale=k_scale, v_scale=v_scale,
                                scratch_k=scratch_k, scratch_v=scratch_v, q_lens=q_lens,
                                scratch_lens=scratch_lens)
        args = _lib.pd_args(
            q=_ptr(q), k_pages=_ptr(k_pages), v_pages=_ptr(v_pages),
            k_scale=_ptr(k_scale), v_scale=_ptr(v_scale),
            block_table=_ptr(block_table),
            block_table_stride=int(block_table.stride(0)),
            context_lens=_ptr(context_lens),
            scratch_k=_ptr(scratch_k), scratch_v=_ptr(scratch_v),
            out=_ptr(out), lse=_ptr(lse), batch=int(q.shape[0]),
            num_splits=int(num_splits), softmax_scale=float(softmax_scale),
            q_lens=_ptr(q_lens), scratch_lens=_ptr(scratch_lens),
            num_pages=int(k_pages.shape[0]))
        # The struct holds raw device pointers: keep the tensors alive with it,
        # so arguments reused across calls never point at freed memory.
        args.tensors = (q, k_pages, v_pages, block_table, context_lens, out, lse, k_scale,
                        v_scale, scratch_k, scratch_v, q_lens, scratch_lens)
        return args

    def check(self, args: _lib.pd_args, stream: Optional[int] = None) -> Tuple[int, int]:
        """Validate the device-side inputs of a decode call (paged_decode_check).

        Returns (violated pd_check_flag bits, lowest bad sequence index or
        NO_BAD_SEQUENCE); waits for the stream.
        """
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        flags = torch.empty(2, dtype=torch.int32, device=torch.device("cuda", self.device))
        _lib.check(_lib.paged_decode_check(self._handle, args, _ptr(flags), stream))
        torch.cuda.synchronize(self.device)
        mask, first = (int(x) & 0xFFFFFFFF for x in flags.cpu().tolist())
        return mask, first

    def launch(self, args: _lib.pd_args, workspace: Optional[torch.Tensor],
               stream: Optional[int] = None) -> None:
        """run then reduce on ``stream`` (default: torch's current stream).

        With PAGED_DECODE_CHECK=1 in the environment the inputs are validated
        first (outside graph capture) and a violation raises ValueError.
        """
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        if os.environ.get("PAGED_DECODE_CHECK") == "1" and \
                not torch.cuda.is_current_stream_capturing():
            mask, first = self.check(args, stream)
            if mask:
                names = [n for bit, n in _lib.CHECK_NAMES.items() if mask & bit]
                raise ValueError(f"paged decode inputs violate the contract of "
                                 f"{', '.join(names)} (first at sequence {first})")
        ws = _ptr(workspace) or 0
        nbytes = 0 if workspace is None else workspace.numel()
        _lib.check(_lib.paged_decode_run(self._handle, args, ws, nbytes, stream))
        _lib.check(_lib.paged_decode_reduce(self._handle, args, ws, nbytes, stream))

    def write_kv(self, k, v, slot_mapping, k_pages, v_pages, *, k_scale=None, v_scale=None,
                 stream: Optional[int] = None) -> None:
        """Write new tokens' K/V rows [N, Hkv, D] into the paged cache at
        ``slot_mapping`` [N] int64 (page * block_size + slot; negative skips)."""
        validate_write_tensors(self.cfg, self.torch_device, k, v, slot_mapping, k_pages,
                               v_pages, k_scale=k_scale, v_scale=v_scale)
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        # Pool capacity in slots (pages x tokens per page, in either layout):
        # slots at or past it are skipped on the device.
        a = _lib.pd_write_args(k=_ptr(k), v=_ptr(v), slot_mapping=_ptr(slot_mapping),
                               num_tokens=int(slot_mapping.shape[0]), k_pages=_ptr(k_pages),
                               v_pages=_ptr(v_pages), k_scale=_ptr(k_scale),
                               v_scale=_ptr(v_scale),
                               num_slots=int(k_pages.shape[0]) * self.cfg.block_size)
        _lib.check(_lib.paged_decode_write_kv(self._handle, a, stream))

    def __call__(self, q, k_pages, v_pages, block_table, context_lens, *,
                 softmax_scale: float, num_splits: int = 0, k_scale=None, v_scale=None,
                 scratch_k=None, scratch_v=None, out=None, lse=None,
                 workspace=None, want_lse: bool = True, q_lens=None,
                 scratch_lens=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
        B, Tq, Hq, D = q.shape
        if out is None:
            out = torch.empty_like(q)
        if lse is None and want_lse:
            lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = self.alloc_workspace(B, num_splits, q.device)
        args = self.make_args(q, k_pages, v_pages, block_table, context_lens, out,
                              softmax_scale=softmax_scale, lse=lse, num_splits=num_splits,
                              k_scale=k_scale, v_scale=v_scale, scratch_k=scratch_k,
                              scratch_v=scratch_v, q_lens=q_lens, scratch_lens=scratch_lens)
        self.launch(args, workspace)
        return out, lse


def config_for(q: torch.Tensor, k_pages: torch.Tensor, block_table: torch.Tensor, *,
               kv_fp8: bool = False, scratch_tokens: int = 0,
               max_num_splits: int = 64, scratch_mask: str = "none",
               scale_dtype: str = "f32") -> DecodeConfig:
    """DecodeConfig matching tensors of the documented layouts."""
    B, Tq, Hq, D = q.shape
    P, bs, Hkv, Dk = k_pages.shape
    assert D == Dk
    return DecodeConfig(
        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs, q_tokens=Tq,
        scratch_tokens=scratch_tokens, q_dtype=_TORCH_TO_CODE[q.dtype],
        kv_dtype="fp8" if kv_fp8 else _TORCH_TO_CODE[q.dtype], max_batch=max(1, B),
        max_blocks_per_seq=int(block_table.shape[1]), max_num_splits=max_num_splits,
        scratch_mask=scratch_mask, scale_dtype=scale_dtype)


def paged_decode(q, k_pages, v_pages, block_table, context_lens, *, softmax_scale: float,
                 num_splits: int = 0, k_scale=None, v_scale=None, scratch_k=None,
                 scratch_v=None, max_num_splits: int = 64, scratch_mask: str = "none"):
    """One-shot decode call (creates a handle each time; use PagedDecoder in loops)."""
    kv_fp8 = k_pages.dtype in _FP8_POOL_DTYPES
    stok = 0 if scratch_k is None else int(scratch_k.shape[1])
    dec = PagedDecoder(config_for(q, k_pages, block_table, kv_fp8=kv_fp8,
                                  scratch_tokens=stok, scratch_mask=scratch_mask,
                                  scale_dtype="f16" if k_scale is not None
                                  and k_scale.dtype == torch.float16 else "f32",
                                  max_num_splits=max(max_num_splits, num_splits)))
    try:
        return dec(q, k_pages, v_pages, block_table, context_lens,
                   softmax_scale=softmax_scale, num_splits=num_splits, k_scale=k_scale,
                   v_scale=v_scale, scratch_k=scratch_k, scratch_v=scratch_v)
    finally:
        dec.close()
