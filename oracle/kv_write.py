"""Writing new K/V tokens into the paged cache, on the CPU.

TEST INFRASTRUCTURE: part of the CPU oracle. Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import it. It shares no code with
the HIP path.

The write step precedes decode: each new token's K and V rows land in the
page slot the caller names, and for an e4m3fn cache they are quantised there,
with one symmetric scale per (token, kv head). "[ROCm] Add FlyDSL
paged-attention decode backend (dense + fp8) with benchmark" (review thread)
places the fp8 scales at KV-quantisation time rather than in each decode
call; its kernel reads e4m3fn codes with a symmetric per-token scale
(Kernels).

Readings (also in the design notes):

* the target of token i is slot_mapping[i] = page * bs + slot, and a
  negative entry skips the token (the usual slot-mapping convention of paged
  caches; the pages do not spell the write interface out);
* fp8: absmax over the D values of the (token, kv head) row, scale =
  absmax / 448 and y = x / scale, both single-precision divisions (the
  precision the GPU takes these decisions in); codes are e4m3fn of
  clamp(y, -448, 448) rounded to nearest, ties to even; a zero row gets
  scale 0 and codes 0.
* f16 scale storage (the pull request's inputs carry a use_fp32_scales
  switch, off by default): the f32 scale is rounded to the nearest f16
  (ties to even; capped at the largest finite f16, 65504) and that rounded
  value is both the divisor and the stored scale; a row whose rounded scale
  is 0 gets codes 0.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import e4m3fn

E4M3_MAX = np.float32(448.0)
F16_MAX = np.float32(65504.0)


def quantise_row(x: np.ndarray, scale_dtype: str = "f32") -> Tuple[np.ndarray, np.float32]:
    """e4m3fn codes [D] and the scale (as f32) of one (token, kv head) row."""
    x = np.asarray(x, dtype=np.float32)
    absmax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    scale = np.float32(absmax / E4M3_MAX)
    if scale_dtype == "f16":
        scale = np.float32(np.float16(min(scale, F16_MAX)))   # numpy rounds to nearest even
    else:
        assert scale_dtype == "f32"
    if scale == 0.0:
        return np.zeros(x.shape, dtype=np.uint8), np.float32(0.0)
    y = (x / scale).astype(np.float32)          # f32 division, per element
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    return e4m3fn.encode(y), scale


def write_kv(k_pages: np.ndarray, v_pages: np.ndarray, new_k: np.ndarray, new_v: np.ndarray,
             slot_mapping: np.ndarray, *, kv_format: str = "dense",
             k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None,
             kv_layout: str = "token"):
    """Return copies of the pools (and scales) with the new tokens written.

    new_k, new_v [N, Hkv, D]; slot_mapping [N]; pools [P, bs, Hkv, D], or
    [P, Hkv, bs, D] for kv_layout "head" (uint8 codes for fp8, with scales
    [P, bs, Hkv] or [P, Hkv, bs]: float32, or float16 for f16 storage, the
    storage type being that of the arrays passed).
    """
    assert kv_format in ("dense", "fp8") and kv_layout in ("token", "head")
    kp, vp = k_pages.copy(), v_pages.copy()
    ks = None if k_scale is None else k_scale.copy()
    vs = None if v_scale is None else v_scale.copy()
    head = kv_layout == "head"
    sdt = "f16" if (ks is not None and ks.dtype == np.float16) else "f32"
    bs = kp.shape[2] if head else kp.shape[1]
    H = kp.shape[1] if head else kp.shape[2]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        page, off = int(slot) // bs, int(slot) % bs
        for h in range(H):
            at = (page, h, off) if head else (page, off, h)
            if kv_format == "dense":
                kp[at] = new_k[i, h]
                vp[at] = new_v[i, h]
            else:
                kp[at], ks[at] = quantise_row(new_k[i, h], sdt)
                vp[at], vs[at] = quantise_row(new_v[i, h], sdt)
    return kp, vp, ks, vs
