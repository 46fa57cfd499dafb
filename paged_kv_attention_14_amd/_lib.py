"""ctypes binding of libpaged_decode.so (the C ABI in include/paged_decode.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI. There is no fallback; if the shared library is
missing, loading raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpaged_decode.so")

PD_OK = 0
PD_ERR_INVALID_ARG = 1
PD_ERR_UNSUPPORTED = 2
PD_ERR_WORKSPACE_TOO_SMALL = 3
PD_ERR_HIP = 4
STATUS_NAMES = {
    PD_OK: "PD_OK",
    PD_ERR_INVALID_ARG: "PD_ERR_INVALID_ARG",
    PD_ERR_UNSUPPORTED: "PD_ERR_UNSUPPORTED",
    PD_ERR_WORKSPACE_TOO_SMALL: "PD_ERR_WORKSPACE_TOO_SMALL",
    PD_ERR_HIP: "PD_ERR_HIP",
}

PD_DTYPE_BF16 = 0
PD_DTYPE_F16 = 1
PD_DTYPE_FP8_E4M3FN = 2
DTYPE_CODES = {"bf16": PD_DTYPE_BF16, "f16": PD_DTYPE_F16, "fp8": PD_DTYPE_FP8_E4M3FN}

PD_SCRATCH_MASK_NONE = 0
PD_SCRATCH_MASK_CAUSAL = 1
MASK_CODES = {"none": PD_SCRATCH_MASK_NONE, "causal": PD_SCRATCH_MASK_CAUSAL}

PD_KV_LAYOUT_TOKEN_MAJOR = 0
PD_KV_LAYOUT_HEAD_MAJOR = 1
LAYOUT_CODES = {"token": PD_KV_LAYOUT_TOKEN_MAJOR, "head": PD_KV_LAYOUT_HEAD_MAJOR}

# Bits of the flags word paged_decode_check writes.
PD_CHECK_CONTEXT_LENS = 1
PD_CHECK_BLOCK_TABLE = 2
PD_CHECK_Q_LENS = 4
PD_CHECK_SCRATCH_LENS = 8
CHECK_NAMES = {
    PD_CHECK_CONTEXT_LENS: "context_lens",
    PD_CHECK_BLOCK_TABLE: "block_table",
    PD_CHECK_Q_LENS: "q_lens",
    PD_CHECK_SCRATCH_LENS: "scratch_lens",
}
NO_BAD_SEQUENCE = 0xFFFFFFFF

PD_SCALE_F32 = 0
PD_SCALE_F16 = 1
SCALE_CODES = {"f32": PD_SCALE_F32, "f16": PD_SCALE_F16}


class pd_config(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("q_tokens", ctypes.c_int32),
        ("scratch_tokens", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_num_splits", ctypes.c_int32),
        ("scratch_mask", ctypes.c_int32),
        ("kv_layout", ctypes.c_int32),
        ("scale_dtype", ctypes.c_int32),
    ]


class pd_args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("block_table_stride", ctypes.c_int64),
        ("context_lens", ctypes.c_void_p),
        ("scratch_k", ctypes.c_void_p),
        ("scratch_v", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_lens", ctypes.c_void_p),
        ("scratch_lens", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
    ]


class pd_write_args(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("slot_mapping", ctypes.c_void_p),
        ("num_tokens", ctypes.c_int32),
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("num_slots", ctypes.c_int64),
    ]


class PagedDecodeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None

# Every entry point the header declares, with its ctypes signature.
SIGNATURES = {
    "paged_decode_create": (ctypes.c_int, [ctypes.POINTER(pd_config), ctypes.POINTER(ctypes.c_void_p)]),
    "paged_decode_destroy": (None, [ctypes.c_void_p]),
    "paged_decode_num_splits": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.POINTER(ctypes.c_int32)]),
    "paged_decode_workspace_size": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.POINTER(ctypes.c_size_t)]),
    "paged_decode_run": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(pd_args), ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]),
    "paged_decode_reduce": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(pd_args), ctypes.c_void_p,
                                           ctypes.c_size_t, ctypes.c_void_p]),
    "paged_decode_run_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(pd_args),
                                                ctypes.c_void_p]),
    "paged_decode_write_kv": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(pd_write_args),
                                             ctypes.c_void_p]),
    "paged_decode_check": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(pd_args), ctypes.c_void_p,
                                          ctypes.c_void_p]),
    "paged_decode_last_error": (ctypes.c_char_p, []),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m paged_kv_attention_14_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, argtypes) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = argtypes
    _lib = lib
    return lib


def last_error() -> str:
    msg = load_library().paged_decode_last_error()
    return msg.decode() if msg else ""


def check(status: int) -> None:
    if status != PD_OK:
        raise PagedDecodeError(status, last_error())


# --- the C entry points under their own names -------------------------------

def paged_decode_create(cfg: pd_config) -> int:
    """Create a handle for ``cfg``; returns the opaque handle as an int."""
    h = ctypes.c_void_p()
    check(load_library().paged_decode_create(ctypes.byref(cfg), ctypes.byref(h)))
    return int(h.value)


def paged_decode_destroy(handle: int) -> None:
    load_library().paged_decode_destroy(ctypes.c_void_p(handle))


def paged_decode_num_splits(handle: int, batch: int, requested: int) -> int:
    out = ctypes.c_int32()
    check(load_library().paged_decode_num_splits(ctypes.c_void_p(handle), batch, requested,
                                                 ctypes.byref(out)))
    return int(out.value)


def paged_decode_workspace_size(handle: int, batch: int, num_splits: int) -> int:
    out = ctypes.c_size_t()
    check(load_library().paged_decode_workspace_size(ctypes.c_void_p(handle), batch, num_splits,
                                                     ctypes.byref(out)))
    return int(out.value)


def paged_decode_run(handle: int, args: pd_args, workspace: int, workspace_bytes: int,
                     stream: int) -> int:
    """Launch the decode kernel; returns the status (raise with ``check``)."""
    return load_library().paged_decode_run(ctypes.c_void_p(handle), ctypes.byref(args),
                                           ctypes.c_void_p(workspace or None), workspace_bytes,
                                           ctypes.c_void_p(stream or None))


def paged_decode_reduce(handle: int, args: pd_args, workspace: int, workspace_bytes: int,
                        stream: int) -> int:
    """Launch the split-K combine; returns the status (raise with ``check``)."""
    return load_library().paged_decode_reduce(ctypes.c_void_p(handle), ctypes.byref(args),
                                              ctypes.c_void_p(workspace or None), workspace_bytes,
                                              ctypes.c_void_p(stream or None))


def paged_decode_run_noalloc(handle: int, args: pd_args, stream: int) -> int:
    """Launch run + reduce with the library-owned split workspace (no
    allocation); returns the status (raise with ``check``)."""
    return load_library().paged_decode_run_noalloc(ctypes.c_void_p(handle), ctypes.byref(args),
                                                   ctypes.c_void_p(stream or None))


NOALLOC_WORKSPACE_BYTES = 16 << 20


def paged_decode_write_kv(handle: int, args: pd_write_args, stream: int) -> int:
    """Launch the KV-cache write; returns the status (raise with ``check``)."""
    return load_library().paged_decode_write_kv(ctypes.c_void_p(handle), ctypes.byref(args),
                                                ctypes.c_void_p(stream or None))


def paged_decode_check(handle: int, args: pd_args, flags: int, stream: int) -> int:
    """Launch the input validation into device words ``flags`` [2] uint32;
    returns the status (raise with ``check``)."""
    return load_library().paged_decode_check(ctypes.c_void_p(handle), ctypes.byref(args),
                                             ctypes.c_void_p(flags or None),
                                             ctypes.c_void_p(stream or None))


def paged_decode_last_error() -> str:
    return last_error()
