"""Paged-KV split-K decode attention for MI355X (gfx950).

The computation lives in ``libpaged_decode.so`` (hand-written HIP kernels
behind the C ABI of ``include/paged_decode.h``). This package is its thin
Python binding: ``_lib`` exposes the C entry points under their own names,
``decode`` wraps them for torch device tensors.
"""

from . import _lib  # noqa: F401
from ._lib import PagedDecodeError, load_library  # noqa: F401
from .decode import DecodeConfig, PagedDecoder, config_for, paged_decode  # noqa: F401
