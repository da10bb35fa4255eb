"""Paged attention for AMD Instinct MI355X (gfx950).

The compute lives in libpa.so (hand-written HIP kernels behind a C ABI declared
in include/pa.h); `lib` is its thin ctypes binding.
"""
from . import lib
from .lib import (pa_decode, pa_decode_splitk_reduce, pa_decode_workspace_bytes,
                  pa_prefill_chunk, pa_reshape_and_cache, PagedAttentionError)

__all__ = ["lib", "pa_decode", "pa_decode_splitk_reduce", "pa_decode_workspace_bytes",
           "pa_prefill_chunk", "pa_reshape_and_cache", "PagedAttentionError"]
