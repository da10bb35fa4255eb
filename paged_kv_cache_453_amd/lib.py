"""ctypes binding of libpa.so: argument marshalling only.

Each function takes torch tensors that already live on the GPU, checks that
they have the dtype, shape and contiguity the C ABI expects, and passes their
device pointers, the sizes and torch's current HIP stream to the library.  No
computation happens here; a missing library raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_F32 = 0
PA_BF16 = 1

_lib: Optional[ctypes.CDLL] = None


class PagedAttentionError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib.pa_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} returned {status}: {msg}")


def load() -> ctypes.CDLL:
    """Load libpa.so (built by paged_kv_cache_453_amd.build); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m paged_kv_cache_453_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.pa_status_string.argtypes = [i32]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i64,
                                         i32, vp]
    lib.pa_reshape_and_cache.restype = i32
    lib.pa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.pa_decode_workspace_bytes.restype = sz
    lib.pa_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64, i32,
                              f32, i32, vp, sz, i32, vp]
    lib.pa_decode.restype = i32
    lib.pa_decode_splitk_reduce.argtypes = [vp, vp, sz, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.pa_decode_splitk_reduce.restype = i32
    lib.pa_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                     i32, i64, i32, f32, i32, vp]
    lib.pa_prefill_chunk.restype = i32
    _lib = lib
    return lib


EXPORTED = ("pa_reshape_and_cache", "pa_decode_workspace_bytes", "pa_decode",
            "pa_decode_splitk_reduce", "pa_prefill_chunk", "pa_status_string")


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(cond: bool, what: str):
    if not cond:
        raise ValueError(what)


def _check(fn: str, status: int):
    if status != 0:
        raise PagedAttentionError(fn, status)


def _on_gpu(*ts):
    for t in ts:
        _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous and on the GPU")


# --------------------------------------------------------------------------
# the four entry points (plus the workspace query)
# --------------------------------------------------------------------------
def pa_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, stream=None) -> None:
    """key/value [T, Hkv, D] (token stride may exceed Hkv*D); caches [NB, Hkv, 16, D]; slot_mapping int64 [T]."""
    torch = _torch()
    lib = load()
    _on_gpu(key_cache, value_cache, slot_mapping)
    _need(key.is_cuda and value.is_cuda, "key/value must be on the GPU")
    _need(key.dim() == 3 and value.shape == key.shape, "key/value must be [T, Hkv, D]")
    _need(key.stride(2) == 1 and key.stride(1) == key.shape[2] and value.stride(2) == 1 and
          value.stride(1) == value.shape[2], "heads must be contiguous inside a token")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == key.shape[0],
          "slot_mapping must be int64 [T]")
    _need(key.dtype == key_cache.dtype == value.dtype == value_cache.dtype, "dtype mismatch")
    nb, hkv, bs, d = key_cache.shape
    _need(tuple(value_cache.shape) == (nb, hkv, bs, d), "cache shapes differ")
    _need(key.shape[1] == hkv and key.shape[2] == d, "key shape does not match the cache")
    _check("pa_reshape_and_cache", lib.pa_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping),
        key.shape[0], key.stride(0), value.stride(0), hkv, d, bs, nb, _dtype_code(key_cache),
        _stream(stream)))


def pa_decode_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                              partition_size: int) -> int:
    return int(load().pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len,
                                                partition_size))


def pa_decode(out, query, key_cache, value_cache, block_tables, context_lens, scale: float,
              max_context_len: int, partition_size: int = 0, workspace=None, stream=None,
              shared_prefix_blocks=None) -> None:
    """out/query [S, Hq, D]; caches [NB, Hkv, 16, D]; block_tables int32 [S, MB]; context_lens
    int32 [S]; shared_prefix_blocks optional int32 [S] (cache hint, see include/pa.h)."""
    torch = _torch()
    lib = load()
    _on_gpu(out, query, key_cache, value_cache, block_tables, context_lens)
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    s, hq, d = query.shape
    nb, hkv, bs, d2 = key_cache.shape
    _need(d2 == d and tuple(out.shape) == (s, hq, d), "shape mismatch")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == s and context_lens.numel() == s,
          "block_tables must be [S, MB] and context_lens [S]")
    _need(out.dtype == query.dtype == key_cache.dtype == value_cache.dtype, "dtype mismatch")
    if shared_prefix_blocks is not None:
        _on_gpu(shared_prefix_blocks)
        _need(shared_prefix_blocks.dtype == torch.int32 and shared_prefix_blocks.numel() == s,
              "shared_prefix_blocks must be int32 [S]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _on_gpu(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check("pa_decode", lib.pa_decode(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(shared_prefix_blocks), s, hq, hkv, d, bs, block_tables.shape[1],
        nb, int(max_context_len),
        float(scale), int(partition_size), ws_ptr, ws_bytes, _dtype_code(query), _stream(stream)))


def pa_decode_splitk_reduce(out, workspace, context_lens, max_context_len: int,
                            partition_size: int, stream=None) -> None:
    """Merge the split-K partials pa_decode left in workspace into out [S, Hq, D]."""
    lib = load()
    _on_gpu(out, workspace, context_lens)
    s, hq, d = out.shape
    _check("pa_decode_splitk_reduce", lib.pa_decode_splitk_reduce(
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(context_lens), s, hq, d, int(max_context_len), int(partition_size),
        _dtype_code(out), _stream(stream)))


def pa_prefill_chunk(out, query, key_cache, value_cache, block_tables, query_start_loc,
                     context_lens, scale: float, max_query_len: int, stream=None) -> None:
    """out/query [Tq, Hq, D]; query_start_loc int32 [S+1]; context_lens int32 [S] (chunk included)."""
    torch = _torch()
    lib = load()
    _on_gpu(out, query, key_cache, value_cache, block_tables, query_start_loc, context_lens)
    _need(block_tables.dtype == torch.int32 and query_start_loc.dtype == torch.int32 and
          context_lens.dtype == torch.int32, "index arrays must be int32")
    tq, hq, d = query.shape
    nb, hkv, bs, d2 = key_cache.shape
    s = context_lens.numel()
    _need(d2 == d and tuple(out.shape) == (tq, hq, d), "shape mismatch")
    _need(query_start_loc.numel() == s + 1 and block_tables.shape[0] == s, "sequence count mismatch")
    _need(out.dtype == query.dtype == key_cache.dtype == value_cache.dtype, "dtype mismatch")
    _check("pa_prefill_chunk", lib.pa_prefill_chunk(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(query_start_loc), _ptr(context_lens), s, tq, hq, hkv, d, bs, block_tables.shape[1],
        nb, int(max_query_len), float(scale), _dtype_code(query), _stream(stream)))
