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
PA_FP8_E4M3 = 2

_lib: Optional[ctypes.CDLL] = None


PA_ERR_SHAPE, PA_ERR_NO_BLOCKS, PA_ERR_SEQ, PA_ERR_BUSY = -2, -6, -7, -8


class PagedAttentionError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib.pa_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} returned {status}: {msg}")


class OutOfBlocks(PagedAttentionError):
    """A pool has too few free blocks; the manager changed nothing."""


class Busy(PagedAttentionError):
    """Pending block moves must be taken and run first; nothing changed."""


class SequenceError(PagedAttentionError):
    """Unknown or duplicate sequence id, or the wrong side of a swap."""


class ShapeError(PagedAttentionError):
    """A size or index argument is out of range."""


_ERRORS = {PA_ERR_NO_BLOCKS: OutOfBlocks, PA_ERR_BUSY: Busy, PA_ERR_SEQ: SequenceError,
           PA_ERR_SHAPE: ShapeError}


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
    lib.pa_decode_no_alloc_scratch_bytes.argtypes = []
    lib.pa_decode_no_alloc_scratch_bytes.restype = sz
    lib.pa_decode_no_alloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                       i64, i32, f32, i32, i32, vp]
    lib.pa_decode_no_alloc.restype = i32
    lib.pa_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                     i32, i64, i32, f32, i32, vp]
    lib.pa_prefill_chunk.restype = i32
    lib.pa_reshape_and_cache_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32,
                                             i64, i32, f32, f32, vp]
    lib.pa_reshape_and_cache_fp8.restype = i32
    lib.pa_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64,
                                  i32, f32, f32, f32, i32, vp, sz, i32, vp]
    lib.pa_decode_fp8.restype = i32
    lib.pa_decode_shared_prefix.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                            i32, i32, i32, i64, i32, f32, i32, vp, sz, i32, vp]
    lib.pa_decode_shared_prefix.restype = i32
    lib.pa_decode_fp8_shared_prefix.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                                i32, i32, i32, i32, i64, i32, f32, f32, f32, i32,
                                                vp, sz, i32, vp]
    lib.pa_decode_fp8_shared_prefix.restype = i32
    lib.pa_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.pa_prefill_workspace_bytes.restype = sz
    lib.pa_prefill_chunk_split.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                           i32, i32, i64, i32, i32, i32, f32, vp, sz, i32, vp]
    lib.pa_prefill_chunk_split.restype = i32
    lib.pa_prefill_chunk_fp8_split.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                               i32, i32, i32, i64, i32, i32, i32, f32, f32, f32,
                                               vp, sz, i32, vp]
    lib.pa_prefill_chunk_fp8_split.restype = i32
    lib.pa_sample.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp, vp, i32, vp]
    lib.pa_sample.restype = i32
    lib.pa_copy_blocks.argtypes = [vp, vp, vp, i64, i32, i32, i32, i64, i32, vp]
    lib.pa_copy_blocks.restype = i32
    lib.pa_swap_blocks.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, vp]
    lib.pa_swap_blocks.restype = i32
    lib.pa_prefill_chunk_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                         i32, i32, i64, i32, f32, f32, f32, i32, vp]
    lib.pa_prefill_chunk_fp8.restype = i32
    lib.pa_stream_read_sink_words.argtypes = []
    lib.pa_stream_read_sink_words.restype = i32
    lib.pa_stream_read.argtypes = [vp, i64, vp, vp]
    lib.pa_stream_read.restype = i32
    pp = ctypes.POINTER(ctypes.c_void_p)
    for name, args, res in (
            ("pa_bm_create", [i64, i64, i32, pp], i32),
            ("pa_bm_destroy", [vp], None),
            ("pa_bm_add_sequence", [vp, i64], i32),
            ("pa_bm_fork", [vp, i64, i64], i32),
            ("pa_bm_share", [vp, i64, i64, vp, i32], i32),
            ("pa_bm_free_sequence", [vp, i64], i32),
            ("pa_bm_append_slots", [vp, i64, i32, vp], i32),
            ("pa_bm_append_batch", [vp, vp, vp, i32, vp, vp], i32),
            ("pa_bm_swap_out", [vp, vp, i32], i32),
            ("pa_bm_swap_in", [vp, vp, i32], i32),
            ("pa_bm_pending_moves", [vp, vp], i32),
            ("pa_bm_take_moves", [vp, vp, vp, vp], i32),
            ("pa_bm_num_tokens", [vp, i64, vp], i32),
            ("pa_bm_is_swapped", [vp, i64, vp], i32),
            ("pa_bm_block_table", [vp, i64, vp, i32, vp], i32),
            ("pa_bm_num_free", [vp, i32], i64),
            ("pa_bm_build_batch", [vp, vp, i32, i32, vp, vp, vp], i32),
            ("pa_bm_check", [vp], i32),
            ("pa_bm_prefix_groups", [vp, vp, i32, vp, vp, vp], i32),
            ("pa_bm_prefix_keys", [vp, i64, ctypes.c_uint64, vp], i32),
            ("pa_bm_add_prompt", [vp, i64, vp, i64, ctypes.c_uint64, vp], i32),
            ("pa_bm_append_tokens", [vp, i64, vp, i32, vp], i32),
            ("pa_bm_num_cached_blocks", [vp], i64)):
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


EXPORTED = ("pa_reshape_and_cache", "pa_decode_workspace_bytes", "pa_decode",
            "pa_decode_splitk_reduce", "pa_decode_no_alloc", "pa_decode_no_alloc_scratch_bytes", "pa_prefill_chunk", "pa_reshape_and_cache_fp8",
            "pa_decode_fp8", "pa_prefill_chunk_fp8", "pa_decode_shared_prefix",
            "pa_decode_fp8_shared_prefix", "pa_prefill_workspace_bytes", "pa_prefill_chunk_split",
            "pa_prefill_chunk_fp8_split", "pa_sample", "pa_copy_blocks",
            "pa_swap_blocks", "pa_stream_read_sink_words", "pa_stream_read", "pa_status_string")


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t, fp8_ok: bool = False) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if fp8_ok and t.dtype == torch.uint8:
        return PA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16"
                    + (" (or uint8 FP8 codes)" if fp8_ok else ""))


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
        raise _ERRORS.get(status, PagedAttentionError)(fn, status)


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


def pa_decode_no_alloc_scratch_bytes() -> int:
    return int(load().pa_decode_no_alloc_scratch_bytes())


def pa_decode_no_alloc(out, query, key_cache, value_cache, block_tables, context_lens,
                       scale: float, max_context_len: int, partition_size: int = 0, stream=None,
                       shared_prefix_blocks=None) -> None:
    """pa_decode plus the split-K merge in one call, with the partials in the library's fixed
    device buffer (no workspace, nothing allocated); raises for PA_ERR_SCRATCH when they do not
    fit pa_decode_no_alloc_scratch_bytes()."""
    lib = load()
    s, hq, d, nb, hkv, bs, _, _ = _decode_marshal(
        out, query, key_cache, value_cache, block_tables, context_lens, None,
        shared_prefix_blocks)
    _check("pa_decode_no_alloc", lib.pa_decode_no_alloc(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(shared_prefix_blocks), s, hq, hkv, d, bs, block_tables.shape[1],
        nb, int(max_context_len), float(scale), int(partition_size), _dtype_code(query),
        _stream(stream)))


def _decode_marshal(out, query, key_cache, value_cache, block_tables, context_lens,
                    workspace, shared_prefix_blocks, prefix_group=None, fp8: bool = False):
    """Shape / dtype checks shared by the decode wrappers; returns (S, Hq, D, NB, Hkv, BS,
    workspace pointer, workspace bytes)."""
    torch = _torch()
    _on_gpu(out, query, key_cache, value_cache, block_tables, context_lens)
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    if fp8:
        _need(key_cache.dtype == torch.uint8 and value_cache.dtype == torch.uint8,
              "FP8 caches are uint8 tensors of E4M3 codes")
    s, hq, d = query.shape
    nb, hkv, bs, d2 = key_cache.shape
    _need(d2 == d and tuple(out.shape) == (s, hq, d) and value_cache.shape == key_cache.shape,
          "shape mismatch")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == s and context_lens.numel() == s,
          "block_tables must be [S, MB] and context_lens [S]")
    if fp8:
        _need(out.dtype == query.dtype, "query and output dtypes differ")
    else:
        _need(out.dtype == query.dtype == key_cache.dtype == value_cache.dtype, "dtype mismatch")
    for name, t in (("shared_prefix_blocks", shared_prefix_blocks), ("prefix_group", prefix_group)):
        if t is not None:
            _on_gpu(t)
            _need(t.dtype == torch.int32 and t.numel() == s, f"{name} must be int32 [S]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _on_gpu(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return s, hq, d, nb, hkv, bs, ws_ptr, ws_bytes


def pa_decode_shared_prefix(out, query, key_cache, value_cache, block_tables, context_lens,
                            scale: float, max_context_len: int, partition_size: int, workspace,
                            shared_prefix_blocks, prefix_group, max_group_size: int,
                            stream=None) -> None:
    """pa_decode for groups of sequences sharing leading blocks: prefix_group int32 [S] names
    each sequence's group leader, shared_prefix_blocks int32 [S] the shared table entries
    (see include/pa.h).  Follow with pa_decode_splitk_reduce."""
    lib = load()
    s, hq, d, nb, hkv, bs, ws_ptr, ws_bytes = _decode_marshal(
        out, query, key_cache, value_cache, block_tables, context_lens, workspace,
        shared_prefix_blocks, prefix_group)
    _check("pa_decode_shared_prefix", lib.pa_decode_shared_prefix(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(shared_prefix_blocks), _ptr(prefix_group), int(max_group_size),
        s, hq, hkv, d, bs, block_tables.shape[1], nb, int(max_context_len), float(scale),
        int(partition_size), ws_ptr, ws_bytes, _dtype_code(query), _stream(stream)))


def pa_decode_fp8_shared_prefix(out, query, key_cache, value_cache, block_tables, context_lens,
                                scale: float, k_scale: float, v_scale: float,
                                max_context_len: int, partition_size: int, workspace,
                                shared_prefix_blocks, prefix_group, max_group_size: int,
                                stream=None) -> None:
    """pa_decode_shared_prefix over uint8 E4M3 caches (codes stand for value * k/v scale)."""
    lib = load()
    s, hq, d, nb, hkv, bs, ws_ptr, ws_bytes = _decode_marshal(
        out, query, key_cache, value_cache, block_tables, context_lens, workspace,
        shared_prefix_blocks, prefix_group, fp8=True)
    _check("pa_decode_fp8_shared_prefix", lib.pa_decode_fp8_shared_prefix(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(shared_prefix_blocks), _ptr(prefix_group), int(max_group_size),
        s, hq, hkv, d, bs, block_tables.shape[1], nb, int(max_context_len), float(scale),
        float(k_scale), float(v_scale), int(partition_size), ws_ptr, ws_bytes,
        _dtype_code(query), _stream(stream)))


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


def pa_prefill_workspace_bytes(num_query_tokens: int, num_heads: int, head_dim: int,
                               max_context_len: int, split_tokens: int) -> int:
    return int(load().pa_prefill_workspace_bytes(num_query_tokens, num_heads, head_dim,
                                                 max_context_len, split_tokens))


def _prefill_marshal(out, query, key_cache, value_cache, block_tables, query_start_loc,
                     context_lens, workspace, fp8: bool):
    torch = _torch()
    _on_gpu(out, query, key_cache, value_cache, block_tables, query_start_loc, context_lens,
            workspace)
    _need(block_tables.dtype == torch.int32 and query_start_loc.dtype == torch.int32 and
          context_lens.dtype == torch.int32, "index arrays must be int32")
    tq, hq, d = query.shape
    nb, hkv, bs, d2 = key_cache.shape
    s = context_lens.numel()
    _need(d2 == d and tuple(out.shape) == (tq, hq, d) and value_cache.shape == key_cache.shape,
          "shape mismatch")
    _need(query_start_loc.numel() == s + 1 and block_tables.shape[0] == s, "sequence count mismatch")
    if fp8:
        _need(key_cache.dtype == torch.uint8 and value_cache.dtype == torch.uint8,
              "FP8 caches are uint8 tensors of E4M3 codes")
        _need(out.dtype == query.dtype, "query and output dtypes differ")
    else:
        _need(out.dtype == query.dtype == key_cache.dtype == value_cache.dtype, "dtype mismatch")
    return s, tq, hq, hkv, d, bs, nb, workspace.numel() * workspace.element_size()


def pa_prefill_chunk_split(out, query, key_cache, value_cache, block_tables, query_start_loc,
                           context_lens, scale: float, max_query_len: int, max_context_len: int,
                           split_tokens: int, workspace, stream=None) -> None:
    """pa_prefill_chunk with long causal key ranges split over workgroups (split_tokens keys
    each) and merged; workspace of pa_prefill_workspace_bytes() bytes."""
    lib = load()
    s, tq, hq, hkv, d, bs, nb, wsb = _prefill_marshal(
        out, query, key_cache, value_cache, block_tables, query_start_loc, context_lens,
        workspace, fp8=False)
    _check("pa_prefill_chunk_split", lib.pa_prefill_chunk_split(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(query_start_loc), _ptr(context_lens), s, tq, hq, hkv, d, bs, block_tables.shape[1],
        nb, int(max_query_len), int(max_context_len), int(split_tokens), float(scale),
        _ptr(workspace), wsb, _dtype_code(query), _stream(stream)))


def pa_prefill_chunk_fp8_split(out, query, key_cache, value_cache, block_tables, query_start_loc,
                               context_lens, scale: float, k_scale: float, v_scale: float,
                               max_query_len: int, max_context_len: int, split_tokens: int,
                               workspace, stream=None) -> None:
    """pa_prefill_chunk_split over uint8 E4M3 caches."""
    lib = load()
    s, tq, hq, hkv, d, bs, nb, wsb = _prefill_marshal(
        out, query, key_cache, value_cache, block_tables, query_start_loc, context_lens,
        workspace, fp8=True)
    _check("pa_prefill_chunk_fp8_split", lib.pa_prefill_chunk_fp8_split(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(query_start_loc), _ptr(context_lens), s, tq, hq, hkv, d, bs, block_tables.shape[1],
        nb, int(max_query_len), int(max_context_len), int(split_tokens), float(scale),
        float(k_scale), float(v_scale), _ptr(workspace), wsb, _dtype_code(query),
        _stream(stream)))


# --------------------------------------------------------------------------
# FP8 (E4M3) KV cache
# --------------------------------------------------------------------------
def pa_reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale: float,
                             v_scale: float, stream=None) -> None:
    """key/value [T, Hkv, D] fp32 or bf16; caches uint8 [NB, Hkv, 16, D] (E4M3 codes);
    slot_mapping int64 [T]; code = E4M3(x / scale)."""
    torch = _torch()
    lib = load()
    _on_gpu(key_cache, value_cache, slot_mapping)
    _need(key.is_cuda and value.is_cuda, "key/value must be on the GPU")
    _need(key.dim() == 3 and value.shape == key.shape, "key/value must be [T, Hkv, D]")
    _need(key.stride(2) == 1 and key.stride(1) == key.shape[2] and value.stride(2) == 1 and
          value.stride(1) == value.shape[2], "heads must be contiguous inside a token")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == key.shape[0],
          "slot_mapping must be int64 [T]")
    _need(key.dtype == value.dtype, "key and value dtypes differ")
    _need(key_cache.dtype == torch.uint8 and value_cache.dtype == torch.uint8,
          "FP8 caches are uint8 tensors of E4M3 codes")
    nb, hkv, bs, d = key_cache.shape
    _need(tuple(value_cache.shape) == (nb, hkv, bs, d), "cache shapes differ")
    _need(key.shape[1] == hkv and key.shape[2] == d, "key shape does not match the cache")
    _check("pa_reshape_and_cache_fp8", lib.pa_reshape_and_cache_fp8(
        _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping),
        key.shape[0], key.stride(0), value.stride(0), hkv, d, bs, nb, _dtype_code(key),
        float(k_scale), float(v_scale), _stream(stream)))


def pa_decode_fp8(out, query, key_cache, value_cache, block_tables, context_lens, scale: float,
                  k_scale: float, v_scale: float, max_context_len: int, partition_size: int = 0,
                  workspace=None, stream=None, shared_prefix_blocks=None) -> None:
    """pa_decode over uint8 E4M3 caches whose codes stand for value * k_scale / v_scale."""
    torch = _torch()
    lib = load()
    _on_gpu(out, query, key_cache, value_cache, block_tables, context_lens)
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    _need(key_cache.dtype == torch.uint8 and value_cache.dtype == torch.uint8,
          "FP8 caches are uint8 tensors of E4M3 codes")
    s, hq, d = query.shape
    nb, hkv, bs, d2 = key_cache.shape
    _need(d2 == d and tuple(out.shape) == (s, hq, d) and value_cache.shape == key_cache.shape,
          "shape mismatch")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == s and context_lens.numel() == s,
          "block_tables must be [S, MB] and context_lens [S]")
    _need(out.dtype == query.dtype, "query and output dtypes differ")
    if shared_prefix_blocks is not None:
        _on_gpu(shared_prefix_blocks)
        _need(shared_prefix_blocks.dtype == torch.int32 and shared_prefix_blocks.numel() == s,
              "shared_prefix_blocks must be int32 [S]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _on_gpu(workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check("pa_decode_fp8", lib.pa_decode_fp8(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(shared_prefix_blocks), s, hq, hkv, d, bs, block_tables.shape[1],
        nb, int(max_context_len), float(scale), float(k_scale), float(v_scale),
        int(partition_size), ws_ptr, ws_bytes, _dtype_code(query), _stream(stream)))


def pa_prefill_chunk_fp8(out, query, key_cache, value_cache, block_tables, query_start_loc,
                         context_lens, scale: float, k_scale: float, v_scale: float,
                         max_query_len: int, stream=None) -> None:
    """pa_prefill_chunk over uint8 E4M3 caches whose codes stand for value * k_scale /
    v_scale; out/query bf16 [Tq, Hq, D]."""
    torch = _torch()
    lib = load()
    _on_gpu(out, query, key_cache, value_cache, block_tables, query_start_loc, context_lens)
    _need(block_tables.dtype == torch.int32 and query_start_loc.dtype == torch.int32 and
          context_lens.dtype == torch.int32, "index arrays must be int32")
    _need(key_cache.dtype == torch.uint8 and value_cache.dtype == torch.uint8,
          "FP8 caches are uint8 tensors of E4M3 codes")
    tq, hq, d = query.shape
    nb, hkv, bs, d2 = key_cache.shape
    s = context_lens.numel()
    _need(d2 == d and tuple(out.shape) == (tq, hq, d) and value_cache.shape == key_cache.shape,
          "shape mismatch")
    _need(query_start_loc.numel() == s + 1 and block_tables.shape[0] == s, "sequence count mismatch")
    _need(out.dtype == query.dtype, "query and output dtypes differ")
    _check("pa_prefill_chunk_fp8", lib.pa_prefill_chunk_fp8(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        _ptr(query_start_loc), _ptr(context_lens), s, tq, hq, hkv, d, bs, block_tables.shape[1],
        nb, int(max_query_len), float(scale), float(k_scale), float(v_scale),
        _dtype_code(query), _stream(stream)))


# --------------------------------------------------------------------------
# next-token sampling
# --------------------------------------------------------------------------
def pa_sample(tokens, logits, temperature, top_k, top_p, uniform, stream=None) -> None:
    """tokens int32 [S]; logits [S, V] fp32/bf16 (row stride may exceed V); temperature,
    top_p, uniform float32 [S]; top_k int32 [S] -- all on the GPU."""
    torch = _torch()
    lib = load()
    _on_gpu(tokens, temperature, top_k, top_p, uniform)
    _need(logits.is_cuda and logits.dim() == 2 and logits.stride(1) == 1,
          "logits must be a [S, V] GPU tensor with contiguous rows")
    s, v = logits.shape
    _need(tokens.dtype == torch.int32 and tokens.numel() == s, "tokens must be int32 [S]")
    _need(top_k.dtype == torch.int32 and top_k.numel() == s, "top_k must be int32 [S]")
    for t in (temperature, top_p, uniform):
        _need(t.dtype == torch.float32 and t.numel() == s, "per-row parameters must be float32 [S]")
    _check("pa_sample", lib.pa_sample(
        _ptr(tokens), _ptr(logits), logits.stride(0), s, v, _ptr(temperature), _ptr(top_k),
        _ptr(top_p), _ptr(uniform), _dtype_code(logits), _stream(stream)))


def pa_stream_read_sink_words() -> int:
    """Words of the sink pa_stream_read writes (one per workgroup)."""
    return int(load().pa_stream_read_sink_words())


def pa_stream_read(buffer, sink, stream=None) -> None:
    """Read every byte of `buffer` (a contiguous GPU tensor, 16-byte aligned,
    a multiple of 16 bytes) with plain 16-byte loads; `sink` is a GPU int32 or
    uint32 tensor of pa_stream_read_sink_words() elements, which receives the
    per-workgroup XOR folds.  A measurement aid, not an operation of the method."""
    lib = load()
    _on_gpu(buffer, sink)
    _need(buffer.is_contiguous(), "buffer must be contiguous")
    _need(sink.is_contiguous() and sink.element_size() == 4 and
          sink.numel() >= lib.pa_stream_read_sink_words(), "sink too small")
    nbytes = buffer.numel() * buffer.element_size()
    _check("pa_stream_read", lib.pa_stream_read(_ptr(buffer), nbytes, _ptr(sink), _stream(stream)))


# --------------------------------------------------------------------------
# block data movement
# --------------------------------------------------------------------------
def pa_copy_blocks(key_cache, value_cache, block_mapping, stream=None) -> None:
    """Copy block src onto block dst in both pools for each row (src, dst) of
    block_mapping (device int32 [n, 2]); pairs must be independent."""
    torch = _torch()
    lib = load()
    _on_gpu(key_cache, value_cache, block_mapping)
    _need(block_mapping.dtype == torch.int32 and block_mapping.dim() == 2 and
          block_mapping.shape[1] == 2, "block_mapping must be int32 [n, 2]")
    _need(key_cache.dtype == value_cache.dtype and key_cache.shape == value_cache.shape,
          "caches differ")
    nb, hkv, bs, d = key_cache.shape
    _check("pa_copy_blocks", lib.pa_copy_blocks(
        _ptr(key_cache), _ptr(value_cache), _ptr(block_mapping), block_mapping.shape[0], hkv, d,
        bs, nb, _dtype_code(key_cache, fp8_ok=True), _stream(stream)))


def pa_swap_blocks(src_key, src_value, dst_key, dst_value, block_mapping, stream=None) -> None:
    """Copy block src of (src_key, src_value) onto block dst of (dst_key, dst_value) for each
    row of block_mapping (host int32 [n, 2]: numpy array or CPU tensor).  Either side may be
    host memory (pinned for asynchronous copies) or device memory."""
    import numpy as np
    lib = load()
    m = np.ascontiguousarray(np.asarray(block_mapping, dtype=np.int32).reshape(-1, 2))
    for t in (src_key, src_value, dst_key, dst_value):
        _need(t.is_contiguous(), "pools must be contiguous")
    _need(src_key.shape == src_value.shape and dst_key.shape == dst_value.shape and
          src_key.shape[1:] == dst_key.shape[1:], "pool shapes differ")
    _need(src_key.dtype == src_value.dtype == dst_key.dtype == dst_value.dtype, "dtype mismatch")
    nbs, hkv, bs, d = src_key.shape
    _check("pa_swap_blocks", lib.pa_swap_blocks(
        _ptr(src_key), _ptr(src_value), _ptr(dst_key), _ptr(dst_value),
        m.ctypes.data if m.size else None, m.shape[0], nbs, dst_key.shape[0], hkv, d, bs,
        _dtype_code(src_key, fp8_ok=True), _stream(stream)))


# --------------------------------------------------------------------------
# block manager (host object behind an opaque handle)
# --------------------------------------------------------------------------
def _np():
    import numpy as np
    return np


def _i64s(xs):
    np = _np()
    a = np.ascontiguousarray(np.asarray(xs, dtype=np.int64).reshape(-1))
    return a, (a.ctypes.data if a.size else None)


def pa_bm_create(num_blocks: int, num_host_blocks: int = 0, block_size: int = 16):
    h = ctypes.c_void_p()
    _check("pa_bm_create", load().pa_bm_create(num_blocks, num_host_blocks, block_size,
                                               ctypes.byref(h)))
    return h


def pa_bm_destroy(h) -> None:
    load().pa_bm_destroy(h)


def pa_bm_add_sequence(h, seq: int) -> None:
    _check("pa_bm_add_sequence", load().pa_bm_add_sequence(h, seq))


def pa_bm_fork(h, parent: int, child: int) -> None:
    _check("pa_bm_fork", load().pa_bm_fork(h, parent, child))


def pa_bm_share(h, src: int, dst: int, logical_blocks) -> None:
    np = _np()
    idx = np.ascontiguousarray(np.asarray(logical_blocks, dtype=np.int32).reshape(-1))
    _check("pa_bm_share", load().pa_bm_share(h, src, dst, idx.ctypes.data if idx.size else None,
                                             idx.size))


def pa_bm_free_sequence(h, seq: int) -> None:
    _check("pa_bm_free_sequence", load().pa_bm_free_sequence(h, seq))


def pa_bm_append_slots(h, seq: int, count: int):
    """int64 numpy array of the count reserved slots."""
    np = _np()
    slots = np.empty(max(count, 0), dtype=np.int64)
    _check("pa_bm_append_slots", load().pa_bm_append_slots(
        h, seq, count, slots.ctypes.data if slots.size else None))
    return slots


def pa_bm_append_batch(h, seqs, counts):
    """(slot_mapping int64 of the served sequences' slots, num_done, status)."""
    np = _np()
    s, sp = _i64s(seqs)
    c = np.ascontiguousarray(np.asarray(counts, dtype=np.int32).reshape(-1))
    _need(c.size == s.size, "one count per sequence")
    out = np.empty(int(c.astype(np.int64).sum()), dtype=np.int64)
    done = ctypes.c_int32(0)
    st = load().pa_bm_append_batch(h, sp, c.ctypes.data if c.size else None, s.size,
                                   out.ctypes.data if out.size else None, ctypes.byref(done))
    return out[:int(c[:done.value].astype(np.int64).sum())], done.value, st


def pa_bm_swap_out(h, seqs) -> None:
    s, sp = _i64s(seqs)
    _check("pa_bm_swap_out", load().pa_bm_swap_out(h, sp, s.size))


def pa_bm_swap_in(h, seqs) -> None:
    s, sp = _i64s(seqs)
    _check("pa_bm_swap_in", load().pa_bm_swap_in(h, sp, s.size))


def pa_bm_pending_moves(h):
    np = _np()
    c = np.zeros(3, dtype=np.int64)
    _check("pa_bm_pending_moves", load().pa_bm_pending_moves(h, c.ctypes.data))
    return tuple(int(x) for x in c)


def pa_bm_take_moves(h):
    """(copies, swap_out, swap_in): int32 numpy arrays [n, 2] of (src, dst)."""
    np = _np()
    bufs = [np.empty((n, 2), dtype=np.int32) for n in pa_bm_pending_moves(h)]
    ptrs = [b.ctypes.data if b.size else None for b in bufs]
    _check("pa_bm_take_moves", load().pa_bm_take_moves(h, *ptrs))
    return tuple(bufs)


def pa_bm_num_tokens(h, seq: int) -> int:
    n = ctypes.c_int64()
    _check("pa_bm_num_tokens", load().pa_bm_num_tokens(h, seq, ctypes.byref(n)))
    return n.value


def pa_bm_is_swapped(h, seq: int) -> bool:
    v = ctypes.c_int32()
    _check("pa_bm_is_swapped", load().pa_bm_is_swapped(h, seq, ctypes.byref(v)))
    return bool(v.value)


def pa_bm_block_table(h, seq: int):
    np = _np()
    n = ctypes.c_int32()
    load().pa_bm_block_table(h, seq, None, 0, ctypes.byref(n))
    t = np.empty(n.value, dtype=np.int32)
    _check("pa_bm_block_table", load().pa_bm_block_table(
        h, seq, t.ctypes.data if t.size else None, t.size, ctypes.byref(n)))
    return t


def pa_bm_num_free(h, host: bool = False) -> int:
    n = load().pa_bm_num_free(h, 1 if host else 0)
    if n < 0:
        raise PagedAttentionError("pa_bm_num_free", int(n))
    return int(n)


def pa_bm_build_batch(h, seqs, max_blocks_per_seq: int):
    """(block_tables int32 [S, MB], context_lens int32 [S], shared_prefix_blocks int32 [S])."""
    np = _np()
    s, sp = _i64s(seqs)
    tables = np.empty((s.size, max_blocks_per_seq), dtype=np.int32)
    lens = np.empty(s.size, dtype=np.int32)
    shared = np.empty(s.size, dtype=np.int32)
    _check("pa_bm_build_batch", load().pa_bm_build_batch(
        h, sp, s.size, max_blocks_per_seq, tables.ctypes.data, lens.ctypes.data,
        shared.ctypes.data))
    return tables, lens, shared


def pa_bm_prefix_groups(h, seqs):
    """(prefix_group int32 [S], group_blocks int32 [S], max_group_size) of a decode batch, for
    pa_decode_shared_prefix (group_blocks goes in as its shared_prefix_blocks)."""
    np = _np()
    s, sp = _i64s(seqs)
    group = np.empty(s.size, dtype=np.int32)
    blocks = np.empty(s.size, dtype=np.int32)
    largest = ctypes.c_int32()
    _check("pa_bm_prefix_groups", load().pa_bm_prefix_groups(
        h, sp, s.size, group.ctypes.data if s.size else None,
        blocks.ctypes.data if s.size else None, ctypes.byref(largest)))
    return group, blocks, int(largest.value)


def pa_bm_check(h) -> None:
    _check("pa_bm_check", load().pa_bm_check(h))


def _i32s(xs):
    np = _np()
    a = np.ascontiguousarray(np.asarray(xs, dtype=np.int32).reshape(-1))
    return a, (a.ctypes.data if a.size else None)


def pa_bm_prefix_keys(tokens, salt: int = 0):
    """uint64 numpy array: chained keys of the full 16-token blocks of tokens."""
    np = _np()
    t, tp = _i32s(tokens)
    keys = np.empty(t.size // 16, dtype=np.uint64)
    _check("pa_bm_prefix_keys", load().pa_bm_prefix_keys(
        tp, t.size, int(salt) & 0xFFFFFFFFFFFFFFFF, keys.ctypes.data if keys.size else None))
    return keys


def pa_bm_add_prompt(h, seq: int, tokens, salt: int = 0) -> int:
    t, tp = _i32s(tokens)
    n = ctypes.c_int64()
    _check("pa_bm_add_prompt", load().pa_bm_add_prompt(
        h, seq, tp, t.size, int(salt) & 0xFFFFFFFFFFFFFFFF, ctypes.byref(n)))
    return n.value


def pa_bm_append_tokens(h, seq: int, tokens):
    np = _np()
    t, tp = _i32s(tokens)
    slots = np.empty(t.size, dtype=np.int64)
    _check("pa_bm_append_tokens", load().pa_bm_append_tokens(
        h, seq, tp, t.size, slots.ctypes.data if slots.size else None))
    return slots


def pa_bm_num_cached_blocks(h) -> int:
    n = load().pa_bm_num_cached_blocks(h)
    if n < 0:
        raise PagedAttentionError("pa_bm_num_cached_blocks", int(n))
    return int(n)


class BlockManager:
    """The native block manager as an object (the pa_bm_* calls on one handle)."""

    def __init__(self, num_blocks: int, block_size: int = 16, num_host_blocks: int = 0):
        self.num_blocks = num_blocks
        self.num_host_blocks = num_host_blocks
        self.block_size = block_size
        self._h = pa_bm_create(num_blocks, num_host_blocks, block_size)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _lib is not None:
            _lib.pa_bm_destroy(h)

    def add_sequence(self, seq): pa_bm_add_sequence(self._h, seq)
    def fork(self, parent, child): pa_bm_fork(self._h, parent, child)
    def share(self, src, dst, logical_blocks): pa_bm_share(self._h, src, dst, logical_blocks)
    def free_sequence(self, seq): pa_bm_free_sequence(self._h, seq)
    def append_slots(self, seq, count): return pa_bm_append_slots(self._h, seq, count)
    def append_batch(self, seqs, counts): return pa_bm_append_batch(self._h, seqs, counts)
    def swap_out(self, seqs): pa_bm_swap_out(self._h, seqs)
    def swap_in(self, seqs): pa_bm_swap_in(self._h, seqs)
    def pending_moves(self): return pa_bm_pending_moves(self._h)
    def take_moves(self): return pa_bm_take_moves(self._h)
    def num_tokens(self, seq): return pa_bm_num_tokens(self._h, seq)
    def is_swapped(self, seq): return pa_bm_is_swapped(self._h, seq)
    def block_table(self, seq): return pa_bm_block_table(self._h, seq)
    def num_free(self, host=False): return pa_bm_num_free(self._h, host)
    def check_invariants(self): pa_bm_check(self._h)
    def add_prompt(self, seq, tokens, salt=0): return pa_bm_add_prompt(self._h, seq, tokens, salt)
    def append_tokens(self, seq, tokens): return pa_bm_append_tokens(self._h, seq, tokens)
    def num_cached_blocks(self): return pa_bm_num_cached_blocks(self._h)

    def build_batch(self, seqs, max_blocks_per_seq):
        return pa_bm_build_batch(self._h, seqs, max_blocks_per_seq)

    def prefix_groups(self, seqs):
        return pa_bm_prefix_groups(self._h, seqs)

    def shared_prefix_blocks(self, seq):
        n = max(1, len(self.block_table(seq)))
        return int(self.build_batch([seq], n)[2][0])
