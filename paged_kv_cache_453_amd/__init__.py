"""Paged attention for AMD Instinct MI355X (gfx950).

The compute lives in libpa.so (hand-written HIP kernels and the native block
manager behind a C ABI declared in include/pa.h); `lib` is its thin ctypes
binding.
"""
from . import lib
from .lib import (pa_decode, pa_decode_splitk_reduce, pa_decode_workspace_bytes,
                  pa_decode_no_alloc, pa_decode_no_alloc_scratch_bytes,
                  pa_prefill_chunk, pa_reshape_and_cache, pa_reshape_and_cache_fp8,
                  pa_decode_fp8, pa_prefill_chunk_fp8, pa_decode_shared_prefix,
                  pa_decode_fp8_shared_prefix, pa_prefill_workspace_bytes,
                  pa_prefill_chunk_split, pa_prefill_chunk_fp8_split, pa_sample, pa_copy_blocks, pa_swap_blocks,
                  pa_stream_read, pa_stream_read_sink_words,
                  pa_bm_create, pa_bm_destroy, pa_bm_add_sequence, pa_bm_fork, pa_bm_share,
                  pa_bm_free_sequence, pa_bm_append_slots, pa_bm_append_batch, pa_bm_swap_out,
                  pa_bm_swap_in, pa_bm_pending_moves, pa_bm_take_moves, pa_bm_num_tokens,
                  pa_bm_is_swapped, pa_bm_block_table, pa_bm_num_free, pa_bm_build_batch,
                  pa_bm_check, pa_bm_prefix_groups, pa_bm_prefix_keys, pa_bm_add_prompt, pa_bm_append_tokens,
                  pa_bm_num_cached_blocks, BlockManager, Busy, OutOfBlocks, PagedAttentionError,
                  SequenceError, ShapeError)

__all__ = ["lib", "pa_decode", "pa_decode_splitk_reduce", "pa_decode_workspace_bytes",
           "pa_decode_no_alloc", "pa_decode_no_alloc_scratch_bytes",
           "pa_prefill_chunk", "pa_reshape_and_cache", "pa_reshape_and_cache_fp8",
           "pa_decode_fp8", "pa_prefill_chunk_fp8", "pa_decode_shared_prefix",
           "pa_decode_fp8_shared_prefix", "pa_prefill_workspace_bytes",
           "pa_prefill_chunk_split", "pa_prefill_chunk_fp8_split", "pa_sample", "pa_copy_blocks", "pa_swap_blocks",
           "pa_stream_read", "pa_stream_read_sink_words",
           "pa_bm_create", "pa_bm_destroy", "pa_bm_add_sequence", "pa_bm_fork", "pa_bm_share",
           "pa_bm_free_sequence", "pa_bm_append_slots", "pa_bm_append_batch", "pa_bm_swap_out",
           "pa_bm_swap_in", "pa_bm_pending_moves", "pa_bm_take_moves", "pa_bm_num_tokens",
           "pa_bm_is_swapped", "pa_bm_block_table", "pa_bm_num_free", "pa_bm_build_batch",
           "pa_bm_check", "pa_bm_prefix_groups", "pa_bm_prefix_keys", "pa_bm_add_prompt", "pa_bm_append_tokens",
           "pa_bm_num_cached_blocks", "BlockManager", "Busy", "OutOfBlocks", "PagedAttentionError",
           "SequenceError", "ShapeError"]
