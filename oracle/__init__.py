"""fp64 CPU oracle for paged attention, and the reference block manager.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the package smoke check and by
the benchmark's CPU-baseline leg, never by the product path.
"""
from .paged_attention import (to_f64, reshape_and_cache, gather, attend, decode,
                              decode_partials, merge_partials, prefill)
from .block_manager import (BlockManager, OutOfBlocks, copy_blocks, swap_blocks, fnv1a64,
                            block_key, prefix_keys)
from . import kv_fp8, sampler

__all__ = ["to_f64", "reshape_and_cache", "gather", "attend", "decode", "decode_partials",
           "merge_partials", "prefill", "BlockManager", "OutOfBlocks", "copy_blocks",
           "swap_blocks", "fnv1a64", "block_key", "prefix_keys", "kv_fp8", "sampler"]
