"""Byte and flop accounting for the paged-attention workloads.

Algorithmic traffic only: what the method must move or compute, independent of
how a kernel does it.  The per-sequence KV size follows the intelliparadigm.com
article, section 2.1 (K and V, per head, per token, per layer: 2 x heads x
tokens x head_dim x bytes per element).
"""
from __future__ import annotations

import numpy as np


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, elem_bytes: int, num_layers: int = 1) -> int:
    """K plus V bytes one token occupies across num_layers layers."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def kv_cache_bytes(seq_len: int, num_kv_heads: int, head_dim: int, elem_bytes: int,
                   num_layers: int = 1) -> int:
    """KV cache bytes of one sequence of seq_len tokens."""
    return seq_len * kv_bytes_per_token(num_kv_heads, head_dim, elem_bytes, num_layers)


def decode_kv_bytes(context_lens, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes one decode step must read from the cache: every live K and V row once."""
    total = int(np.asarray(context_lens, dtype=np.int64).sum())
    return total * kv_bytes_per_token(num_kv_heads, head_dim, elem_bytes)


def unique_kv_bytes(block_tables, context_lens, num_kv_heads: int, head_dim: int,
                    elem_bytes: int, block_size: int = 16) -> int:
    """Bytes of distinct live rows when sequences share physical blocks."""
    rows = {}
    for s, L in enumerate(np.asarray(context_lens, dtype=np.int64)):
        nb = -(-int(L) // block_size)
        for j in range(nb):
            b = int(block_tables[s][j])
            rows[b] = max(rows.get(b, 0), min(block_size, int(L) - j * block_size))
    return sum(rows.values()) * kv_bytes_per_token(num_kv_heads, head_dim, elem_bytes)


def scatter_bytes(num_tokens: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """reshape_and_cache traffic: read new K and V once, write them once."""
    return 2 * kv_cache_bytes(num_tokens, num_kv_heads, head_dim, elem_bytes)


def prefill_pairs(query_start_loc, context_lens) -> int:
    """Number of (query, key) pairs a causal chunked prefill evaluates."""
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    total = 0
    for s, L in enumerate(np.asarray(context_lens, dtype=np.int64)):
        c = int(qsl[s + 1] - qsl[s])
        p = int(L) - c
        # query i (0-based) sees p + i + 1 keys
        total += c * (p + 1) + c * (c - 1) // 2
    return total


def prefill_flops(query_start_loc, context_lens, num_heads: int, head_dim: int) -> int:
    """q.k and p.v multiply-adds, 2 flops each, over every visible pair and head."""
    return 4 * head_dim * num_heads * prefill_pairs(query_start_loc, context_lens)
