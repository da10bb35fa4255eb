"""Plain, slow, fp64 CPU oracle for paged attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the tests, the package's smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the GPU kernels
and imports nothing from the product package.

What it computes, and the passages it follows (page titles as printed):

* Attention as a weighted lookup -- each query scores every context token and
  mixes their values by those weights ("vLLM 基本原理", section "Transformer 和
  Attention").  Written out as the textbook definition
  out = softmax(scale * q K^T) V with scale = 1/sqrt(head_dim).
* The KV cache keeps every past token's K and V so a new token attends to all
  of them ("vLLM 基本原理", section "什么是 KV Cache").
* Paging: a sequence is cut into logical blocks of block_size tokens, stored in
  physical blocks anywhere in memory, and a block table maps logical to
  physical ids ("vLLM 基本原理", section "PagedAttention", items 1-3).  The pool
  layout is [num_blocks, num_heads, block_size, head_dim] and a kernel finds a
  block as block_tables[seq][logical_block] (intelliparadigm.com article,
  section 3.1 "内存布局的重构").  Token t of a sequence lives in logical block t // block_size
  at row t % block_size.
* Only the last block of a sequence may be partly filled ("vLLM 基本原理",
  "按需分配"); rows past the sequence length are never read.
* Prefix blocks can be shared between sequences ("vLLM 基本原理", "内存共享";
  xdnf.cn article, section 六.3: whole blocks only).  Sharing is just the same
  physical id in several tables, so the oracle needs nothing special for it.
* Chunked prefill splits one prompt's prefill over several rounds (xdnf.cn
  article, section 六.4: a 12-token prompt in chunks of 4 under a 6-token budget).  A
  chunk's queries are the last C positions of the sequence and see every key
  up to their own position (causal language-model attention).
* Split-K over context partitions with a log-sum-exp merge is exact in real
  arithmetic; the oracle computes the per-partition results and merges them
  the plain way.

bf16 values arrive as uint16 bit patterns and are decoded exactly.  All
arithmetic is float64.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# storage decoding
# --------------------------------------------------------------------------
def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of fp32 storage or bf16 bit patterns."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# reshape_and_cache: write each new token's K/V into its slot
# --------------------------------------------------------------------------
def reshape_and_cache(k_pool, v_pool, key, value, slot_mapping, block_size=16):
    """Return copies of the pools with token i's K/V stored at slot_mapping[i].

    A slot names physical block slot // block_size, row slot % block_size.
    Negative slots are padding and write nothing.  Values are copied bit for
    bit (storage arrays, no conversion).
    """
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    for i in range(len(slot_mapping)):
        slot = int(slot_mapping[i])
        if slot < 0:
            continue
        blk, row = divmod(slot, block_size)
        kp[blk, :, row, :] = key[i]
        vp[blk, :, row, :] = value[i]
    return kp, vp


# --------------------------------------------------------------------------
# gather: a sequence's paged KV as one contiguous [L, Hkv, D] array
# --------------------------------------------------------------------------
def gather(pool, table_row, length, block_size=16):
    """Tokens 0..length-1 of one sequence, read through its block table."""
    t = np.arange(int(length))
    phys = np.asarray(table_row)[t // block_size].astype(np.int64)
    if length and phys.min() < 0:
        raise ValueError("block table entry missing for a live token")
    return pool[phys, :, t % block_size, :]


# --------------------------------------------------------------------------
# the attention definition
# --------------------------------------------------------------------------
def attend(q, k, v, scale, visible=None):
    """softmax(scale * q k^T) v for rows of q, in float64.

    q: [n, D]; k, v: [L, D]; visible: optional bool [n, L] of keys each row sees.
    A row that sees no key returns zeros.
    """
    z = float(scale) * (q @ k.T)
    if visible is not None:
        z = np.where(visible, z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    w = np.exp(z - m)
    den = w.sum(axis=1, keepdims=True)
    out = (w @ v) / np.where(den > 0, den, 1.0)
    return np.where(empty, 0.0, out)


def decode(query, k_pool, v_pool, block_tables, context_lens, scale, dtype, block_size=16):
    """One query token per sequence over its whole cached context.

    query [S, Hq, D]; pools [NB, Hkv, bs, D]; query head h reads kv head
    h // (Hq // Hkv).  Returns float64 [S, Hq, D]; a sequence with no cached
    token returns zeros.
    """
    S, hq, d = query.shape
    hkv = k_pool.shape[1]
    g = hq // hkv
    q64 = to_f64(query, dtype)
    out = np.zeros((S, hq, d), dtype=np.float64)
    for s in range(S):
        L = int(context_lens[s])
        if L == 0:
            continue
        ks = to_f64(gather(k_pool, block_tables[s], L, block_size), dtype)
        vs = to_f64(gather(v_pool, block_tables[s], L, block_size), dtype)
        for h in range(hq):
            kh = h // g
            out[s, h] = attend(q64[s, h][None, :], ks[:, kh, :], vs[:, kh, :], scale)[0]
    return out


def decode_partials(query, k_pool, v_pool, block_tables, context_lens, scale, dtype,
                    partition_size, block_size=16):
    """Per-partition results of decode.

    Partition p of sequence s covers tokens [p*P, min((p+1)*P, L)).  Returns
    o [S, Hq, Pmax, D] (the partition's normalised output), lse [S, Hq, Pmax]
    (natural-log log-sum-exp of its scaled scores) and nparts [S].  Unused
    entries are NaN / -inf.
    """
    S, hq, d = query.shape
    hkv = k_pool.shape[1]
    g = hq // hkv
    nparts = np.array([-(-int(L) // partition_size) for L in context_lens], dtype=np.int64)
    pmax = int(max(1, nparts.max(initial=1)))
    o = np.full((S, hq, pmax, d), np.nan)
    lse = np.full((S, hq, pmax), -np.inf)
    q64 = to_f64(query, dtype)
    for s in range(S):
        L = int(context_lens[s])
        if L == 0:
            continue
        ks = to_f64(gather(k_pool, block_tables[s], L, block_size), dtype)
        vs = to_f64(gather(v_pool, block_tables[s], L, block_size), dtype)
        for p in range(int(nparts[s])):
            lo, hi = p * partition_size, min(L, (p + 1) * partition_size)
            for h in range(hq):
                kh = h // g
                z = float(scale) * (ks[lo:hi, kh, :] @ q64[s, h])
                m = z.max()
                w = np.exp(z - m)
                o[s, h, p] = (w @ vs[lo:hi, kh, :]) / w.sum()
                lse[s, h, p] = m + np.log(w.sum())
    return o, lse, nparts


def merge_partials(o, lse, nparts):
    """Combine partition results: weights exp(lse_p - max lse), normalised."""
    S, hq, _, d = o.shape
    out = np.zeros((S, hq, d))
    for s in range(S):
        n = int(nparts[s])
        if n == 0:
            continue
        l = lse[s, :, :n]
        m = l.max(axis=1, keepdims=True)
        w = np.exp(l - m)
        out[s] = np.einsum("hp,hpd->hd", w, o[s, :, :n, :]) / w.sum(axis=1)[:, None]
    return out


def prefill(query, k_pool, v_pool, block_tables, query_start_loc, context_lens, scale, dtype,
            block_size=16):
    """Causal attention of a chunk of new tokens over the paged cache.

    Sequence s owns query rows query_start_loc[s]..query_start_loc[s+1]-1
    (C of them); its cache holds L = context_lens[s] tokens including the
    chunk, so query i sits at position L - C + i and sees keys 0..L - C + i.
    Returns float64 [Tq, Hq, D].
    """
    tq, hq, d = query.shape
    hkv = k_pool.shape[1]
    g = hq // hkv
    q64 = to_f64(query, dtype)
    out = np.zeros((tq, hq, d))
    for s in range(len(context_lens)):
        a, b = int(query_start_loc[s]), int(query_start_loc[s + 1])
        C, L = b - a, int(context_lens[s])
        if C == 0:
            continue
        if C > L:
            raise ValueError("chunk longer than the cached context")
        ks = to_f64(gather(k_pool, block_tables[s], L, block_size), dtype)
        vs = to_f64(gather(v_pool, block_tables[s], L, block_size), dtype)
        pos = (L - C) + np.arange(C)
        visible = np.arange(L)[None, :] <= pos[:, None]
        for h in range(hq):
            kh = h // g
            out[a:b, h] = attend(q64[a:b, h, :], ks[:, kh, :], vs[:, kh, :], scale, visible)
    return out
