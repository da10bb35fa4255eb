"""Seeded synthetic inputs for the paged-attention hot path.

This module draws inputs only: sequence lengths, shuffled physical block ids,
block tables, slot numbers for the newest tokens, and N(0, 1) query / key /
value contents.  It holds none of the attention arithmetic, so the CPU oracle
and the GPU path can both consume what it produces without sharing any of the
method's code.

The five workloads follow the shapes the pages reason about ("vLLM 基本原理",
section "PagedAttention": logical blocks of 16 tokens, physical blocks
scattered anywhere in memory, a per-sequence block table; intelliparadigm.com
article, section 3.1: pool layout [num_blocks, num_heads, block_size, head_dim]):

  0  tiny fp32 decode: 4 sequences, lengths {1, 7, 16, 33}, 2 heads, head_dim
     64, a pool of 16 blocks handed out by a seeded permutation, plus the
     scatter of each sequence's newest token;
  1  Llama-2-7B-shaped decode, bf16: 64 sequences, 32/32 heads, head_dim 128,
     lengths uniform in [128, 2048], pool of 16384 shuffled blocks;
  2  Llama-2-13B-shaped decode, bf16: 256 sequences, 40/40 heads, head_dim 128,
     lognormal lengths (median 1024, sigma 0.5) clipped to [16, 4096], pool of
     65536 blocks, scatter of the 256 newest tokens before attention;
  3  long-context GQA decode, bf16: 32 sequences, 32 query heads over 8 kv heads,
     lengths uniform in [8192, 32768], pool of 65536 blocks;
  4  mixed batch, bf16, 40/40 heads: 4 chunked-prefill sequences (512-token
     query chunks over prefixes of 0..3584 tokens) and 192 decode sequences
     (64 prompts x 3 samples sharing the physical blocks of a 2048-token
     prefix, 0..512 private tokens each), pool of 16384 blocks.

Only blocks that hold live tokens are materialised on the host.  Every other
row of the pool -- unused blocks and the tail rows of each partially filled
last block -- holds NaN, so a kernel that reads a row it should skip turns its
output into NaN.

bf16 data is carried as uint16 bit patterns (numpy has no bfloat16); fp32 -> bf16
uses round-to-nearest-even.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK_SIZE = 16
BF16_NAN = np.uint16(0x7FC0)
BASE_SEED = 453


# --------------------------------------------------------------------------
# storage helpers (input quantisation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = BF16_NAN
    return rounded


def storage_dtype(dtype: str):
    if dtype == "f32":
        return np.float32
    if dtype == "bf16":
        return np.uint16
    raise ValueError(f"unknown dtype {dtype!r}")


def nan_fill(dtype: str):
    return np.float32(np.nan) if dtype == "f32" else BF16_NAN


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_fill(out_storage: np.ndarray, dtype: str, seed_seq: np.random.SeedSequence,
                 rows_per_chunk: int) -> None:
    """Fill out_storage (leading axis = rows) with N(0,1) draws.

    Each chunk of rows has its own child seed, so the result does not depend on
    the number of threads.
    """
    n_rows = out_storage.shape[0]
    n_chunks = max(1, math.ceil(n_rows / rows_per_chunk))
    kids = seed_seq.spawn(n_chunks)

    def work(c: int) -> None:
        lo = c * rows_per_chunk
        hi = min(n_rows, lo + rows_per_chunk)
        if lo >= hi:
            return
        rng = np.random.default_rng(kids[c])
        vals = rng.standard_normal(size=out_storage[lo:hi].shape, dtype=np.float32)
        if dtype == "f32":
            out_storage[lo:hi] = vals
        else:
            out_storage[lo:hi] = f32_to_bf16_bits(vals)

    if n_chunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_chunks)))


def _normal(shape, dtype: str, seed_seq: np.random.SeedSequence) -> np.ndarray:
    out = np.empty(shape, dtype=storage_dtype(dtype))
    rows = max(1, (1 << 22) // max(1, int(np.prod(shape[1:])))) if len(shape) > 1 else 1 << 22
    _normal_fill(out, dtype, seed_seq, rows)
    return out


# --------------------------------------------------------------------------
# FP8 (E4M3) cache contents: random codes, drawn directly as bytes
# --------------------------------------------------------------------------
FP8_NAN_CODE = np.uint8(0x7F)


def fp8_codes(shape, seed_seq: np.random.SeedSequence, max_exp_field: int = 9) -> np.ndarray:
    """Random E4M3 codes: random sign, exponent field uniform in [0, max_exp_field],
    mantissa uniform in [0, 7] -- magnitudes up to 2^(max_exp_field-7) * 1.875,
    never NaN for max_exp_field < 15.  Chunked with child seeds, so the result
    does not depend on the number of threads."""
    out = np.empty(shape, dtype=np.uint8)
    flat = out.reshape(-1)
    n = flat.shape[0]
    chunk = 1 << 24
    kids = seed_seq.spawn(max(1, math.ceil(n / chunk)))

    def work(c: int) -> None:
        lo, hi = c * chunk, min(n, (c + 1) * chunk)
        rng = np.random.default_rng(kids[c])
        sign = rng.integers(0, 2, hi - lo, dtype=np.uint8) << 7
        e = rng.integers(0, max_exp_field + 1, hi - lo, dtype=np.uint8) << 3
        m = rng.integers(0, 8, hi - lo, dtype=np.uint8)
        flat[lo:hi] = sign | e | m

    if len(kids) == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(len(kids))))
    return out


def fp8_pools(w: "Workload", seed: int, max_exp_field: int = 9):
    """Host code pools shaped like w.k_host / w.v_host: random codes where w's
    pools hold data, the NaN code where they hold NaN (unused rows, slots a
    scatter fills), so the same rows stay poisoned.  max_exp_field = 14 spans
    every finite code (magnitudes up to 448)."""
    kids = np.random.SeedSequence(seed).spawn(2)
    out = []
    for src, kid in ((w.k_host, kids[0]), (w.v_host, kids[1])):
        codes = fp8_codes(src.shape, kid, max_exp_field)
        poison = np.isnan(src) if w.dtype == "f32" else (src == BF16_NAN)
        codes[poison] = FP8_NAN_CODE
        out.append(codes)
    return out[0], out[1]


# --------------------------------------------------------------------------
# next-token sampling inputs
# --------------------------------------------------------------------------
# (temperature, top_k, top_p): the pages' example first, then a spread
SAMPLER_PARAMS = [(0.7, 50, 0.9), (1.0, 0, 1.0), (0.5, 1, 1.0), (1.2, 1000, 0.8),
                  (0.9, 0, 0.5), (2.0, 32000, 0.99), (0.3, 20, 1.0), (1.0, 40, 0.95)]


def sampler_inputs(num_rows: int, vocab: int, seed: int):
    """Logits shaped like a language model's: N(0, 1.5) over the vocabulary plus
    a few strong candidates per row (N(6, 1.5) on 8 random tokens); per-row
    parameters cycling through SAMPLER_PARAMS; one uniform draw in [0, 1) per
    row.  Returns (logits fp32 [S, V], temperature f32, top_k i32, top_p f32, u f32)."""
    rng = np.random.default_rng(seed)
    logits = rng.normal(0.0, 1.5, (num_rows, vocab)).astype(np.float32)
    for r in range(num_rows):
        hot = rng.choice(vocab, size=min(8, vocab), replace=False)
        logits[r, hot] = rng.normal(6.0, 1.5, hot.size).astype(np.float32)
    par = [SAMPLER_PARAMS[r % len(SAMPLER_PARAMS)] for r in range(num_rows)]
    temperature = np.array([p[0] for p in par], dtype=np.float32)
    top_k = np.array([p[1] for p in par], dtype=np.int32)
    top_p = np.array([p[2] for p in par], dtype=np.float32)
    u = rng.random(num_rows).astype(np.float32)
    return logits, temperature, top_k, top_p, u


# --------------------------------------------------------------------------
# the workload record
# --------------------------------------------------------------------------
@dataclass
class SeqGroup:
    """Sequences that one kernel call handles (a decode batch or a prefill batch)."""

    context_lens: np.ndarray            # int32 [S]: tokens in the cache, newest included
    block_tables: np.ndarray            # int32 [S, MB]: physical ids, -1 past the last used entry
    query: np.ndarray                   # storage [S, Hq, D] (decode) or [Tq, Hq, D] (prefill)
    query_start_loc: Optional[np.ndarray] = None   # int32 [S+1] (prefill only)
    # int32 [S] (decode only): leading table entries whose physical blocks other
    # sequences of the batch also hold -- a cache hint the kernels may use
    shared_prefix_blocks: Optional[np.ndarray] = None
    # int32 [S] (decode only): first sequence of each sequence's sharing group
    # (itself when it shares with no earlier sequence of the batch)
    prefix_group: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def max_query_len(self) -> int:
        if self.query_start_loc is None:
            return 1
        return int(np.diff(self.query_start_loc).max()) if self.num_seqs else 0


@dataclass
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16" (query, cache and output share it)
    num_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int            # physical blocks in each pool on the device
    scale: np.float32          # softmax scale handed to the kernels (fp32)
    host_ids: np.ndarray       # int64 [U]: physical ids whose contents live on the host
    k_host: np.ndarray         # storage [U, Hkv, 16, D]: pool contents before any scatter
    v_host: np.ndarray
    decode: Optional[SeqGroup] = None
    prefill: Optional[SeqGroup] = None
    # scatter of new tokens (done before attention when present)
    slot_mapping: Optional[np.ndarray] = None   # int64 [T], physical slots
    new_k: Optional[np.ndarray] = None          # storage [T, Hkv, D]
    new_v: Optional[np.ndarray] = None
    partition_size: int = 0    # split-K partition length in tokens for decode (0 = single pass)
    block_size: int = BLOCK_SIZE
    meta: dict = field(default_factory=dict)

    # ---- relabelling to the compact host pool (for the CPU oracle) ----
    def _inverse(self) -> np.ndarray:
        inv = np.full(self.num_blocks, -1, dtype=np.int64)
        inv[self.host_ids] = np.arange(self.host_ids.shape[0], dtype=np.int64)
        return inv

    def host_tables(self, tables: np.ndarray) -> np.ndarray:
        """Block tables with physical ids replaced by rows of k_host / v_host."""
        inv = self._inverse()
        out = np.where(tables >= 0, inv[np.maximum(tables, 0)], -1)
        return out.astype(np.int64)

    def host_slots(self) -> np.ndarray:
        inv = self._inverse()
        s = self.slot_mapping.astype(np.int64)
        b = np.where(s >= 0, s // self.block_size, 0)
        o = np.where(s >= 0, s % self.block_size, 0)
        return np.where(s >= 0, inv[b] * self.block_size + o, -1)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------
def _blocks_needed(lens: np.ndarray) -> np.ndarray:
    return (lens.astype(np.int64) + BLOCK_SIZE - 1) // BLOCK_SIZE


def _tables_from_pool(lens: np.ndarray, pool_ids: np.ndarray, start: int, mb: Optional[int] = None):
    """Hand out consecutive ids from a shuffled pool; returns (tables, next_start)."""
    nb = _blocks_needed(lens)
    mb = int(nb.max()) if mb is None else mb
    mb = max(mb, 1)
    tables = np.full((lens.shape[0], mb), -1, dtype=np.int32)
    pos = start
    for s, n in enumerate(nb):
        tables[s, :n] = pool_ids[pos:pos + n]
        pos += n
    return tables, pos


def _live_rows(tables: np.ndarray, lens: np.ndarray):
    """(physical id, rows filled) for every block a set of sequences uses."""
    out = {}
    for s in range(lens.shape[0]):
        L = int(lens[s])
        nb = (L + BLOCK_SIZE - 1) // BLOCK_SIZE
        for j in range(nb):
            rows = min(BLOCK_SIZE, L - j * BLOCK_SIZE)
            bid = int(tables[s, j])
            out[bid] = max(out.get(bid, 0), rows)
    return out


def _materialise(live: dict, dtype: str, hkv: int, d: int, ss_k, ss_v, holes=()):
    """Host pool of the live blocks: N(0,1) rows, NaN in rows past each block's fill.

    holes: (physical id, row) pairs that must hold NaN (slots a later scatter fills).
    """
    ids = np.array(sorted(live), dtype=np.int64)
    shape = (ids.shape[0], hkv, BLOCK_SIZE, d)
    k = _normal(shape, dtype, ss_k)
    v = _normal(shape, dtype, ss_v)
    fill = nan_fill(dtype)
    rows = np.array([live[int(b)] for b in ids], dtype=np.int64)
    for i in np.nonzero(rows < BLOCK_SIZE)[0]:
        k[i, :, rows[i]:, :] = fill
        v[i, :, rows[i]:, :] = fill
    if holes:
        pos = {int(b): i for i, b in enumerate(ids)}
        for bid, r in holes:
            k[pos[bid], :, r, :] = fill
            v[pos[bid], :, r, :] = fill
    return ids, k, v


def _newest_slots(tables: np.ndarray, lens: np.ndarray) -> np.ndarray:
    last = lens.astype(np.int64) - 1
    bids = tables[np.arange(lens.shape[0]), last // BLOCK_SIZE].astype(np.int64)
    return bids * BLOCK_SIZE + last % BLOCK_SIZE


def _scale(d: int) -> np.float32:
    return np.float32(1.0 / math.sqrt(d))


# --------------------------------------------------------------------------
# decode-only workloads (configs 0-3 and their variants)
# --------------------------------------------------------------------------
def make_decode(name: str, seed: int, dtype: str, lens: np.ndarray, hq: int, hkv: int, d: int,
                num_blocks: int, with_scatter: bool, partition_size: int = 0,
                pool_perm: Optional[np.ndarray] = None, rng_kids=None) -> Workload:
    """A decode batch whose KV comes from a shuffled pool of num_blocks blocks."""
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(6) if rng_kids is None else rng_kids
    lens = np.asarray(lens, dtype=np.int32)
    if pool_perm is None:
        pool_perm = np.random.default_rng(kids[0]).permutation(num_blocks)
    need = int(_blocks_needed(lens).sum())
    if need > num_blocks:
        raise ValueError(f"{name}: {need} blocks needed, pool has {num_blocks}")
    tables, _ = _tables_from_pool(lens, pool_perm, 0)
    live = _live_rows(tables, lens)
    holes = ()
    slots = None
    if with_scatter:
        slots = _newest_slots(tables, lens)
        holes = [(int(s // BLOCK_SIZE), int(s % BLOCK_SIZE)) for s in slots]
    ids, k, v = _materialise(live, dtype, hkv, d, kids[1], kids[2], holes)
    query = _normal((lens.shape[0], hq, d), dtype, kids[3])
    w = Workload(name=name, dtype=dtype, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                 num_blocks=num_blocks, scale=_scale(d), host_ids=ids, k_host=k, v_host=v,
                 decode=SeqGroup(context_lens=lens, block_tables=tables, query=query),
                 partition_size=partition_size)
    if with_scatter:
        w.slot_mapping = slots.astype(np.int64)
        w.new_k = _normal((lens.shape[0], hkv, d), dtype, kids[4])
        w.new_v = _normal((lens.shape[0], hkv, d), dtype, kids[5])
    return w


def lens_config1(rng: np.random.Generator, n: int = 64) -> np.ndarray:
    return rng.integers(128, 2048, size=n, endpoint=True).astype(np.int32)


def lens_config2(rng: np.random.Generator, n: int = 256) -> np.ndarray:
    raw = rng.lognormal(mean=math.log(1024.0), sigma=0.5, size=n)
    return np.clip(np.rint(raw), 16, 4096).astype(np.int32)


def lens_config3(rng: np.random.Generator, n: int = 32) -> np.ndarray:
    return rng.integers(8192, 32768, size=n, endpoint=True).astype(np.int32)


def config0(seed: Optional[int] = None) -> Workload:
    seed = BASE_SEED + 0 if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(6)
    perm = np.random.default_rng(kids[0]).permutation(16)
    return make_decode("tiny-f32-decode", seed, "f32", np.array([1, 7, 16, 33]), 2, 2, 64, 16,
                       with_scatter=True, pool_perm=perm, rng_kids=kids)


def config1(seed: Optional[int] = None, dtype: str = "bf16", num_seqs: int = 64,
            partition_size: int = 0) -> Workload:
    seed = BASE_SEED + 1 if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(7)
    lens = lens_config1(np.random.default_rng(kids[6]), num_seqs)
    return make_decode(f"llama2-7b-decode-{dtype}-S{num_seqs}", seed, dtype, lens, 32, 32, 128,
                       16384, with_scatter=False, partition_size=partition_size, rng_kids=kids[:6])


def config2(seed: Optional[int] = None, dtype: str = "bf16", num_seqs: int = 256,
            partition_size: int = 512, num_blocks: int = 65536) -> Workload:
    seed = BASE_SEED + 2 if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(7)
    lens = lens_config2(np.random.default_rng(kids[6]), num_seqs)
    return make_decode(f"llama2-13b-decode-{dtype}-S{num_seqs}", seed, dtype, lens, 40, 40, 128,
                       num_blocks, with_scatter=True, partition_size=partition_size,
                       rng_kids=kids[:6])


def config3(seed: Optional[int] = None, dtype: str = "bf16", num_seqs: int = 32,
            partition_size: int = 512) -> Workload:
    seed = BASE_SEED + 3 if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(7)
    lens = lens_config3(np.random.default_rng(kids[6]), num_seqs)
    return make_decode(f"llama3-8b-gqa-long-decode-{dtype}-S{num_seqs}", seed, dtype, lens, 32, 8,
                       128, 65536, with_scatter=False, partition_size=partition_size,
                       rng_kids=kids[:6])


# --------------------------------------------------------------------------
# mixed prefill + decode (config 4)
# --------------------------------------------------------------------------
def config4(seed: Optional[int] = None, dtype: str = "bf16", num_prompts: int = 64,
            samples: int = 3, shared_prefix: int = 2048, max_private: int = 512,
            num_prefill: int = 4, chunk: int = 512, max_prefix: int = 3584,
            num_blocks: int = 16384, heads: int = 40, head_dim: int = 128,
            partition_size: int = 512, kv_heads: Optional[int] = None) -> Workload:
    """Chunked-prefill sequences plus decoders that share whole prefix blocks
    (heads query heads over kv_heads kv heads, by default as many).

    Sharing follows "vLLM 基本原理" (section "内存共享": samples of one prompt
    point at the same physical prompt blocks, private blocks only past the fork)
    and the xdnf.cn article (section 六.3: only whole blocks are shared).  The shared prefix
    is a whole number of blocks.
    """
    if shared_prefix % BLOCK_SIZE:
        raise ValueError("shared prefix must be whole blocks")
    seed = BASE_SEED + 4 if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(8)
    rng = np.random.default_rng(kids[0])
    perm = rng.permutation(num_blocks)
    pos = 0
    # decoders: prompt p owns shared_prefix/16 blocks; each sample adds private blocks
    n_dec = num_prompts * samples
    priv = rng.integers(0, max_private, size=n_dec, endpoint=True).astype(np.int64)
    dec_lens = (shared_prefix + priv).astype(np.int32)
    nsh = shared_prefix // BLOCK_SIZE
    mb_dec = int(_blocks_needed(dec_lens).max())
    dec_tables = np.full((n_dec, mb_dec), -1, dtype=np.int32)
    for p in range(num_prompts):
        shared_ids = perm[pos:pos + nsh]
        pos += nsh
        for smp in range(samples):
            s = p * samples + smp
            dec_tables[s, :nsh] = shared_ids
            n_priv = int(_blocks_needed(dec_lens[s:s + 1])[0]) - nsh
            dec_tables[s, nsh:nsh + n_priv] = perm[pos:pos + n_priv]
            pos += n_priv
    # prefill sequences: prefix P ~ U{0..max_prefix}, chunk of `chunk` new tokens
    prefix = rng.integers(0, max_prefix, size=num_prefill, endpoint=True).astype(np.int32)
    pre_lens = (prefix + chunk).astype(np.int32)
    pre_tables, pos = _tables_from_pool(pre_lens, perm, pos)
    if pos > num_blocks:
        raise ValueError("pool too small")
    live = _live_rows(dec_tables, dec_lens)
    live.update(_live_rows(pre_tables, pre_lens))
    hkv = heads if kv_heads is None else kv_heads
    if heads % hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    ids, k, v = _materialise(live, dtype, hkv, head_dim, kids[1], kids[2])
    dec_q = _normal((n_dec, heads, head_dim), dtype, kids[3])
    qsl = np.zeros(num_prefill + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(np.full(num_prefill, chunk, dtype=np.int32))
    pre_q = _normal((int(qsl[-1]), heads, head_dim), dtype, kids[4])
    w = Workload(name=f"mixed-prefill-decode-{dtype}", dtype=dtype, num_heads=heads,
                 num_kv_heads=hkv, head_dim=head_dim, num_blocks=num_blocks,
                 scale=_scale(head_dim), host_ids=ids, k_host=k, v_host=v,
                 decode=SeqGroup(context_lens=dec_lens, block_tables=dec_tables, query=dec_q,
                                 shared_prefix_blocks=np.full(n_dec, nsh, dtype=np.int32),
                                 prefix_group=(np.arange(n_dec) // samples * samples
                                               ).astype(np.int32)),
                 prefill=SeqGroup(context_lens=pre_lens, block_tables=pre_tables, query=pre_q,
                                  query_start_loc=qsl),
                 partition_size=partition_size)
    w.meta.update(num_prompts=num_prompts, samples=samples, shared_prefix=shared_prefix,
                  prefixes=prefix.tolist())
    return w


def make_prefill(name: str, seed: int, dtype: str, prefix_lens, chunk_lens, hq: int, hkv: int,
                 d: int, num_blocks: int) -> Workload:
    """A chunked-prefill batch: sequence s has prefix_lens[s] cached tokens and a
    chunk of chunk_lens[s] new query tokens whose K/V are already in the cache."""
    kids = np.random.SeedSequence(seed).spawn(5)
    prefix = np.asarray(prefix_lens, dtype=np.int32)
    chunks = np.asarray(chunk_lens, dtype=np.int32)
    lens = (prefix + chunks).astype(np.int32)
    perm = np.random.default_rng(kids[0]).permutation(num_blocks)
    tables, _ = _tables_from_pool(lens, perm, 0)
    live = _live_rows(tables, lens)
    ids, k, v = _materialise(live, dtype, hkv, d, kids[1], kids[2])
    qsl = np.zeros(lens.shape[0] + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(chunks)
    q = _normal((int(qsl[-1]), hq, d), dtype, kids[3])
    return Workload(name=name, dtype=dtype, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                    num_blocks=num_blocks, scale=_scale(d), host_ids=ids, k_host=k, v_host=v,
                    prefill=SeqGroup(context_lens=lens, block_tables=tables, query=q,
                                     query_start_loc=qsl))


CONFIGS = {0: config0, 1: config1, 2: config2, 3: config3, 4: config4}


def make_config(k: int, **kw) -> Workload:
    return CONFIGS[k](**kw)


# --------------------------------------------------------------------------
# relabelling helpers used by invariance tests (pure data movement)
# --------------------------------------------------------------------------
def permute_block_ids(w: Workload, seed: int) -> Workload:
    """Same logical contents under a random relabelling of physical block ids."""
    rng = np.random.default_rng(seed)
    pi = rng.permutation(w.num_blocks).astype(np.int64)

    def relabel(t):
        return np.where(t >= 0, pi[np.maximum(t, 0)], -1).astype(t.dtype)

    import copy
    w2 = copy.copy(w)
    w2.host_ids = pi[w.host_ids]
    order = np.argsort(w2.host_ids)
    w2.host_ids = w2.host_ids[order]
    w2.k_host = w.k_host[order]
    w2.v_host = w.v_host[order]
    for name in ("decode", "prefill"):
        g = getattr(w, name)
        if g is not None:
            setattr(w2, name, SeqGroup(g.context_lens, relabel(g.block_tables), g.query,
                                       g.query_start_loc, g.shared_prefix_blocks,
                                       g.prefix_group))
    if w.slot_mapping is not None:
        s = w.slot_mapping
        w2.slot_mapping = np.where(s >= 0, pi[np.maximum(s, 0) // BLOCK_SIZE] * BLOCK_SIZE
                                   + np.maximum(s, 0) % BLOCK_SIZE, -1).astype(np.int64)
    return w2


def unshare_blocks(w: Workload) -> Workload:
    """Give every decode sequence private copies of blocks it shares with others."""
    import copy
    g = w.decode
    tables = g.block_tables.copy()
    used = set(int(x) for x in w.host_ids)
    free = [b for b in range(w.num_blocks) if b not in used]
    if w.prefill is not None:
        used |= set(int(x) for x in w.prefill.block_tables.ravel() if x >= 0)
        free = [b for b in range(w.num_blocks) if b not in used]
    seen = set()
    pos_of = {int(b): i for i, b in enumerate(w.host_ids)}
    new_ids, new_k, new_v = [], [], []
    fi = 0
    for s in range(g.num_seqs):
        nb = (int(g.context_lens[s]) + BLOCK_SIZE - 1) // BLOCK_SIZE
        for j in range(nb):
            b = int(tables[s, j])
            if b in seen:
                nbid = free[fi]
                fi += 1
                tables[s, j] = nbid
                new_ids.append(nbid)
                new_k.append(w.k_host[pos_of[b]])
                new_v.append(w.v_host[pos_of[b]])
            else:
                seen.add(b)
    w2 = copy.copy(w)
    if new_ids:
        ids = np.concatenate([w.host_ids, np.array(new_ids, dtype=np.int64)])
        k = np.concatenate([w.k_host, np.stack(new_k)])
        v = np.concatenate([w.v_host, np.stack(new_v)])
        order = np.argsort(ids)
        w2.host_ids, w2.k_host, w2.v_host = ids[order], k[order], v[order]
    w2.decode = SeqGroup(g.context_lens, tables, g.query, g.query_start_loc)
    return w2
