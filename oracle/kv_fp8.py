"""Plain reference of an FP8 (OCP E4M3) KV cache with one scale per tensor.

TEST INFRASTRUCTURE ONLY: imported by tests/, the package smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the GPU kernels.

The pages suggest choosing a lower precision for attention, fp8 among them
(intelliparadigm.com article, section 7.1).  Read here as: the cache stores
K and V as 8-bit floats, which halves the bytes that decode must stream
(decode is bound by memory, xdnf.cn article, section 六.5), and attention runs
on the values those codes stand for.

Format (OCP 8-bit floating point, E4M3): 1 sign bit, 4 exponent bits with bias
7, 3 mantissa bits.  Exponent field 0 holds subnormals m * 2^-9; fields 1..15
hold 2^(e-7) * (1 + m/8), except field 15 with mantissa 7, which is NaN.
There are no infinities; the largest finite magnitude is 448.

Readings where the pages are silent (listed with the design notes):
* Encoding rounds to the nearest representable value, ties to the even code
  (even mantissa); magnitudes above 448, infinities included, saturate to
  448; NaN encodes as 0x7F.  The sign is kept, so -0.0 and negative values
  that round to zero give 0x80.
* A stored code is encode(float32(x * float32(1 / scale))): the reciprocal is
  taken once in float32 and the product is rounded to float32 before encoding,
  so the quantised integer is decided in float32 on both sides.
* A code stands for decode(code) * scale.  Attention over an FP8 cache is the
  plain definition applied to those values (paged_attention.attend).
"""
from __future__ import annotations

import numpy as np

from . import paged_attention as pa

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def decode_codes(codes) -> np.ndarray:
    """Exact float64 values of E4M3 codes (uint8), from the format definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m * 2.0 ** -9
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


# the 127 non-negative finite values, in code order (code i -> value i)
_POS = decode_codes(np.arange(0x7F, dtype=np.uint8))


def encode_values(x) -> np.ndarray:
    """Nearest E4M3 code for each float32 value x (ties to even, saturating)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    sat = np.minimum(a, MAX_FINITE)
    lo = np.searchsorted(_POS, sat, side="right") - 1          # _POS[lo] <= sat
    hi = np.minimum(lo + 1, len(_POS) - 1)
    d_lo = sat - _POS[lo]
    d_hi = _POS[hi] - sat
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(NAN_CODE), code).astype(np.uint8)


def quantize(x, scale: float) -> np.ndarray:
    """Codes stored for float32 values x with the given per-tensor scale."""
    inv = np.float32(1.0) / np.float32(scale)
    q = np.asarray(x, dtype=np.float32) * inv                  # float32 product
    return encode_values(q)


def values(codes, scale: float) -> np.ndarray:
    """float64 values the codes stand for."""
    return decode_codes(codes) * float(np.float32(scale))


def reshape_and_cache(k_pool, v_pool, key, value, slot_mapping, key_dtype: str,
                      k_scale: float, v_scale: float, block_size: int = 16):
    """Pools (uint8 codes) after quantising token i's K/V into slot_mapping[i].

    key/value are storage arrays of key_dtype ("f32" or "bf16" bit patterns).
    """
    k32 = pa.to_f64(key, key_dtype).astype(np.float32)   # exact: bf16 and fp32 fit fp32
    v32 = pa.to_f64(value, key_dtype).astype(np.float32)
    return pa.reshape_and_cache(k_pool, v_pool, quantize(k32, k_scale), quantize(v32, v_scale),
                                slot_mapping, block_size)


def decode(query, k_pool, v_pool, block_tables, context_lens, scale, k_scale, v_scale,
           query_dtype: str, block_size: int = 16) -> np.ndarray:
    """One query token per sequence over an FP8 cache: the plain attention
    definition on the values the codes stand for."""
    S, hq, d = query.shape
    hkv = k_pool.shape[1]
    g = hq // hkv
    q64 = pa.to_f64(query, query_dtype)
    out = np.zeros((S, hq, d), dtype=np.float64)
    for s in range(S):
        L = int(context_lens[s])
        if L == 0:
            continue
        ks = values(pa.gather(k_pool, block_tables[s], L, block_size), k_scale)
        vs = values(pa.gather(v_pool, block_tables[s], L, block_size), v_scale)
        for h in range(hq):
            kh = h // g
            out[s, h] = pa.attend(q64[s, h][None, :], ks[:, kh, :], vs[:, kh, :], scale)[0]
    return out


def prefill(query, k_pool, v_pool, block_tables, query_start_loc, context_lens, scale, k_scale,
            v_scale, query_dtype: str, block_size: int = 16) -> np.ndarray:
    """Causal chunked prefill over an FP8 cache (xdnf.cn article, section 六.4):
    sequence s's chunk of C new queries sits at the last C of its L cached
    positions, and query i sees keys 0 .. L - C + i -- the plain definition on
    the values the codes stand for.  Returns float64 [Tq, Hq, D]."""
    tq, hq, d = query.shape
    hkv = k_pool.shape[1]
    g = hq // hkv
    q64 = pa.to_f64(query, query_dtype)
    out = np.zeros((tq, hq, d), dtype=np.float64)
    for s in range(len(context_lens)):
        a, b = int(query_start_loc[s]), int(query_start_loc[s + 1])
        C, L = b - a, int(context_lens[s])
        if C == 0:
            continue
        if C > L:
            raise ValueError("chunk longer than the cached context")
        ks = values(pa.gather(k_pool, block_tables[s], L, block_size), k_scale)
        vs = values(pa.gather(v_pool, block_tables[s], L, block_size), v_scale)
        pos = (L - C) + np.arange(C)
        visible = np.arange(L)[None, :] <= pos[:, None]
        for h in range(hq):
            kh = h // g
            out[a:b, h] = pa.attend(q64[a:b, h, :], ks[:, kh, :], vs[:, kh, :], scale, visible)
    return out
