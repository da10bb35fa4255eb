"""Shared pieces of the GPU parity tests: run the library on a workload, run
the oracle on the same inputs, compare with the stated tolerances."""
from __future__ import annotations

import sys
from typing import Optional, Sequence

import numpy as np

import oracle
from workloads import Workload
from workloads.device import DeviceWorkload, to_device, torch_to_storage

# Attention tolerances, elementwise on fp64 values: |gpu - ref| <= atol + rtol*|ref|.
# fp32 KV: 1e-5 + 1e-5|ref|.  bf16 KV with fp32 accumulation (output rounded to
# bf16): 4e-3 + 1e-2|ref|.
TOL = {"f32": (1e-5, 1e-5), "bf16": (4e-3, 1e-2)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_close(got, ref, dtype: str, what: str):
    atol, rtol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))   # NaN fails
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance "
            f"(max err {np.nanmax(err):.3e}); first at {idx.tolist()}: "
            f"got {[got[tuple(i)] for i in idx]}, ref {[ref[tuple(i)] for i in idx]}")
    return float(err.max()) if err.size else 0.0


def as_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


# --------------------------------------------------------------------------
# library calls (all through the C ABI)
# --------------------------------------------------------------------------
def lib():
    from paged_kv_cache_453_amd import lib as L
    L.load()
    return L


def gpu_scatter(dw: DeviceWorkload):
    lib().pa_reshape_and_cache(dw.new_k, dw.new_v, dw.k_cache, dw.v_cache, dw.slot_mapping)


def gpu_decode(dw: DeviceWorkload, partition_size: Optional[int] = None, group=None,
               use_shared_hint: bool = True):
    import torch
    L = lib()
    g = dw.decode if group is None else group
    w = dw.w
    ps = w.partition_size if partition_size is None else partition_size
    ws = None
    if ps > 0:
        nbytes = L.pa_decode_workspace_bytes(g.query.shape[0], w.num_heads, w.head_dim,
                                             g.max_context_len, ps)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=g.query.device)
    hint = getattr(g, "shared_prefix_blocks", None) if use_shared_hint else None
    L.pa_decode(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables, g.context_lens, w.scale,
                g.max_context_len, ps, ws, shared_prefix_blocks=hint)
    if ps > 0:
        L.pa_decode_splitk_reduce(g.out, ws, g.context_lens, g.max_context_len, ps)
    return ws


def gpu_prefill(dw: DeviceWorkload):
    g = dw.prefill
    w = dw.w
    lib().pa_prefill_chunk(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                           g.query_start_loc, g.context_lens, w.scale, g.max_query_len)


# --------------------------------------------------------------------------
# oracle on the same inputs
# --------------------------------------------------------------------------
def host_pools(w: Workload, scattered: bool):
    k, v = w.k_host, w.v_host
    if scattered and w.slot_mapping is not None:
        k, v = oracle.reshape_and_cache(k, v, w.new_k, w.new_v, w.host_slots())
    return k, v


def oracle_decode(w: Workload, seqs: Optional[Sequence[int]] = None, scattered: bool = True):
    k, v = host_pools(w, scattered)
    g = w.decode
    idx = np.arange(g.num_seqs) if seqs is None else np.asarray(seqs)
    return oracle.decode(g.query[idx], k, v, w.host_tables(g.block_tables[idx]),
                         g.context_lens[idx], w.scale, w.dtype)


def oracle_prefill(w: Workload):
    g = w.prefill
    return oracle.prefill(g.query, w.k_host, w.v_host, w.host_tables(g.block_tables),
                          g.query_start_loc, g.context_lens, w.scale, w.dtype)


__all__ = ["TOL", "say", "assert_close", "as_f64", "lib", "gpu_scatter", "gpu_decode",
           "gpu_prefill", "host_pools", "oracle_decode", "oracle_prefill", "to_device",
           "torch_to_storage"]
