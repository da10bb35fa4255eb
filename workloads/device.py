"""Place a seeded workload in GPU memory (torch is used for allocation and copies only).

The pools are allocated at their full physical size.  Every row starts as NaN
and the host-held live blocks are copied to their physical ids, so unused
blocks and the unused tail rows of partly filled blocks stay NaN.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .generate import Workload


def torch_dtype(dtype: str):
    import torch
    return torch.float32 if dtype == "f32" else torch.bfloat16


def host_to_torch(arr: np.ndarray, dtype: str, device):
    """Storage array (fp32 or bf16 bits) -> torch tensor of the right dtype on device."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    bits = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device)
    return bits.view(torch.bfloat16)


def torch_to_storage(t, dtype: str) -> np.ndarray:
    """Device tensor -> host storage array (fp32 values or bf16 bit patterns)."""
    import torch
    t = t.detach()
    if dtype == "f32":
        return t.cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def fill_nan(t, dtype: str):
    import torch
    if dtype == "f32":
        t.fill_(float("nan"))
    else:
        t.view(torch.int16).fill_(0x7FC0)


@dataclass
class DeviceGroup:
    context_lens: object
    block_tables: object
    query: object
    out: object
    query_start_loc: Optional[object] = None
    max_context_len: int = 0
    max_query_len: int = 0
    shared_prefix_blocks: Optional[object] = None
    prefix_group: Optional[object] = None


@dataclass
class DeviceWorkload:
    w: Workload
    k_cache: object
    v_cache: object
    decode: Optional[DeviceGroup] = None
    prefill: Optional[DeviceGroup] = None
    slot_mapping: Optional[object] = None
    new_k: Optional[object] = None
    new_v: Optional[object] = None
    workspace: Optional[object] = None


def upload_pools(w: Workload, device="cuda"):
    import torch
    td = torch_dtype(w.dtype)
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    k = torch.empty(shape, dtype=td, device=device)
    v = torch.empty(shape, dtype=td, device=device)
    fill_nan(k, w.dtype)
    fill_nan(v, w.dtype)
    ids = torch.from_numpy(w.host_ids).to(device)
    # copy in slices to bound the staging memory
    step = 4096
    for lo in range(0, w.host_ids.shape[0], step):
        hi = min(w.host_ids.shape[0], lo + step)
        k[ids[lo:hi]] = host_to_torch(w.k_host[lo:hi], w.dtype, device)
        v[ids[lo:hi]] = host_to_torch(w.v_host[lo:hi], w.dtype, device)
    return k, v


def upload_fp8_pools(w: Workload, k_codes: np.ndarray, v_codes: np.ndarray, device="cuda"):
    """uint8 device pools [num_blocks, Hkv, 16, D]: the NaN code everywhere, the
    host code rows at w.host_ids."""
    import torch
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    k = torch.full(shape, 0x7F, dtype=torch.uint8, device=device)
    v = torch.full(shape, 0x7F, dtype=torch.uint8, device=device)
    ids = torch.from_numpy(w.host_ids).to(device)
    step = 4096
    for lo in range(0, w.host_ids.shape[0], step):
        hi = min(w.host_ids.shape[0], lo + step)
        k[ids[lo:hi]] = torch.from_numpy(np.ascontiguousarray(k_codes[lo:hi])).to(device)
        v[ids[lo:hi]] = torch.from_numpy(np.ascontiguousarray(v_codes[lo:hi])).to(device)
    return k, v


def _group(g, dtype, hq, d, device):
    import torch
    q = host_to_torch(g.query, dtype, device)
    out = torch.empty_like(q)
    fill_nan(out, dtype)
    qsl = None
    if g.query_start_loc is not None:
        qsl = torch.from_numpy(g.query_start_loc.astype(np.int32)).to(device)
    shared = None
    if g.shared_prefix_blocks is not None:
        shared = torch.from_numpy(g.shared_prefix_blocks.astype(np.int32)).to(device)
    group = None
    if g.prefix_group is not None:
        group = torch.from_numpy(g.prefix_group.astype(np.int32)).to(device)
    return DeviceGroup(
        shared_prefix_blocks=shared, prefix_group=group,
        context_lens=torch.from_numpy(g.context_lens.astype(np.int32)).to(device),
        block_tables=torch.from_numpy(g.block_tables.astype(np.int32)).to(device),
        query=q, out=out, query_start_loc=qsl, max_context_len=g.max_context_len,
        max_query_len=g.max_query_len)


def to_device(w: Workload, device="cuda", workspace_bytes: Optional[int] = None,
              pools: bool = True) -> DeviceWorkload:
    """Upload a workload; pools=False leaves the caches out (k_cache / v_cache None)."""
    import torch
    k, v = upload_pools(w, device) if pools else (None, None)
    dw = DeviceWorkload(w=w, k_cache=k, v_cache=v)
    if w.decode is not None:
        dw.decode = _group(w.decode, w.dtype, w.num_heads, w.head_dim, device)
    if w.prefill is not None:
        dw.prefill = _group(w.prefill, w.dtype, w.num_heads, w.head_dim, device)
    if w.slot_mapping is not None:
        dw.slot_mapping = torch.from_numpy(w.slot_mapping.astype(np.int64)).to(device)
        dw.new_k = host_to_torch(w.new_k, w.dtype, device)
        dw.new_v = host_to_torch(w.new_v, w.dtype, device)
    if workspace_bytes:
        dw.workspace = torch.empty(int(workspace_bytes), dtype=torch.uint8, device=device)
    return dw
