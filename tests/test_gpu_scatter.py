"""reshape_and_cache on the GPU: bit-exact against the oracle's slot copy."""
import numpy as np
import pytest

import oracle
from workloads import config0, config2
from workloads.device import fill_nan, host_to_torch, to_device, torch_to_storage

from pa_harness import gpu_scatter, lib, say

pytestmark = pytest.mark.gpu


def full_host_pool(w, k_host):
    """The whole physical pool as the device holds it: NaN rows + live blocks."""
    shape = (w.num_blocks, w.num_kv_heads, 16, w.head_dim)
    if w.dtype == "f32":
        pool = np.full(shape, np.float32(np.nan), dtype=np.float32)
    else:
        pool = np.full(shape, 0x7FC0, dtype=np.uint16)
    pool[w.host_ids] = k_host
    return pool


def bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def test_scatter_tiny_fp32_whole_pool_bit_exact(gpu):
    import torch
    say("scatter config0")
    w = config0()
    dw = to_device(w)
    gpu_scatter(dw)
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache(full_host_pool(w, w.k_host), full_host_pool(w, w.v_host),
                                      w.new_k, w.new_v, w.slot_mapping)
    gk = torch_to_storage(dw.k_cache, w.dtype)
    gv = torch_to_storage(dw.v_cache, w.dtype)
    assert np.array_equal(bits(gk), bits(ek))
    assert np.array_equal(bits(gv), bits(ev))


def test_scatter_padding_and_out_of_pool_slots_write_nothing(gpu):
    import torch
    w = config0()
    dw = to_device(w)
    before_k = dw.k_cache.clone()
    slots = w.slot_mapping.copy()
    slots[0] = -1
    slots[2] = w.num_blocks * 16 + 5     # past the pool: skipped by the kernel
    dw.slot_mapping = torch.from_numpy(slots).cuda()
    gpu_scatter(dw)
    torch.cuda.synchronize()
    keep = np.array([s >= 0 and s < w.num_blocks * 16 for s in slots])
    ek, _ = oracle.reshape_and_cache(full_host_pool(w, w.k_host), full_host_pool(w, w.v_host),
                                     w.new_k[keep], w.new_v[keep], slots[keep])
    assert np.array_equal(bits(torch_to_storage(dw.k_cache, w.dtype)), bits(ek))
    assert not torch.equal(before_k.view(torch.int32), dw.k_cache.view(torch.int32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("stride_extra", [0, 8, 1])
def test_scatter_strided_and_unaligned_sources(gpu, dtype, stride_extra):
    """Token stride larger than one token (a slice of a fused qkv buffer), and
    an odd stride that forces the element-wise path."""
    import torch
    rng = np.random.default_rng(5)
    nb, hkv, d, t = 8, 3, 64, 20
    w_dtype = torch.float32 if dtype == "f32" else torch.bfloat16
    kc = torch.zeros((nb, hkv, 16, d), dtype=w_dtype, device="cuda")
    vc = torch.zeros_like(kc)
    stride = hkv * d + stride_extra
    flat_k = torch.randn(t * stride + 8, dtype=w_dtype, device="cuda")
    flat_v = torch.randn(t * stride + 8, dtype=w_dtype, device="cuda")
    key = flat_k.as_strided((t, hkv, d), (stride, d, 1))
    value = flat_v.as_strided((t, hkv, d), (stride, d, 1))
    slots = rng.choice(nb * 16, size=t, replace=False).astype(np.int64)
    slots[3] = -7
    lib().pa_reshape_and_cache(key, value, kc, vc, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    kh = torch_to_storage(key.contiguous(), dtype)
    vh = torch_to_storage(value.contiguous(), dtype)
    zero = np.zeros((nb, hkv, 16, d), dtype=kh.dtype)
    ek, ev = oracle.reshape_and_cache(zero, zero, kh, vh, slots)
    assert np.array_equal(bits(torch_to_storage(kc, dtype)), bits(ek))
    assert np.array_equal(bits(torch_to_storage(vc, dtype)), bits(ev))


@pytest.mark.slow
def test_scatter_llama13b_full_size_bit_exact(gpu):
    """256 new tokens of 40 heads x 128 into a 65536-block bf16 pool."""
    import torch
    say("scatter config2 full size: generating")
    w = config2()
    dw = to_device(w)
    before_k = dw.k_cache.clone()
    before_v = dw.v_cache.clone()
    say("scatter config2: launching")
    gpu_scatter(dw)
    torch.cuda.synchronize()
    slots = torch.from_numpy(w.slot_mapping).cuda()
    blk, row = slots // 16, slots % 16
    got_k = dw.k_cache[blk, :, row, :]        # [T, Hkv, D]
    got_v = dw.v_cache[blk, :, row, :]
    assert torch.equal(got_k.view(torch.int16), dw.new_k.view(torch.int16))
    assert torch.equal(got_v.view(torch.int16), dw.new_v.view(torch.int16))
    # every other row untouched: restore the written rows in the copy and compare all bits
    before_k[blk, :, row, :] = dw.new_k
    before_v[blk, :, row, :] = dw.new_v
    assert torch.equal(before_k.view(torch.int16), dw.k_cache.view(torch.int16))
    assert torch.equal(before_v.view(torch.int16), dw.v_cache.view(torch.int16))
