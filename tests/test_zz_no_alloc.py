"""pa_decode_no_alloc (decode + split-K merge with the partials in the
library's fixed device buffer) against pa_decode + pa_decode_splitk_reduce
with a caller-owned workspace: the same kernels, so the outputs must be the
same bits.  Two calls in a row, the second smaller, so the second runs over
what the first left in the buffer; both decode kernels (vector ALUs and
matrix cores); and a call whose partials exceed the buffer is refused
without launching anything.
"""
import numpy as np
import pytest

from workloads import make_decode
from workloads.device import to_device

from pa_harness import as_f64, assert_close, lib, oracle_decode, say

pytestmark = pytest.mark.gpu


def with_workspace(L, dw, ps):
    """The existing entry points: pa_decode into a torch workspace, then the merge."""
    import torch
    g, w = dw.decode, dw.w
    out = torch.empty_like(g.out)
    ws = None
    if ps:
        nbytes = L.pa_decode_workspace_bytes(g.query.shape[0], w.num_heads, w.head_dim,
                                             g.max_context_len, ps)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    L.pa_decode(out, g.query, dw.k_cache, dw.v_cache, g.block_tables, g.context_lens, w.scale,
                g.max_context_len, ps, ws)
    if ps:
        L.pa_decode_splitk_reduce(out, ws, g.context_lens, g.max_context_len, ps)
    return out


@pytest.mark.parametrize("hq,hkv,d,dtype", [(32, 8, 128, "bf16"), (40, 40, 128, "bf16"),
                                            (8, 2, 64, "f32")])
def test_no_alloc_equals_pa_decode_on_two_calls(gpu, hq, hkv, d, dtype):
    import torch
    L = lib()
    rng = np.random.default_rng(401)
    calls = [("large", rng.integers(1, 6000, size=24), 512),
             ("small", rng.integers(1, 1500, size=6), 256)]
    for i, (name, lens, ps) in enumerate(calls):
        say(f"no-alloc decode {hq}/{hkv} d={d} {dtype}: call {i} ({name}, ps={ps})")
        w = make_decode(f"no-alloc-{name}", 402 + i, dtype, lens.astype(np.int32), hq, hkv, d,
                        8192, with_scatter=False)
        dw = to_device(w)
        g = dw.decode
        want = with_workspace(L, dw, ps)
        L.pa_decode_no_alloc(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                             g.context_lens, w.scale, g.max_context_len, ps)
        torch.cuda.synchronize()
        iv = torch.int16 if dtype == "bf16" else torch.int32
        assert torch.equal(g.out.view(iv), want.view(iv)), f"call {i}"
        assert_close(as_f64(g.out), oracle_decode(w), dtype, f"no-alloc call {i} vs oracle")


def test_no_alloc_refuses_partials_larger_than_its_buffer(gpu):
    import torch
    L = lib()
    w = make_decode("no-alloc-too-big", 405, "bf16", np.array([40, 70]), 8, 8, 128, 64,
                    with_scatter=False)
    dw = to_device(w)
    g = dw.decode
    g.out.fill_(3.0)
    big_ctx = 1 << 19    # 32768 partitions of 16 tokens per sequence and head
    need = L.pa_decode_workspace_bytes(2, 8, 128, big_ctx, 16)
    assert need > L.pa_decode_no_alloc_scratch_bytes()
    with pytest.raises(L.PagedAttentionError) as e:
        L.pa_decode_no_alloc(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                             g.context_lens, w.scale, big_ctx, 16)
    assert e.value.status == -11
    torch.cuda.synchronize()
    assert (g.out.float() == 3.0).all()      # nothing was launched
    # the same call within the buffer goes through
    L.pa_decode_no_alloc(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                         g.context_lens, w.scale, g.max_context_len, 16)
    torch.cuda.synchronize()
    assert_close(as_f64(g.out), oracle_decode(w), "bf16", "no-alloc within the buffer")
