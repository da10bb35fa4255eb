"""pa_prefill_chunk_split / pa_prefill_chunk_fp8_split on the GPU.

Long causal key ranges are cut into runs of split_tokens keys, one workgroup
each, and merged by the log-sum-exp rule; the result must match the fp64
oracle like the unsplit prefill.  Cases: the mixed workload's four chunks over
prefixes of 216-3100 tokens at several run lengths (one tile, several, longer
than any range), ragged chunk and prefix lengths where a run starts inside a
wave's causal diagonal (rows that see none of a run's keys), grouped-query
heads, head_dim 64, FP8 caches, and the contract cases (a sequence longer than
max_context_len gets NaN, a short workspace or an fp32 query is refused).  The
workspace is filled with NaN before every run.
"""
import numpy as np
import pytest

from oracle import kv_fp8
from pa_harness import as_f64, assert_close, lib, oracle_prefill, say, to_device
from workloads import config4, fp8_pools, make_prefill
from workloads.device import upload_fp8_pools

pytestmark = pytest.mark.gpu
K_SCALE, V_SCALE = 0.07, 0.11


def run_split(w, split, max_context_len=None, pools=None):
    import torch
    L = lib()
    dw = to_device(w, pools=pools is None)
    kc, vc = (dw.k_cache, dw.v_cache) if pools is None else upload_fp8_pools(w, *pools)
    g = dw.prefill
    tq, hq, d = g.query.shape
    maxc = int(w.prefill.context_lens.max()) if max_context_len is None else max_context_len
    ws = torch.empty(max(L.pa_prefill_workspace_bytes(tq, hq, d, maxc, split), 16),
                     dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    g.out.view(torch.int16).fill_(0x7FC0)
    if pools is None:
        L.pa_prefill_chunk_split(g.out, g.query, kc, vc, g.block_tables, g.query_start_loc,
                                 g.context_lens, w.scale, g.max_query_len, maxc, split, ws)
    else:
        L.pa_prefill_chunk_fp8_split(g.out, g.query, kc, vc, g.block_tables, g.query_start_loc,
                                     g.context_lens, float(w.scale), K_SCALE, V_SCALE,
                                     g.max_query_len, maxc, split, ws)
    torch.cuda.synchronize()
    return g.out


@pytest.mark.parametrize("split", [64, 1024, 2048, 8192])   # 2048: the launch bench.py times
def test_mixed_chunks_split(gpu, split):
    say(f"split prefill: mixed workload's 4 x 512-token chunks, runs of {split} keys")
    w = config4()
    w.decode = None
    out = run_split(w, split)
    assert_close(as_f64(out), oracle_prefill(w), "bf16", f"mixed prefill split {split}")


@pytest.mark.parametrize("hq,hkv,d,split", [(8, 2, 128, 64), (8, 2, 128, 192), (6, 3, 64, 128),
                                            (4, 4, 128, 320)])
def test_ragged_split(gpu, hq, hkv, d, split):
    say(f"split prefill: ragged {hq}/{hkv}/{d}, runs of {split} keys")
    prefix = [0, 5, 16, 100, 777, 3000]
    chunk = [1, 70, 64, 130, 33, 200]
    w = make_prefill(f"split-{hq}-{hkv}-{d}", 81 + hq, "bf16", prefix, chunk, hq, hkv, d, 512)
    out = run_split(w, split)
    assert_close(as_f64(out), oracle_prefill(w), "bf16", f"ragged split {hq}/{hkv}/{d}/{split}")


def test_fp8_split(gpu):
    say("split prefill over an FP8 cache")
    w = make_prefill("split-fp8", 85, "bf16", [0, 700, 2500], [90, 256, 300], 8, 4, 128, 512)
    kq, vq = fp8_pools(w, 86)
    out = run_split(w, 256, pools=(kq, vq))
    g = w.prefill
    want = kv_fp8.prefill(g.query, kq, vq, w.host_tables(g.block_tables), g.query_start_loc,
                          g.context_lens, w.scale, K_SCALE, V_SCALE, "bf16")
    assert_close(as_f64(out), want, "bf16", "fp8 split prefill")


def test_split_block_outside_pool_gives_nan(gpu):
    """A negative block id in one key run: that run's partials are NaN, so the
    merge gives NaN for the whole chunk of its sequence; other sequences match."""
    import torch
    L = lib()
    w = make_prefill("split-bad-id", 89, "bf16", [300, 900, 50], [40, 100, 60], 4, 2, 128, 128)
    dw = to_device(w)
    g = dw.prefill
    bt = g.block_tables.clone()
    bt[1, 20] = -3                  # keys 320..335 of 1000: the second run of 256
    g.block_tables = bt
    tq, hq, d = g.query.shape
    maxc = int(w.prefill.context_lens.max())
    ws = torch.empty(L.pa_prefill_workspace_bytes(tq, hq, d, maxc, 256), dtype=torch.uint8,
                     device="cuda")
    ws.fill_(0xFF)
    say("split prefill (runs of 256) with block id -3 in sequence 1 of 3")
    L.pa_prefill_chunk_split(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                             g.query_start_loc, g.context_lens, w.scale, g.max_query_len, maxc,
                             256, ws)
    torch.cuda.synchronize()
    out = as_f64(g.out)
    ref = oracle_prefill(w)
    q = w.prefill.query_start_loc
    assert np.isnan(out[q[1]:q[2]]).all()
    for s in (0, 2):
        assert_close(out[q[s]:q[s + 1]], ref[q[s]:q[s + 1]], "bf16", f"sequence {s}")


def test_split_contract(gpu):
    """A sequence longer than max_context_len gets NaN rows and nobody else
    changes; a short workspace and an fp32 query are refused."""
    import torch
    L = lib()
    w = make_prefill("split-contract", 87, "bf16", [100, 2000], [50, 50], 4, 4, 128, 256)
    out = run_split(w, 256, max_context_len=1000)
    ref = oracle_prefill(w)
    got = as_f64(out)
    assert_close(got[:50], ref[:50], "bf16", "healthy sequence")
    assert np.isnan(got[50:]).all()
    dw = to_device(w)
    g = dw.prefill
    need = L.pa_prefill_workspace_bytes(100, 4, 128, 2050, 256)
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.PagedAttentionError):
        L.pa_prefill_chunk_split(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                                 g.query_start_loc, g.context_lens, w.scale, g.max_query_len,
                                 2050, 256, ws)
    wf = make_prefill("split-f32", 88, "f32", [10], [20], 4, 4, 128, 64)
    dwf = to_device(wf)
    gf = dwf.prefill
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.PagedAttentionError):
        L.pa_prefill_chunk_split(gf.out, gf.query, dwf.k_cache, dwf.v_cache, gf.block_tables,
                                 gf.query_start_loc, gf.context_lens, wf.scale, gf.max_query_len,
                                 30, 64, ws)


@pytest.mark.slow
@pytest.mark.parametrize("split", [3072, 5504])
def test_long_prefix_split_launch(gpu, split):
    """The launch bench.py --workload prefill_long times: three even runs of
    5504 keys (and six of 3072) over a 16384-token prefix with a 128-token
    chunk (one sequence, 8 heads, so the oracle finishes in seconds).  One
    query tile per sequence and one query head per kv head: the launch that
    streams its K/V with the nontemporal hint."""
    say(f"split prefill: 128-token chunk over a 16384-token prefix, runs of {split} keys")
    w = make_prefill("split-long", 89, "bf16", [16384], [128], 8, 8, 128, 1040)
    out = run_split(w, split)
    assert_close(as_f64(out), oracle_prefill(w), "bf16", f"long prefix split {split}")
