"""pa_prefill_chunk on the GPU against the fp64 oracle.

bf16 runs on the MFMA kernel, fp32 on the per-token vector path.  Cases: the
mixed workload's four 512-token chunks over paged prefixes, chunks with no
prefix, ragged chunk and prefix lengths (not multiples of 16 or 64), GQA heads,
head_dim 64, a one-token chunk equal to decode, and a prompt prefilled in two
chunks equal to the same prompt in one chunk (xdnf.cn article, section 六.4).
"""
import numpy as np
import pytest

from workloads import config4, make_prefill

from pa_harness import (as_f64, assert_close, gpu_decode, gpu_prefill, oracle_decode,
                        oracle_prefill, say, to_device)

pytestmark = pytest.mark.gpu


def run(w):
    import torch
    dw = to_device(w)
    gpu_prefill(dw)
    torch.cuda.synchronize()
    return dw


def test_mixed_workload_prefill_part(gpu):
    say("prefill config4: 4 x 512-token chunks")
    w = config4()
    w.decode = None
    dw = run(w)
    assert_close(as_f64(dw.prefill.out), oracle_prefill(w), "bf16", "config4 prefill")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 128), (8, 2, 128), (6, 3, 64)])
def test_ragged_chunks(gpu, dtype, hq, hkv, d):
    prefix = [0, 5, 16, 100, 777]
    chunk = [1, 70, 64, 130, 33]
    w = make_prefill(f"ragged-{hq}-{hkv}-{d}", 71 + hq, dtype, prefix, chunk, hq, hkv, d, 256)
    dw = run(w)
    assert_close(as_f64(dw.prefill.out), oracle_prefill(w), dtype, f"ragged {dtype} {hq}/{hkv}/{d}")


def test_no_prefix_long_chunk(gpu):
    w = make_prefill("noprefix", 72, "bf16", [0, 0], [1000, 257], 8, 8, 128, 256)
    dw = run(w)
    assert_close(as_f64(dw.prefill.out), oracle_prefill(w), "bf16", "no prefix")


def test_fp32_prefill_tight(gpu):
    w = make_prefill("f32", 73, "f32", [0, 300, 1000], [200, 64, 17], 8, 4, 128, 256)
    dw = run(w)
    assert_close(as_f64(dw.prefill.out), oracle_prefill(w), "f32", "f32 prefill")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_token_chunk_equals_decode(gpu, dtype):
    import torch
    w = make_prefill("one", 74, dtype, [0, 40, 500], [1, 1, 1], 8, 2, 128, 64)
    dw = run(w)
    g = dw.prefill
    from workloads.device import DeviceGroup
    dec = DeviceGroup(context_lens=g.context_lens, block_tables=g.block_tables, query=g.query,
                      out=torch.empty_like(g.out), max_context_len=int(g.context_lens.max().item()))
    gpu_decode(dw, 0, group=dec)
    torch.cuda.synchronize()
    assert_close(as_f64(g.out), as_f64(dec.out), dtype, "prefill(1) vs decode")
    assert_close(as_f64(g.out), oracle_prefill(w), dtype, "prefill(1) vs oracle")


def test_two_chunks_equal_one_shot(gpu):
    import torch
    w = make_prefill("oneshot", 75, "bf16", [0], [1024], 8, 8, 128, 128)
    dw = run(w)
    one = as_f64(dw.prefill.out)
    g = dw.prefill
    for lo in (0, 512):
        out = torch.empty((512, 8, 128), dtype=g.out.dtype, device="cuda")
        from paged_kv_cache_453_amd import lib
        lib.pa_prefill_chunk(out, g.query[lo:lo + 512].contiguous(), dw.k_cache, dw.v_cache,
                             g.block_tables, torch.tensor([0, 512], dtype=torch.int32, device="cuda"),
                             torch.tensor([lo + 512], dtype=torch.int32, device="cuda"), w.scale, 512)
        torch.cuda.synchronize()
        assert_close(as_f64(out), one[lo:lo + 512], "bf16", f"chunk at {lo}")
    assert_close(one, oracle_prefill(w), "bf16", "one shot")


def test_prefill_contract_violation_gives_nan(gpu):
    import torch
    w = make_prefill("bad", 76, "bf16", [10, 10], [20, 20], 4, 4, 128, 64)
    dw = to_device(w)
    g = dw.prefill
    lens = g.context_lens.clone()
    lens[1] = 5                     # chunk longer than its context
    g.context_lens = lens
    gpu_prefill(dw)
    torch.cuda.synchronize()
    out = as_f64(g.out)
    assert np.isnan(out[20:]).all()
    assert_close(out[:20], oracle_prefill(w)[:20], "bf16", "healthy sequence")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_chunk_longer_than_max_query_len_gives_nan(gpu, dtype):
    """max_query_len = 100 while sequence 1 brings 300 query rows: its whole
    chunk is NaN, rows past the first 128-row tile included; sequence 0 (100
    rows) is unchanged."""
    import torch
    from paged_kv_cache_453_amd import lib as L
    w = make_prefill("too-long", 78, dtype, [10, 10], [100, 300], 4, 4, 128, 64)
    dw = to_device(w)
    g = dw.prefill
    say(f"prefill {dtype}: chunk of 300 rows with max_query_len 100")
    L.pa_prefill_chunk(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                       g.query_start_loc, g.context_lens, w.scale, 100)
    torch.cuda.synchronize()
    out = as_f64(g.out)
    assert np.isnan(out[100:]).all()
    assert_close(out[:100], oracle_prefill(w)[:100], dtype, "healthy sequence")


@pytest.mark.parametrize("bad_id", ["past_pool", "negative"])
def test_prefill_block_outside_pool_gives_nan(gpu, bad_id):
    """A live block id outside the pool (past its end, or negative) turns that
    sequence's chunk into NaN; nothing is read for it, and the other sequences
    are unchanged."""
    import torch
    w = make_prefill("bad-id", 77, "bf16", [40, 100, 30], [20, 70, 90], 4, 2, 128, 64)
    dw = to_device(w)
    g = dw.prefill
    bt = g.block_tables.clone()
    bt[1, 3] = w.num_blocks if bad_id == "past_pool" else -7   # keys 48..63 of 170: live
    g.block_tables = bt
    say(f"prefill with block id {int(bt[1, 3])} in sequence 1 of 3")
    gpu_prefill(dw)
    torch.cuda.synchronize()
    out = as_f64(g.out)
    ref = oracle_prefill(w)
    q = w.prefill.query_start_loc
    assert np.isnan(out[q[1]:q[2]]).all()
    for s in (0, 2):
        assert_close(out[q[s]:q[s + 1]], ref[q[s]:q[s + 1]], "bf16", f"sequence {s}")


@pytest.mark.slow
@pytest.mark.parametrize("ps", [512, 2048])   # 2048: the launch bench.py times
def test_mixed_step_prefill_then_decode(gpu, ps):
    """The whole mixed batch on one stream: 4 prefill chunks, then 192 decoders
    that share 2048-token prefixes in groups of 3 (with the sharing hint)."""
    import torch
    say(f"mixed step config4 ps={ps}")
    w = config4(partition_size=ps)
    dw = to_device(w)
    gpu_prefill(dw)
    gpu_decode(dw)
    torch.cuda.synchronize()
    assert_close(as_f64(dw.prefill.out), oracle_prefill(w), "bf16", "mixed: prefill part")
    assert_close(as_f64(dw.decode.out), oracle_decode(w), "bf16", "mixed: decode part")


@pytest.mark.slow
def test_mixed_step_two_streams(gpu):
    """Prefill on a second stream running beside decode (the overlapped step
    bench.py also times) gives the same results: both only read the pools."""
    import torch
    from paged_kv_cache_453_amd import lib as L
    say("mixed step on two streams")
    w = config4(partition_size=2048)
    dw = to_device(w)
    g, p = dw.decode, dw.prefill
    nbytes = L.pa_decode_workspace_bytes(g.query.shape[0], w.num_heads, w.head_dim,
                                         g.max_context_len, 2048)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    fork = torch.cuda.Event()
    fork.record(main)
    side.wait_event(fork)
    L.pa_prefill_chunk(p.out, p.query, dw.k_cache, dw.v_cache, p.block_tables,
                       p.query_start_loc, p.context_lens, w.scale, p.max_query_len, stream=side)
    L.pa_decode(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables, g.context_lens, w.scale,
                g.max_context_len, 2048, ws, stream=main,
                shared_prefix_blocks=g.shared_prefix_blocks)
    L.pa_decode_splitk_reduce(g.out, ws, g.context_lens, g.max_context_len, 2048, stream=main)
    join = torch.cuda.Event()
    join.record(side)
    main.wait_event(join)
    torch.cuda.synchronize()
    assert_close(as_f64(p.out), oracle_prefill(w), "bf16", "two streams: prefill")
    assert_close(as_f64(g.out), oracle_decode(w), "bf16", "two streams: decode")
