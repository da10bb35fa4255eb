"""Split-K partials on the GPU against the oracle's per-partition results.

The workspace layout is part of the ABI: fp32 o_part [S, Hq, P, D] followed by
fp32 lse_part [S, Hq, P] (natural log).  The merge is checked separately: any
partition length gives the same final output within tolerance.
"""
import numpy as np
import pytest

import oracle
from workloads import make_decode

from pa_harness import as_f64, assert_close, gpu_decode, lib, oracle_decode, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,hq,hkv", [("bf16", 32, 8), ("f32", 8, 8), ("bf16", 40, 40)])
def test_partials_match_oracle(gpu, dtype, hq, hkv):
    import torch
    rng = np.random.default_rng(61)
    lens = np.concatenate([[1, 511, 512, 513], rng.integers(600, 3000, size=4)])
    ps = 512
    w = make_decode("parts", 61, dtype, lens, hq, hkv, 128, 2048, with_scatter=False)
    dw = to_device(w)
    g = dw.decode
    ws = gpu_decode(dw, ps)
    torch.cuda.synchronize()
    S, P, D = len(lens), -(-int(lens.max()) // ps), 128
    host = ws.cpu().numpy()
    o_part = host[:S * hq * P * D * 4].view(np.float32).reshape(S, hq, P, D)
    lse = host[S * hq * P * D * 4:S * hq * P * (D + 1) * 4].view(np.float32).reshape(S, hq, P)
    ro, rl, n = oracle.decode_partials(w.decode.query, w.k_host, w.v_host,
                                       w.host_tables(w.decode.block_tables), w.decode.context_lens,
                                       w.scale, w.dtype, ps)
    for s in range(S):
        if n[s] <= 1:
            continue   # written straight to the output, no partials
        assert_close(o_part[s, :, :n[s]], ro[s, :, :n[s]], dtype, f"o_part seq {s}")
        # lse: scores come from fp32 dot products of 128 terms; 1e-4 absolute covers
        # their rounding.  The matrix-core path (bf16, head_dim 128, 4 or more query
        # heads per kv head) also rounds each probability to bf16 (relative error
        # <= 2^-8) and sums the rounded weights, which moves the log of the sum by
        # at most ln(1 + 2^-8) < 3.9e-3; the vector-ALU path keeps fp32 weights.
        matrix_cores = dtype == "bf16" and hq // hkv >= 4
        lse_atol = 1e-4 + 3.9e-3 if matrix_cores else 1e-4
        err = np.abs(lse[s, :, :n[s]].astype(np.float64) - rl[s, :, :n[s]])
        assert (err <= lse_atol + 1e-5 * np.abs(rl[s, :, :n[s]])).all(), err.max()
    assert_close(as_f64(g.out), oracle_decode(w), dtype, "merged")


@pytest.mark.parametrize("ps", [16, 48, 512, 4096, 0])
def test_any_partition_length_gives_the_same_answer(gpu, ps):
    rng = np.random.default_rng(62)
    lens = rng.integers(1, 3000, size=10)
    w = make_decode("anyps", 62, "f32", lens, 8, 2, 64, 2048, with_scatter=True)
    dw = to_device(w)
    from pa_harness import gpu_scatter
    import torch
    gpu_scatter(dw)
    gpu_decode(dw, ps)
    torch.cuda.synchronize()
    assert_close(as_f64(dw.decode.out), oracle_decode(w), "f32", f"ps={ps}")


def test_workspace_size_formula(gpu):
    L = lib()
    sched = 64 + 32 * 64   # the schedule: header and (sequence, partition) pairs
    assert L.pa_decode_workspace_bytes(32, 32, 128, 32768, 512) == 32 * 32 * 64 * (128 + 1) * 4 + sched * 4
    assert L.pa_decode_workspace_bytes(4, 8, 64, 100, 0) == 0


def _decode_into(dw, ps, ws):
    """pa_decode + merge of dw into its output, with the given workspace."""
    import torch
    L = lib()
    g, w = dw.decode, dw.w
    L.pa_decode(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables, g.context_lens, w.scale,
                g.max_context_len, ps, ws)
    L.pa_decode_splitk_reduce(g.out, ws, g.context_lens, g.max_context_len, ps)
    torch.cuda.synchronize()


def test_dealt_schedule_with_fewer_units_than_xcds(gpu):
    """One sequence, one kv head, two 16-token partitions: two units for a launch
    of eight XCDs' slots, so most workgroups find no unit and must do nothing."""
    import torch
    w = make_decode("deal2", 71, "f32", np.array([20]), 1, 1, 64, 8, with_scatter=False)
    dw = to_device(w)
    nbytes = lib().pa_decode_workspace_bytes(1, 1, 64, 20, 16)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    _decode_into(dw, 16, ws)
    assert_close(as_f64(dw.decode.out), oracle_decode(w), "f32", "2 units")


def test_dealt_schedule_long_partitions_then_smaller_batch(gpu):
    """Partitions of 1100 blocks (past the length sort's last bucket, 1023 blocks)
    over lengths from 1 to 40000 tokens, an empty sequence among them; then a
    smaller batch through the same workspace, whose schedule is rewritten whole."""
    import torch
    ps = 1100 * 16
    lens = np.array([40000, 2 * ps + 5, 0, 1, ps + 1, 30000, 16, 1234])
    w = make_decode("deal_long", 72, "f32", lens, 4, 2, 64, 8192, with_scatter=False)
    dw = to_device(w)
    g = dw.decode
    nbytes = lib().pa_decode_workspace_bytes(len(lens), 4, 64, g.max_context_len, ps)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    _decode_into(dw, ps, ws)
    out = as_f64(g.out)
    live = [i for i, n in enumerate(lens) if n > 0]
    assert_close(out[live], oracle_decode(w, seqs=live), "f32", "long partitions")
    assert (out[2] == 0).all()
    say(f"long partitions: {len(live)} sequences within tolerance, the empty one zero")

    small = make_decode("deal_small", 73, "f32", np.array([3000, 17, 17600]), 4, 2, 64, 2048,
                        with_scatter=False)
    ds = to_device(small)
    assert lib().pa_decode_workspace_bytes(3, 4, 64, ds.decode.max_context_len, ps) <= nbytes
    _decode_into(ds, ps, ws)
    assert_close(as_f64(ds.decode.out), oracle_decode(small), "f32", "smaller batch, same workspace")


def test_dealt_schedule_with_many_sequences(gpu):
    """5000 sequences of 0-40 tokens in 16-token partitions: the schedule's
    threads take several sequences each, and those past the first 4096 are
    re-read rather than cached in LDS between its two passes."""
    import torch
    rng = np.random.default_rng(74)
    lens = rng.integers(0, 41, size=5000)
    w = make_decode("deal_many", 74, "f32", lens, 2, 1, 64, 16384, with_scatter=False)
    dw = to_device(w)
    g = dw.decode
    nbytes = lib().pa_decode_workspace_bytes(len(lens), 2, 64, g.max_context_len, 16)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    _decode_into(dw, 16, ws)
    out = as_f64(g.out)
    live = np.nonzero(lens > 0)[0]
    assert_close(out[live], oracle_decode(w, seqs=live), "f32", "5000 sequences")
    assert (out[lens == 0] == 0).all()
