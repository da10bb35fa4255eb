"""FP8 (OCP E4M3) KV cache on the GPU against the oracle (oracle/kv_fp8.py).

The scatter must produce the oracle's codes bit for bit, ties, subnormals,
saturation and NaN included.  Every one of the 256 codes must dequantise
exactly on each kernel path (a one-token context returns V).  Decode must
match the oracle's attention over the values the codes stand for, at the
tolerance of the query dtype (fp32 accumulation in both cases: the codes
themselves are exact), across the vector-ALU path (groups up to 4, fp32 and
bf16 queries) and the matrix-core path (bf16 grouped-query heads), with and
without split-K.  Unused rows and partial-block tails hold the NaN code.
"""
import numpy as np
import pytest

from oracle import kv_fp8
from pa_harness import TOL, as_f64, assert_close, say
from workloads import config2, config4, fp8_codes, fp8_pools, make_decode, make_prefill
from workloads.device import host_to_torch, to_device, torch_to_storage, upload_fp8_pools
from workloads.generate import f32_to_bf16_bits

pytestmark = pytest.mark.gpu
BS = 16
K_SCALE, V_SCALE = 0.07, 0.11


def storage(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def special_values(k_scale):
    """Inputs that land on every kind of code: representable values, midpoints
    (ties), subnormals, the saturation edge and beyond, NaN, signed zero."""
    pos = kv_fp8.decode_codes(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    xs = np.concatenate([pos, mids, -pos, -mids, [448, 463.9, 464, 500, 1e30, np.inf, -np.inf,
                                                  np.nan, -0.0, 2.0 ** -11, -2.0 ** -12]])
    return (xs * k_scale).astype(np.float32)


@pytest.mark.parametrize("src,hkv,d,scales", [("f32", 4, 128, (0.25, 0.5)),
                                              ("bf16", 4, 128, (0.25, 0.5)),
                                              ("f32", 2, 64, (0.0123, 0.0311)),
                                              ("bf16", 8, 128, (0.0123, 0.0311))])
def test_fp8_scatter_bit_exact(gpu, src, hkv, d, scales):
    import torch
    ks, vs = scales
    say(f"fp8 scatter src={src} hkv={hkv} d={d} scales={scales}")
    rng = np.random.default_rng(31)
    nb, t = 12, 24
    k0 = fp8_codes((nb, hkv, BS, d), np.random.SeedSequence(1))
    v0 = fp8_codes((nb, hkv, BS, d), np.random.SeedSequence(2))
    key = (rng.standard_normal((t, hkv, d)) * 4).astype(np.float32)
    val = (rng.standard_normal((t, hkv, d)) * 4).astype(np.float32)
    sp = special_values(ks)
    key.reshape(-1)[:sp.size] = sp
    val.reshape(-1)[:sp.size] = special_values(vs)
    key, val = storage(key, src), storage(val, src)
    slots = rng.choice(nb * BS, t, replace=False).astype(np.int64)
    slots[3], slots[9] = -1, nb * BS + 3                    # padding, past the pool
    kc = torch.from_numpy(k0.copy()).cuda()
    vc = torch.from_numpy(v0.copy()).cuda()
    gpu.pa_reshape_and_cache_fp8(host_to_torch(key, src, "cuda"), host_to_torch(val, src, "cuda"),
                                 kc, vc, torch.from_numpy(slots).cuda(), ks, vs)
    torch.cuda.synchronize()
    ok_slots = np.where(slots < nb * BS, slots, -1)
    want_k, want_v = kv_fp8.reshape_and_cache(k0, v0, key, val, ok_slots, src, ks, vs)
    assert np.array_equal(kc.cpu().numpy(), want_k)
    assert np.array_equal(vc.cpu().numpy(), want_v)


@pytest.mark.parametrize("qdtype,hq,hkv", [("f32", 2, 2), ("bf16", 2, 2), ("bf16", 8, 2),
                                            ("f32", 8, 2)])
def test_fp8_every_code_dequantises_exactly(gpu, qdtype, hq, hkv):
    """One-token contexts return V: out = value(code) * v_scale, exactly
    (v_scale = 2 and every E4M3 value fits fp32 and bf16)."""
    import torch
    say(f"fp8 dequant of all codes q={qdtype} hq={hq} hkv={hkv}")
    d, nseq = 128, 2
    codes = np.arange(256, dtype=np.uint8)
    rows = [codes[:128], codes[128:], codes[::-1][:128], codes[::-1][128:]]
    v = np.zeros((nseq, hkv, BS, d), dtype=np.uint8)
    for s in range(nseq):
        for h in range(hkv):
            v[s, h, 0] = rows[(2 * s + h) % 4]
    k = fp8_codes((nseq, hkv, BS, d), np.random.SeedSequence(5))
    q = storage(np.random.default_rng(6).standard_normal((nseq, hq, d)), qdtype)
    qt = host_to_torch(q, qdtype, "cuda")
    out = torch.empty_like(qt)
    tables = torch.tensor([[0], [1]], dtype=torch.int32, device="cuda")
    lens = torch.tensor([1, 1], dtype=torch.int32, device="cuda")
    gpu.pa_decode_fp8(out, qt, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), tables,
                      lens, 0.088, 0.5, 2.0, 1)
    torch.cuda.synchronize()
    got = as_f64(out)
    g = hq // hkv
    for s in range(nseq):
        for h in range(hq):
            want = kv_fp8.decode_codes(v[s, h // g, 0]) * 2.0
            same = (got[s, h] == want) | (np.isnan(got[s, h]) & np.isnan(want))
            assert same.all(), (s, h, np.nonzero(~same)[0][:5])


CASES = [  # (query dtype, hq, hkv, d, partition size): vector ALUs for G <= 4, matrix cores
    ("f32", 8, 8, 128, 0), ("f32", 8, 8, 128, 256), ("bf16", 8, 8, 128, 0),   # for bf16 G >= 4
    ("bf16", 8, 8, 64, 512), ("f32", 8, 4, 64, 0), ("f32", 16, 4, 128, 256),
    ("bf16", 16, 4, 128, 0), ("bf16", 32, 4, 128, 512), ("bf16", 48, 3, 128, 256),
    ("bf16", 4, 2, 64, 0)]


def fp8_workload(qdtype, hq, hkv, d, ps, seed=71, nseq=24):
    rng = np.random.default_rng(seed)
    lens = np.concatenate([[1, 15, 16, 17, 33, 256, 257], rng.integers(1, 700, nseq - 7)])
    return make_decode(f"fp8-{qdtype}-{hq}-{hkv}-{d}", seed, qdtype, lens.astype(np.int32), hq,
                       hkv, d, num_blocks=1024, with_scatter=False, partition_size=ps)


def run_fp8_decode(gpu, w, k_codes, v_codes, ps, hint=None, scales=(K_SCALE, V_SCALE)):
    import torch
    dw = to_device(w)
    kc, vc = upload_fp8_pools(w, k_codes, v_codes)
    g = dw.decode
    ws = None
    if ps:
        nbytes = gpu.pa_decode_workspace_bytes(g.query.shape[0], w.num_heads, w.head_dim,
                                               g.max_context_len, ps)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    gpu.pa_decode_fp8(g.out, g.query, kc, vc, g.block_tables, g.context_lens, float(w.scale),
                      scales[0], scales[1], g.max_context_len, ps, ws, shared_prefix_blocks=hint)
    if ps:
        gpu.pa_decode_splitk_reduce(g.out, ws, g.context_lens, g.max_context_len, ps)
    torch.cuda.synchronize()
    return dw, g.out


@pytest.mark.parametrize("qdtype,hq,hkv,d,ps", CASES)
def test_fp8_decode_matches_oracle(gpu, qdtype, hq, hkv, d, ps):
    say(f"fp8 decode q={qdtype} hq={hq} hkv={hkv} d={d} ps={ps}")
    w = fp8_workload(qdtype, hq, hkv, d, ps)
    kq, vq = fp8_pools(w, 72)
    _, out = run_fp8_decode(gpu, w, kq, vq, ps)
    g = w.decode
    want = kv_fp8.decode(g.query, kq, vq, w.host_tables(g.block_tables), g.context_lens, w.scale,
                         K_SCALE, V_SCALE, qdtype)
    assert_close(as_f64(out), want, qdtype, f"fp8 decode {qdtype} {hq}/{hkv} d={d} ps={ps}")


# Every finite code (exponent fields 0..14, magnitudes up to 448) in K and V, on
# each decode path: the vector ALUs with fp32 and bf16 queries, and the matrix
# cores.  Power-of-two scales keep the values the size of the N(0, 1) workloads
# the tolerance is stated for: |k| <= 448 / 256 = 1.75, |v| <= 448 / 512 = 0.875.
# (The matrix-core paths round each weight to bf16, an error that grows with the
# spread of V: with |v| up to 22, a few elements in 10^5 passed the absolute
# 4e-3 bound, while the vector-ALU paths, which keep fp32 weights, did not.)
FULL_RANGE_SCALES = (2.0 ** -8, 2.0 ** -9)


@pytest.mark.parametrize("qdtype,hq,hkv,d,ps", [("f32", 8, 8, 128, 256), ("bf16", 8, 2, 64, 0),
                                                ("bf16", 16, 4, 128, 256),
                                                ("bf16", 32, 8, 128, 512)])
def test_fp8_decode_full_code_range(gpu, qdtype, hq, hkv, d, ps):
    say(f"fp8 decode, full code range, q={qdtype} hq={hq} hkv={hkv} d={d} ps={ps}")
    w = fp8_workload(qdtype, hq, hkv, d, ps, seed=93)
    kq, vq = fp8_pools(w, 94, max_exp_field=14)
    _, out = run_fp8_decode(gpu, w, kq, vq, ps, scales=FULL_RANGE_SCALES)
    g = w.decode
    want = kv_fp8.decode(g.query, kq, vq, w.host_tables(g.block_tables), g.context_lens, w.scale,
                         *FULL_RANGE_SCALES, qdtype)
    assert_close(as_f64(out), want, qdtype, f"fp8 full-range decode {qdtype} {hq}/{hkv} ps={ps}")


@pytest.mark.parametrize("qdtype,hq,hkv,d,ps", [("bf16", 8, 8, 128, 0), ("bf16", 32, 4, 128, 512)])
def test_fp8_shared_hint_changes_nothing(gpu, qdtype, hq, hkv, d, ps):
    import torch
    say(f"fp8 decode hint bit-identity q={qdtype} hq={hq} hkv={hkv}")
    w = fp8_workload(qdtype, hq, hkv, d, ps)
    kq, vq = fp8_pools(w, 73)
    _, base = run_fp8_decode(gpu, w, kq, vq, ps)
    base = base.clone()
    for val in (3, 0, -5, 10**6):
        hint = torch.full((w.decode.num_seqs,), val, dtype=torch.int32, device="cuda")
        _, out = run_fp8_decode(gpu, w, kq, vq, ps, hint)
        assert torch.equal(out.view(torch.int16), base.view(torch.int16)), val


def test_fp8_rejects_what_it_does_not_run(gpu):
    import torch
    w = fp8_workload("f32", 32, 4, 128, 0, nseq=8)
    kq, vq = fp8_pools(w, 74)
    with pytest.raises(gpu.PagedAttentionError) as e:       # fp32 query, 8 heads per kv head
        run_fp8_decode(gpu, w, kq, vq, 0)
    assert e.value.status == -3
    q = torch.zeros((1, 2, 64), device="cuda")
    kc = torch.zeros((1, 2, 16, 64), dtype=torch.uint8, device="cuda")
    t = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    with pytest.raises(gpu.ShapeError):                     # a scale that is not positive
        gpu.pa_decode_fp8(q, q, kc, kc, t, t[0], 0.1, 0.0, 1.0, 1)


@pytest.mark.slow
def test_fp8_llama13b_scatter_then_decode(gpu):
    """The configuration the FP8 bench line times: 13B-shaped pools of codes,
    the 256 newest bf16 tokens quantised into their slots, decode with
    2048-token partitions and the merge."""
    import torch
    say("fp8 13B: generating")
    w = config2(partition_size=2048)
    kq, vq = fp8_pools(w, 75)
    dw = to_device(w)
    kc, vc = upload_fp8_pools(w, kq, vq)
    del dw.k_cache, dw.v_cache
    g = dw.decode
    say("fp8 13B: scatter + decode")
    gpu.pa_reshape_and_cache_fp8(dw.new_k, dw.new_v, kc, vc, dw.slot_mapping, K_SCALE, V_SCALE)
    nbytes = gpu.pa_decode_workspace_bytes(g.query.shape[0], w.num_heads, w.head_dim,
                                           g.max_context_len, 2048)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gpu.pa_decode_fp8(g.out, g.query, kc, vc, g.block_tables, g.context_lens, float(w.scale),
                      K_SCALE, V_SCALE, g.max_context_len, 2048, ws)
    gpu.pa_decode_splitk_reduce(g.out, ws, g.context_lens, g.max_context_len, 2048)
    torch.cuda.synchronize()
    say("fp8 13B: oracle")
    hs = w.host_slots()
    kq2, vq2 = kv_fp8.reshape_and_cache(kq, vq, w.new_k, w.new_v, hs, "bf16", K_SCALE, V_SCALE)
    # the scattered rows, bit for bit
    slots = w.slot_mapping
    got_k = kc[torch.from_numpy(slots // BS).cuda(), :, torch.from_numpy(slots % BS).cuda()]
    assert np.array_equal(got_k.cpu().numpy(), kq2[hs // BS, :, hs % BS])
    # decode on a sample of sequences, the longest included
    gg = w.decode
    pick = np.unique(np.concatenate([[int(np.argmax(gg.context_lens))],
                                     np.random.default_rng(76).choice(gg.num_seqs, 24, False)]))
    want = kv_fp8.decode(gg.query[pick], kq2, vq2, w.host_tables(gg.block_tables[pick]),
                         gg.context_lens[pick], w.scale, K_SCALE, V_SCALE, "bf16")
    assert_close(as_f64(g.out)[pick], want, "bf16", "fp8 13B decode (sampled)")


def run_fp8_prefill(gpu, w, k_codes, v_codes, scales=(K_SCALE, V_SCALE)):
    import torch
    dw = to_device(w)
    kc, vc = upload_fp8_pools(w, k_codes, v_codes)
    g = dw.prefill
    gpu.pa_prefill_chunk_fp8(g.out, g.query, kc, vc, g.block_tables, g.query_start_loc,
                             g.context_lens, float(w.scale), scales[0], scales[1],
                             g.max_query_len)
    torch.cuda.synchronize()
    return dw, kc, vc


def oracle_fp8_prefill(w, k_codes, v_codes, scales=(K_SCALE, V_SCALE)):
    g = w.prefill
    return kv_fp8.prefill(g.query, k_codes, v_codes, w.host_tables(g.block_tables),
                          g.query_start_loc, g.context_lens, w.scale, scales[0], scales[1],
                          "bf16")


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (6, 3, 64)])
def test_fp8_prefill_full_code_range(gpu, hq, hkv, d):
    """Every finite code in K and V through the prefill's staging widening."""
    say(f"fp8 prefill, full code range, hq={hq} hkv={hkv} d={d}")
    w = make_prefill(f"fp8-prefill-full-{hq}-{hkv}-{d}", 95, "bf16", [0, 37, 300, 1000],
                     [130, 64, 200, 77], hq, hkv, d, 256)
    kq, vq = fp8_pools(w, 96, max_exp_field=14)
    dw, _, _ = run_fp8_prefill(gpu, w, kq, vq, scales=FULL_RANGE_SCALES)
    assert_close(as_f64(dw.prefill.out), oracle_fp8_prefill(w, kq, vq, scales=FULL_RANGE_SCALES),
                 "bf16", f"fp8 full-range prefill {hq}/{hkv} d={d}")


@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 128), (8, 2, 128), (6, 3, 64), (32, 8, 128)])
def test_fp8_prefill_matches_oracle(gpu, hq, hkv, d):
    """Ragged chunks over ragged paged prefixes (not multiples of 16 or 64)."""
    say(f"fp8 prefill hq={hq} hkv={hkv} d={d}")
    w = make_prefill(f"fp8-prefill-{hq}-{hkv}-{d}", 81 + hq, "bf16", [0, 5, 16, 100, 777],
                     [1, 70, 64, 130, 33], hq, hkv, d, 256)
    kq, vq = fp8_pools(w, 82)
    dw, _, _ = run_fp8_prefill(gpu, w, kq, vq)
    assert_close(as_f64(dw.prefill.out), oracle_fp8_prefill(w, kq, vq), "bf16",
                 f"fp8 prefill {hq}/{hkv} d={d}")


def test_fp8_mixed_step_on_one_cache(gpu):
    """A step that prefills chunks and decodes other sequences over the same FP8
    pools: both parts against the oracle."""
    import torch
    say("fp8 mixed step: prefill chunks + shared-prefix decoders on one FP8 cache")
    w = config4(num_prompts=8, samples=3, num_prefill=2, num_blocks=4096)
    kq, vq = fp8_pools(w, 83)
    dw, kc, vc = run_fp8_prefill(gpu, w, kq, vq)
    g = dw.decode
    gpu.pa_decode_fp8(g.out, g.query, kc, vc, g.block_tables, g.context_lens, float(w.scale),
                      K_SCALE, V_SCALE, g.max_context_len, 0)
    torch.cuda.synchronize()
    assert_close(as_f64(dw.prefill.out), oracle_fp8_prefill(w, kq, vq), "bf16", "fp8 mixed prefill")
    d = w.decode
    want = kv_fp8.decode(d.query, kq, vq, w.host_tables(d.block_tables), d.context_lens, w.scale,
                         K_SCALE, V_SCALE, w.dtype)
    assert_close(as_f64(g.out), want, w.dtype, "fp8 mixed decode")
