"""Pins for the fp64 oracle, against things other than itself.

Each check rests on what the pages or plain mathematics fix: brute force on
tiny inputs (pure-Python loops over the block table), closed forms (a context
of one token returns that token's V; identical keys or a zero query give the
mean of V), a library routine (torch's scaled_dot_product_attention in fp64
when the block table is the identity), invariances the pages state (physical
placement and prefix sharing do not change results: "vLLM 基本原理", sections
"PagedAttention" and "内存共享"), exact identities (split-K merge equals the
unsplit result; chunked prefill equals one-shot causal prefill, xdnf.cn article
section 六.4) and the pages' worked byte counts.

The last group plants plausible mistakes in the oracle and checks that the pins
catch every one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import paged_attention as opa
from workloads import (config0, config4, f32_to_bf16_bits, make_decode, make_prefill,
                       permute_block_ids, unshare_blocks)
from workloads import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_worked_numbers.json")


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def host_pools_after_scatter(w):
    """Host pools (compact ids) with the workload's new tokens written in."""
    k, v = w.k_host, w.v_host
    if w.slot_mapping is not None:
        k, v = oracle.reshape_and_cache(k, v, w.new_k, w.new_v, w.host_slots())
    return k, v


def oracle_decode(w, k=None, v=None):
    if k is None:
        k, v = host_pools_after_scatter(w)
    g = w.decode
    return oracle.decode(g.query, k, v, w.host_tables(g.block_tables), g.context_lens, w.scale,
                         w.dtype)


def brute_decode(query, k_pool, v_pool, tables, lens, scale, bs=16):
    """Triple loop with math.exp, reading the pool through the table by hand."""
    S, hq, d = query.shape
    hkv = k_pool.shape[1]
    out = np.zeros((S, hq, d))
    for s in range(S):
        L = int(lens[s])
        if L == 0:
            continue
        for h in range(hq):
            kh = (h * hkv) // hq
            scores = []
            for t in range(L):
                blk = int(tables[s][t // bs])
                row = t % bs
                dot = 0.0
                for e in range(d):
                    dot += float(query[s, h, e]) * float(k_pool[blk, kh, row, e])
                scores.append(float(scale) * dot)
            top = max(scores)
            ws = [math.exp(x - top) for x in scores]
            tot = sum(ws)
            for e in range(d):
                acc_e = 0.0
                for t in range(L):
                    blk = int(tables[s][t // bs])
                    acc_e += ws[t] * float(v_pool[blk, kh, t % bs, e])
                out[s, h, e] = acc_e / tot
    return out


def brute_prefill(query, k_pool, v_pool, tables, qsl, lens, scale, bs=16):
    tq, hq, d = query.shape
    hkv = k_pool.shape[1]
    out = np.zeros((tq, hq, d))
    for s in range(len(lens)):
        a, b = int(qsl[s]), int(qsl[s + 1])
        C, L = b - a, int(lens[s])
        for i in range(C):
            pos = L - C + i
            o = brute_decode(query[a + i:a + i + 1], k_pool, v_pool, [tables[s]], [pos + 1],
                             scale, bs)
            out[a + i] = o[0]
    return out


def tiny_paged(seed, S=3, hq=4, hkv=2, d=8, nb=12, lens=(5, 17, 33)):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((nb, hkv, 16, d))
    v = rng.standard_normal((nb, hkv, 16, d))
    q = rng.standard_normal((S, hq, d))
    perm = rng.permutation(nb)
    mb = max(-(-L // 16) for L in lens)
    tables = np.full((S, mb), -1, dtype=np.int64)
    pos = 0
    for s, L in enumerate(lens):
        n = -(-L // 16)
        tables[s, :n] = perm[pos:pos + n]
        pos += n
    return q, k, v, tables, np.array(lens), np.float64(1.0 / math.sqrt(d))


# --------------------------------------------------------------------------
# storage decoding
# --------------------------------------------------------------------------
def test_bf16_bit_patterns_decode_exactly():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3F81, 0x0001, 0x7FC0],
                    dtype=np.uint16)
    got = oracle.to_f64(bits, "bf16")
    want = [1.0, -2.0, 0.0, -0.0, math.inf, 1.0 + 2.0 ** -7, 2.0 ** -133]
    assert got[:7].tolist() == want
    assert math.copysign(1.0, got[3]) == -1.0
    assert math.isnan(got[7])


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -1.5,
                  np.nan], dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    vals = oracle.to_f64(bits, "bf16")
    assert vals[0] == 1.0                        # tie -> even mantissa
    assert vals[1] == 1.0 + 2 * 2.0 ** -7        # tie -> even (odd neighbour rounds up)
    assert vals[2] == 1.0 + 2.0 ** -7            # above the tie rounds up
    assert vals[3] == -1.5
    assert math.isnan(vals[4])
    ref = torch.from_numpy(x[:4]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (bits[:4] == ref).all()


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_matches_brute_force(seed):
    q, k, v, t, lens, scale = tiny_paged(seed)
    got = oracle.decode(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), t, lens,
                        scale, "f32")
    want = brute_decode(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), t,
                        lens, scale)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_decode_bf16_matches_brute_force_on_decoded_values():
    q, k, v, t, lens, scale = tiny_paged(7, lens=(1, 16, 40))
    qb, kb, vb = (f32_to_bf16_bits(a.astype(np.float32)) for a in (q, k, v))
    got = oracle.decode(qb, kb, vb, t, lens, scale, "bf16")

    def dec(bits):  # independent bf16 decode: mantissa and exponent by hand
        out = np.zeros(bits.shape)
        for idx, b in np.ndenumerate(bits):
            b = int(b)
            sign = -1.0 if b & 0x8000 else 1.0
            ex = (b >> 7) & 0xFF
            man = b & 0x7F
            out[idx] = sign * (man / 128.0) * 2.0 ** -126 if ex == 0 else \
                sign * (1 + man / 128.0) * 2.0 ** (ex - 127)
        return out

    want = brute_decode(dec(qb), dec(kb), dec(vb), t, lens, scale)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_context_of_one_returns_v_exactly():
    w = config0()
    out = oracle_decode(w)
    k, v = host_pools_after_scatter(w)
    g = w.decode
    s = int(np.nonzero(g.context_lens == 1)[0][0])
    blk = int(w.host_tables(g.block_tables)[s, 0])
    for h in range(w.num_heads):
        want = oracle.to_f64(v[blk, h // w.group, 0, :], w.dtype)
        assert np.array_equal(out[s, h], want)


def test_identical_keys_give_mean_of_v():
    q, k, v, t, lens, scale = tiny_paged(3)
    k[:] = k[0, 0, 0]  # every key row identical
    out = oracle.decode(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), t,
                        lens, scale, "f32")
    v32 = v.astype(np.float32).astype(np.float64)
    for s in range(len(lens)):
        L = lens[s]
        rows = np.stack([v32[t[s, i // 16], :, i % 16, :] for i in range(L)])  # [L, Hkv, D]
        for h in range(q.shape[1]):
            np.testing.assert_allclose(out[s, h], rows[:, h // 2].mean(axis=0), rtol=1e-12,
                                       atol=1e-14)


def test_zero_query_gives_mean_and_constant_v_gives_constant():
    q, k, v, t, lens, scale = tiny_paged(4)
    q[:] = 0.0
    out = oracle.decode(q, k, v, t, lens, scale, "f32")
    for s in range(len(lens)):
        rows = np.stack([v[t[s, i // 16], :, i % 16, :] for i in range(lens[s])])
        np.testing.assert_allclose(out[s, 0], rows[:, 0].astype(np.float32).mean(axis=0),
                                   rtol=1e-6, atol=1e-7)
    q, k, v, t, lens, scale = tiny_paged(5)
    v[:] = 0.625
    out = oracle.decode(q, k, v, t, lens, scale, "f32")
    np.testing.assert_allclose(out, 0.625, rtol=1e-14)


def test_identity_tables_match_torch_sdpa():
    rng = np.random.default_rng(11)
    S, H, D, L = 2, 3, 16, 64
    k = rng.standard_normal((S * L // 16, H, 16, D)).astype(np.float32)
    v = rng.standard_normal((S * L // 16, H, 16, D)).astype(np.float32)
    q = rng.standard_normal((S, H, D)).astype(np.float32)
    tables = np.arange(S * L // 16).reshape(S, L // 16)
    scale = np.float32(1 / math.sqrt(D))
    got = oracle.decode(q, k, v, tables, np.full(S, L), scale, "f32")
    for s in range(S):
        kc = torch.from_numpy(k[tables[s]].astype(np.float64))  # [nb, H, 16, D]
        vc = torch.from_numpy(v[tables[s]].astype(np.float64))
        kc = kc.permute(1, 0, 2, 3).reshape(H, L, D)
        vc = vc.permute(1, 0, 2, 3).reshape(H, L, D)
        qs = torch.from_numpy(q[s].astype(np.float64)).reshape(H, 1, D)
        ref = torch.nn.functional.scaled_dot_product_attention(qs, kc, vc, scale=float(scale))
        np.testing.assert_allclose(got[s], ref.reshape(H, D).numpy(), rtol=1e-12, atol=1e-14)


def test_block_relabelling_is_bit_identical():
    w = config0()
    w2 = permute_block_ids(w, seed=99)
    assert not np.array_equal(w.decode.block_tables, w2.decode.block_tables)
    assert np.array_equal(oracle_decode(w), oracle_decode(w2))


def test_shared_prefix_equals_private_copies():
    w = config4(num_prompts=2, samples=3, shared_prefix=64, max_private=40, num_prefill=1,
                chunk=16, max_prefix=48, num_blocks=64, heads=2, head_dim=16)
    t = w.decode.block_tables
    assert np.array_equal(t[0, :4], t[1, :4]) and np.array_equal(t[1, :4], t[2, :4])
    w2 = unshare_blocks(w)
    t2 = w2.decode.block_tables
    assert len(set(t2[:, :4].ravel().tolist())) == t2.shape[0] * 4
    assert np.array_equal(oracle_decode(w), oracle_decode(w2))


# --------------------------------------------------------------------------
# split-K
# --------------------------------------------------------------------------
@pytest.mark.parametrize("psize", [16, 32, 512, 1 << 20])
def test_splitk_merge_equals_unsplit(psize):
    q, k, v, t, lens, scale = tiny_paged(8, lens=(1, 31, 48))
    whole = oracle.decode(q, k, v, t, lens, scale, "f32")
    o, lse, n = oracle.decode_partials(q, k, v, t, lens, scale, "f32", psize)
    np.testing.assert_allclose(oracle.merge_partials(o, lse, n), whole, rtol=1e-12, atol=1e-14)


def test_partials_match_library_logsumexp():
    from scipy.special import logsumexp
    q, k, v, t, lens, scale = tiny_paged(9, S=1, lens=(40,))
    o, lse, n = oracle.decode_partials(q, k, v, t, lens, scale, "f32", 16)
    assert n.tolist() == [3]
    k32, v32, q32 = (a.astype(np.float32).astype(np.float64) for a in (k, v, q))
    for p in range(3):
        lo, hi = 16 * p, min(40, 16 * p + 16)
        for h in range(q.shape[1]):
            kh = h // 2
            z = np.array([scale * (q32[0, h] @ k32[t[0, i // 16], kh, i % 16]) for i in range(lo, hi)])
            assert abs(lse[0, h, p] - logsumexp(z)) < 1e-12
            vv = np.stack([v32[t[0, i // 16], kh, i % 16] for i in range(lo, hi)])
            np.testing.assert_allclose(o[0, h, p], (np.exp(z - logsumexp(z)) @ vv), rtol=1e-12,
                                       atol=1e-14)


# --------------------------------------------------------------------------
# chunked prefill
# --------------------------------------------------------------------------
def test_prefill_matches_brute_force():
    w = make_prefill("t", 5, "f32", prefix_lens=[0, 13, 40], chunk_lens=[5, 9, 3], hq=4, hkv=2,
                     d=8, num_blocks=16)
    g = w.prefill
    ht = w.host_tables(g.block_tables)
    got = oracle.prefill(g.query, w.k_host, w.v_host, ht, g.query_start_loc, g.context_lens,
                         w.scale, "f32")
    want = brute_prefill(g.query, w.k_host, w.v_host, ht, g.query_start_loc, g.context_lens,
                         w.scale)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_prefill_without_prefix_matches_causal_sdpa():
    w = make_prefill("t", 6, "f32", prefix_lens=[0], chunk_lens=[48], hq=2, hkv=2, d=16,
                     num_blocks=8)
    g = w.prefill
    ht = w.host_tables(g.block_tables)
    got = oracle.prefill(g.query, w.k_host, w.v_host, ht, g.query_start_loc, g.context_lens,
                         w.scale, "f32")
    kc = torch.from_numpy(w.k_host[ht[0, :3]].astype(np.float64)).permute(1, 0, 2, 3).reshape(2, 48, 16)
    vc = torch.from_numpy(w.v_host[ht[0, :3]].astype(np.float64)).permute(1, 0, 2, 3).reshape(2, 48, 16)
    qs = torch.from_numpy(g.query.astype(np.float64)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qs, kc, vc, is_causal=True,
                                                           scale=float(w.scale))
    np.testing.assert_allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-14)


def test_chunked_prefill_page_example_equals_one_shot():
    """12-token prompt, read 4 tokens a round in 3 rounds (xdnf.cn article, 六.4)."""
    ex = json.load(open(GOLDEN))["chunked_prefill"]
    n, c = ex["prompt_tokens"], ex["chunk"]
    assert -(-n // c) == ex["rounds"] and c <= ex["budget"]
    w = make_prefill("t", 12, "f32", prefix_lens=[0], chunk_lens=[n], hq=2, hkv=1, d=8,
                     num_blocks=4)
    g = w.prefill
    ht = w.host_tables(g.block_tables)
    one_shot = oracle.prefill(g.query, w.k_host, w.v_host, ht, g.query_start_loc,
                              g.context_lens, w.scale, "f32")
    for r in range(ex["rounds"]):
        lo, hi = r * c, min(n, (r + 1) * c)
        part = oracle.prefill(g.query[lo:hi], w.k_host, w.v_host, ht, np.array([0, hi - lo]),
                              np.array([hi]), w.scale, "f32")
        np.testing.assert_allclose(part, one_shot[lo:hi], rtol=1e-13, atol=1e-15)


def test_single_token_prefill_equals_decode():
    w = make_prefill("t", 13, "f32", prefix_lens=[20, 0], chunk_lens=[1, 1], hq=4, hkv=2, d=8,
                     num_blocks=8)
    g = w.prefill
    ht = w.host_tables(g.block_tables)
    a = oracle.prefill(g.query, w.k_host, w.v_host, ht, g.query_start_loc, g.context_lens,
                       w.scale, "f32")
    b = oracle.decode(g.query, w.k_host, w.v_host, ht, g.context_lens, w.scale, "f32")
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-15)


# --------------------------------------------------------------------------
# scatter
# --------------------------------------------------------------------------
def test_scatter_round_trip_and_skip():
    w = config0()
    slots = w.host_slots().copy()
    slots[1] = -1  # padding token: nothing written
    k, v = oracle.reshape_and_cache(w.k_host, w.v_host, w.new_k, w.new_v, slots)
    for i, sl in enumerate(slots):
        if sl < 0:
            continue
        b, r = divmod(int(sl), 16)
        assert k[b, :, r, :].tobytes() == w.new_k[i].tobytes()
        assert v[b, :, r, :].tobytes() == w.new_v[i].tobytes()
    touched = np.zeros(k.shape[0] * 16, bool)
    touched[slots[slots >= 0]] = True
    kk = k.transpose(0, 2, 1, 3).reshape(-1, *k.shape[1:2], k.shape[3])
    k0 = w.k_host.transpose(0, 2, 1, 3).reshape(-1, *k.shape[1:2], k.shape[3])
    assert kk[~touched].tobytes() == k0[~touched].tobytes()
    # the skipped token's slot still holds its NaN poison
    b, r = divmod(int(w.host_slots()[1]), 16)
    assert np.isnan(k[b, :, r, :]).all()
    # the written rows read back through the block table as the sequence's newest token
    g = w.decode
    ht = w.host_tables(g.block_tables)
    s = 2
    row = oracle.gather(k, ht[s], g.context_lens[s])[-1]
    assert row.tobytes() == w.new_k[s].tobytes()


# --------------------------------------------------------------------------
# the pages' worked numbers
# --------------------------------------------------------------------------
def test_byte_accounting_reproduces_page_numbers():
    gold = json.load(open(GOLDEN))
    e = gold["llama2_7b_kv"]
    per_layer = acc.kv_cache_bytes(e["seq_len"], e["num_kv_heads"], e["head_dim"], e["elem_bytes"])
    assert per_layer == 64 * 2 ** 20 and round(per_layer / 2 ** 20) == e["per_layer_bytes_printed_MB"]
    total = acc.kv_cache_bytes(e["seq_len"], e["num_kv_heads"], e["head_dim"], e["elem_bytes"],
                               e["num_layers"])
    assert total == 2 * 2 ** 30 and total / 2 ** 30 == e["all_layers_printed_GB"]
    c = gold["a100_concurrency"]
    assert c["gpus"] * c["gb_per_gpu"] // c["gb_per_request"] == c["requests_printed"]
    x = gold["llama13b_kv"]
    b13 = acc.kv_cache_bytes(x["seq_len"], x["num_kv_heads"], x["head_dim"], x["elem_bytes"],
                             x["num_layers"])
    assert round(b13 / 1e9, 1) == x["printed_GB"]
    assert gold["block_size"]["tokens"] == 16


def test_prefill_pair_count_matches_enumeration():
    qsl = [0, 3, 8]
    lens = [10, 5]
    brute = 0
    for s in range(2):
        c = qsl[s + 1] - qsl[s]
        for i in range(c):
            brute += sum(1 for t in range(lens[s]) if t <= lens[s] - c + i)
    assert acc.prefill_pairs(qsl, lens) == brute


# --------------------------------------------------------------------------
# planted mistakes: every one must be caught by a pin above
# --------------------------------------------------------------------------
def _mut_drop_last_token(pool, table_row, length, block_size=16):
    return _orig_gather(pool, table_row, max(0, int(length) - 1), block_size) if length > 1 \
        else _orig_gather(pool, table_row, length, block_size)


def _mut_row_index(pool, table_row, length, block_size=16):
    t = np.arange(int(length))
    phys = np.asarray(table_row)[t // block_size].astype(np.int64)
    return pool[phys, :, (t + 1) % block_size, :]


def _mut_logical_as_physical(pool, table_row, length, block_size=16):
    t = np.arange(int(length))
    return pool[t // block_size, :, t % block_size, :]


def _mut_sign(q, k, v, scale, visible=None):
    return _orig_attend(q, k, v, -scale, visible)


def _mut_transpose(q, k, v, scale, visible=None):
    return _orig_attend(q, v, k, scale, visible)


def _mut_no_scale(q, k, v, scale, visible=None):
    return _orig_attend(q, k, v, 1.0, visible)


def _mut_mask_strict(q, k, v, scale, visible=None):
    if visible is not None:
        visible = np.concatenate([visible[:, 1:], np.zeros((visible.shape[0], 1), bool)], 1) & visible
    return _orig_attend(q, k, v, scale, visible)


_orig_gather = opa.gather
_orig_attend = opa.attend


def _pins_pass():
    """Run a compact set of pins; True if all pass."""
    try:
        for seed in (0, 1):
            test_decode_matches_brute_force(seed)
        test_prefill_matches_brute_force()
        test_identity_tables_match_torch_sdpa()
        test_context_of_one_returns_v_exactly()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("target,mutant", [
    ("gather", _mut_drop_last_token),
    ("gather", _mut_row_index),
    ("gather", _mut_logical_as_physical),
    ("attend", _mut_sign),
    ("attend", _mut_transpose),
    ("attend", _mut_no_scale),
    ("attend", _mut_mask_strict),
])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    assert _pins_pass()
    monkeypatch.setattr(opa, target, mutant)
    assert not _pins_pass(), f"pins missed a planted mistake in {target}: {mutant.__name__}"


def test_planted_head_mapping_mistake_is_caught(monkeypatch):
    """kv head chosen as h % Hkv instead of h // group."""
    def bad_decode(query, k_pool, v_pool, block_tables, context_lens, scale, dtype, block_size=16):
        S, hq, d = query.shape
        hkv = k_pool.shape[1]
        q64 = opa.to_f64(query, dtype)
        out = np.zeros((S, hq, d))
        for s in range(S):
            L = int(context_lens[s])
            ks = opa.to_f64(opa.gather(k_pool, block_tables[s], L, block_size), dtype)
            vs = opa.to_f64(opa.gather(v_pool, block_tables[s], L, block_size), dtype)
            for h in range(hq):
                out[s, h] = opa.attend(q64[s, h][None], ks[:, h % hkv], vs[:, h % hkv], scale)[0]
        return out
    monkeypatch.setattr(oracle, "decode", bad_decode)
    with pytest.raises(AssertionError):
        test_decode_matches_brute_force(0)
