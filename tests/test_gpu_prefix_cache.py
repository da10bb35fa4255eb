"""Prefix caching end to end on the GPU (xdnf.cn article, section 六.3).

Prompts that share a system prompt go through the native block manager: the
first one is prefilled whole; later ones start on its cached blocks and only
their remaining tokens are scattered and prefilled, attending to the cached
prefix.  A token's K/V here is a fixed function of (token id, position) -- a
stand-in for a model, for which identical prefixes give identical K/V -- so
the chunk prefilled over cached blocks must equal, within the bf16 tolerance,
the oracle's prefill of the same queries over that prompt's own full K/V.
Tables and slots come from the native manager and must equal the reference
manager's, which the oracle side uses.
"""
import numpy as np
import pytest

import oracle
import oracle.block_manager as ref
from pa_harness import as_f64, assert_close, say
from workloads.device import host_to_torch
from workloads.generate import f32_to_bf16_bits

pytestmark = pytest.mark.gpu
BS = 16


class KV:
    """K/V of a token at a position: embedding rows plus position rows (bf16)."""

    def __init__(self, vocab, max_pos, hkv, d, seed):
        rng = np.random.default_rng(seed)
        self.ek = rng.standard_normal((vocab, hkv, d)).astype(np.float32)
        self.ev = rng.standard_normal((vocab, hkv, d)).astype(np.float32)
        self.pk = 0.5 * rng.standard_normal((max_pos, hkv, d)).astype(np.float32)
        self.pv = 0.5 * rng.standard_normal((max_pos, hkv, d)).astype(np.float32)

    def rows(self, tokens, start):
        pos = np.arange(start, start + len(tokens))
        t = np.asarray(tokens)
        return f32_to_bf16_bits(self.ek[t] + self.pk[pos]), f32_to_bf16_bits(self.ev[t] + self.pv[pos])


def test_prefix_hits_skip_prefill_and_match_the_full_prompt(gpu):
    import torch
    say("prefix cache: shared system prompt, GQA 8/2, head_dim 128, bf16")
    hq, hkv, d, nb = 8, 2, 128, 96
    scale = np.float32(1 / np.sqrt(d))
    kv = KV(vocab=50, max_pos=256, hkv=hkv, d=d, seed=3)
    rng = np.random.default_rng(4)
    system = [int(x) for x in rng.integers(0, 50, 70)]
    prompts = {0: (system + [int(x) for x in rng.integers(0, 50, 30)], 1),
               1: (system + [int(x) for x in rng.integers(0, 50, 45)], 1),
               2: (None, 1),                                   # prompt 0 again
               3: (system + [int(x) for x in rng.integers(0, 50, 45)], 2)}   # another salt
    prompts[2] = (prompts[0][0], 1)
    want_cached = {0: 0, 1: 64, 2: 96, 3: 0}

    nat, plain = gpu.BlockManager(nb), ref.BlockManager(nb)
    shape = (nb, hkv, BS, d)
    kc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    kh = np.full(shape, 0x7FC0, dtype=np.uint16)
    vh = kh.copy()
    for s, (toks, salt) in prompts.items():
        c1, c2 = nat.add_prompt(s, toks, salt), plain.add_prompt(s, toks, salt)
        assert c1 == c2 == want_cached[s], (s, c1, c2)
        rest = toks[c1:]
        sl1, sl2 = nat.append_tokens(s, rest), plain.append_tokens(s, rest)
        assert [int(x) for x in sl1] == sl2
        assert [tuple(m) for m in nat.take_moves()[0].tolist()] == plain.take_moves()[0] == []
        # scatter only the tokens the cache did not cover
        k_new, v_new = kv.rows(rest, c1)
        gpu.pa_reshape_and_cache(host_to_torch(k_new, "bf16", "cuda"),
                                 host_to_torch(v_new, "bf16", "cuda"), kc, vc,
                                 torch.tensor(sl2, dtype=torch.int64, device="cuda"))
        kh, vh = oracle.reshape_and_cache(kh, vh, k_new, v_new, np.array(sl2))
        # prefill the uncovered chunk over the whole context
        table = plain.block_table(s)
        tables, lens, _ = nat.build_batch([s], len(table))
        assert tables[0].tolist() == table and int(lens[0]) == len(toks)
        q = f32_to_bf16_bits(rng.standard_normal((len(rest), hq, d)).astype(np.float32))
        qt = host_to_torch(q, "bf16", "cuda")
        out = torch.empty_like(qt)
        qsl = torch.tensor([0, len(rest)], dtype=torch.int32, device="cuda")
        gpu.pa_prefill_chunk(out, qt, kc, vc, torch.from_numpy(tables).cuda(), qsl,
                             torch.from_numpy(lens).cuda(), float(scale), len(rest))
        torch.cuda.synchronize()
        got = as_f64(out)
        qsl_h = np.array([0, len(rest)], dtype=np.int32)
        via_cache = oracle.prefill(q, kh, vh, np.array([table]), qsl_h, lens, scale, "bf16")
        # the same queries over the prompt's own K/V, no cache involved
        kf, vf = kv.rows(toks, 0)
        nfb = -(-len(toks) // BS)
        kp = np.full((nfb, hkv, BS, d), 0x7FC0, dtype=np.uint16)
        vp = kp.copy()
        kp, vp = oracle.reshape_and_cache(kp, vp, kf, vf, np.arange(len(toks)))
        direct = oracle.prefill(q, kp, vp, np.array([np.arange(nfb)]), qsl_h, lens, scale, "bf16")
        np.testing.assert_array_equal(via_cache, direct)      # the cache is exact
        assert_close(got, direct, "bf16", f"prompt {s} over {c1} cached tokens")
    assert nat.num_cached_blocks() == plain.num_cached_blocks()
    nat.check_invariants()
