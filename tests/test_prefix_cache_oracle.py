"""Pins of the reference prefix cache (oracle/block_manager.py, readings P1-P5).

xdnf.cn article, section 六.3: every full KV block gets a hash; a new request
whose prefix blocks hit reuses them and skips their prefill; a hit needs the
same model / precision / quantisation / adapter (the salt here), identical
tokens from position 0, and whole blocks.

The hash is pinned on FNV-1a's published test vectors.  The content pin
simulates a model: the KV "value" of a token is a function of the salt and of
the sequence's whole prefix up to it, so a block may be reused only by a
sequence whose prefix is identical token for token under the same salt.
Every sequence, read back through its table, must return its own values --
shared, revived, evicted, copied and swapped blocks included.
"""
import numpy as np
import pytest

import oracle.block_manager as ref
from oracle.block_manager import BlockManager, Busy, OutOfBlocks, block_key, fnv1a64, prefix_keys

BS = 16


def test_fnv1a64_published_vectors():
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def test_keys_are_chained_over_whole_blocks():
    rng = np.random.default_rng(0)
    t = [int(x) for x in rng.integers(0, 1000, 100)]
    k = prefix_keys(t, salt=7)
    assert len(k) == 6                                    # 100 tokens: 6 full blocks, tail ignored
    assert prefix_keys(t[:64], 7) == k[:4]                # a prefix has the same first keys
    u = list(t)
    u[40] += 1                                            # a token in block 2
    ku = prefix_keys(u, 7)
    assert ku[:2] == k[:2] and all(a != b for a, b in zip(ku[2:], k[2:]))
    assert all(a != b for a, b in zip(prefix_keys(t, 8), k))   # another salt: every key differs
    assert block_key(0, 7, t[:16]) == k[0]


def _value(salt, prefix):
    return hash((salt,) + tuple(prefix)) & 0x7FFFFFFF


class PCache:
    """Device / host pools of token values, driven by prompts through the reference manager."""

    def __init__(self, nb, nh=0, seed=0):
        self.bm = BlockManager(nb, BS, nh)
        self.dev = np.full((nb, BS), -1, dtype=np.int64)
        self.host = np.full((max(nh, 1), BS), -1, dtype=np.int64)
        self.hist = {}
        self.writes = []
        self.hits = 0
        self.rng = np.random.default_rng(seed)

    def _append(self, s, tokens):
        slots = self.bm.append_tokens(s, tokens)
        toks = self.bm.tok[s]
        salt = self.bm.salt[s]
        start = len(toks) - len(tokens)
        for i, slot in enumerate(slots):
            v = _value(salt, toks[:start + i + 1])
            self.writes.append((s, slot, v))
            self.hist[s].append(v)

    def add_prompt(self, s, tokens, salt):
        n = self.bm.add_prompt(s, tokens, salt)
        self.hits += n
        self.hist[s] = [_value(salt, tokens[:i + 1]) for i in range(n)]
        if len(tokens) > n:
            self._append(s, tokens[n:])
        return n

    def decode(self, s, tokens):
        self._append(s, tokens)

    def fork(self, p, c):
        self.bm.fork(p, c)
        self.hist[c] = list(self.hist[p])

    def free(self, s):
        self.bm.free_sequence(s)
        del self.hist[s]
        self.writes = [w for w in self.writes if w[0] != s]

    def step(self):
        copies, outs, ins = self.bm.take_moves()
        for src, dst in copies:
            self.dev[dst] = self.dev[src]
        for src, dst in outs:
            self.host[dst] = self.dev[src]
        for src, dst in ins:
            self.dev[dst] = self.host[src]
        for _, slot, v in self.writes:
            self.dev[slot // BS, slot % BS] = v
        self.writes = []

    def check(self):
        self.bm.check_invariants()
        for s, h in self.hist.items():
            pool = self.host if self.bm.is_swapped(s) else self.dev
            t = self.bm.block_table(s)
            got = [int(pool[t[i // BS], i % BS]) for i in range(self.bm.num_tokens(s))]
            assert got == h, s


def test_shared_prefix_is_reused_in_whole_blocks():
    c = PCache(32)
    sys_prompt = list(range(100, 140))                   # 40 tokens: 2 full blocks
    a = sys_prompt + [1, 2, 3]
    b = sys_prompt + [4, 5, 6, 7]
    assert c.add_prompt(0, a, salt=1) == 0
    c.step()
    assert c.bm.num_cached_blocks() == 2                  # the partly filled third block is not
    assert c.add_prompt(1, b, salt=1) == 32
    assert c.bm.block_table(1)[:2] == c.bm.block_table(0)[:2]
    assert c.add_prompt(2, b, salt=2) == 0                # another salt: no hit
    d = list(b)
    d[20] = 0                                             # differs inside block 1
    assert c.add_prompt(3, d, salt=1) == 16
    c.step()
    c.check()


def test_last_prompt_token_is_always_computed():
    c = PCache(16)
    p = list(range(48))
    c.add_prompt(0, p, 0)
    c.step()
    assert c.bm.num_cached_blocks() == 3
    assert c.add_prompt(1, p, 0) == 32                    # 48 tokens: at most 2 blocks reused
    assert c.add_prompt(2, p + [99], 0) == 48
    c.step()
    c.check()


def test_cached_blocks_outlive_their_sequence_and_are_evicted_oldest_first():
    c = PCache(8)
    a, b = list(range(33)), list(range(500, 533))
    c.add_prompt(0, a, 0)                                 # 2 full blocks cached + 1 partly filled
    c.add_prompt(1, b, 0)
    c.step()
    c.free(0)
    c.free(1)
    assert c.bm.num_free() == 8 and c.bm.num_cached_blocks() == 4
    c.add_prompt(2, list(range(900, 948)), 0)             # 3 blocks: the uncached idle ones first
    c.step()
    assert len(c.bm._lookup(a, 0, 2)[0]) == 2 and len(c.bm._lookup(b, 0, 2)[0]) == 2
    c.add_prompt(3, list(range(700, 717)), 0)             # 2 blocks: 1 uncached, then 1 eviction
    c.step()
    # the cached block released longest ago is prompt 0's second block (tables are
    # released last entry first)
    assert len(c.bm._lookup(a, 0, 2)[0]) == 1 and len(c.bm._lookup(b, 0, 2)[0]) == 2
    c.check()


def test_revived_block_is_the_same_physical_block():
    c = PCache(16)
    c.add_prompt(0, list(range(40)), 5)
    c.step()
    t0 = c.bm.block_table(0)
    c.free(0)
    assert c.add_prompt(1, list(range(40)) + [7], 5) == 32
    assert c.bm.block_table(1)[:2] == t0[:2]
    c.step()
    c.check()


def test_colliding_key_is_taken_over_without_false_sharing(monkeypatch):
    real = ref.block_key
    monkeypatch.setattr(ref, "block_key",
                        lambda parent, salt, toks: 42 if toks[0] in (1000, 2000) else
                        real(parent, salt, toks))
    c = PCache(16)
    a = [1000] + list(range(16))
    b = [2000] + list(range(16))
    c.add_prompt(0, a, 0)
    c.step()
    c.add_prompt(1, b, 0)                                 # same key, other tokens: a miss
    c.step()
    assert c.bm.cache[42] == c.bm.block_table(1)[0]       # the newer block took the key over
    assert len(c.bm._lookup(a, 0, 1)[0]) == 0             # a is not served b's block
    assert c.add_prompt(3, b, 0) == 16
    c.step()
    c.check()


def test_blocks_filled_in_a_batch_are_reused_from_the_next_one():
    c = PCache(16)
    p = list(range(20))                                   # block 0 full, block 1 holds 4
    c.add_prompt(0, p, 0)
    assert c.add_prompt(1, p, 0) == 0                     # block 0 is not written yet
    c.step()
    c.fork(0, 2)
    c.decode(2, list(range(50, 62)))                      # a copy of block 1, filled to 16
    q = p + list(range(50, 62)) + [1]
    assert c.add_prompt(3, q, 0) == 16                    # neither copied nor written yet
    c.step()
    assert c.add_prompt(4, q, 0) == 32
    c.step()
    c.check()


def test_sequence_freed_before_its_tokens_are_written_caches_nothing():
    c = PCache(16)
    c.add_prompt(0, list(range(40)), 0)
    c.free(0)                                             # in the same batch
    c.step()
    assert c.bm.num_cached_blocks() == 0
    assert c.add_prompt(1, list(range(40)), 0) == 0
    c.step()
    c.check()


@pytest.mark.parametrize("seed", range(6))
def test_random_prompts_keep_every_sequence_contents(seed):
    rng = np.random.default_rng(seed)
    c = PCache(64, nh=24, seed=seed)
    systems = [[int(x) for x in rng.integers(0, 50, int(rng.integers(10, 70)))] for _ in range(4)]
    nxt, evictions = 0, 0
    orig = c.bm._evict

    def counting(b):
        nonlocal evictions
        evictions += 1
        orig(b)
    c.bm.dev.evict = counting
    for _ in range(150):
        for _ in range(int(rng.integers(1, 6))):
            live = sorted(c.hist)
            res = [s for s in live if not c.bm.is_swapped(s)]
            clean = [s for s in res if s not in c.bm.dirty]
            op = int(rng.integers(0, 10))
            try:
                if op < 3 or not res:
                    sysp = systems[int(rng.integers(0, 4))]
                    tail = [int(x) for x in rng.integers(0, 50, int(rng.integers(0, 25)))]
                    nxt += 1
                    c.add_prompt(nxt - 1, sysp + tail, int(rng.integers(0, 2)))
                elif op < 6:
                    s = int(rng.choice(res))
                    c.decode(s, [int(x) for x in rng.integers(0, 50, int(rng.integers(1, 6)))])
                elif op == 6 and clean:
                    nxt += 1
                    c.fork(int(rng.choice(clean)), nxt - 1)
                elif op == 7:
                    c.free(int(rng.choice(live)))
                elif op == 8 and clean:
                    c.bm.swap_out([int(rng.choice(clean))])
                elif op == 9:
                    sw = [s for s in live if c.bm.is_swapped(s)]
                    if sw:
                        c.bm.swap_in([int(rng.choice(sw))])
            except (OutOfBlocks, Busy):
                pass
        c.step()
        c.check()
    assert c.hits > 0 and evictions > 0


def test_planted_key_only_lookup_is_caught(monkeypatch):
    """Trusting the key without comparing tokens, with a weak hash, shares a
    block between prompts that differ -- the contents catch it."""
    monkeypatch.setattr(ref, "block_key", lambda parent, salt, toks: hash((parent, toks[0])))

    def trusting(self, tokens, salt, max_blocks):
        hits, keys, key = [], [], 0
        for j in range(max_blocks):
            key = ref.block_key(key, salt, tuple(tokens[j * BS:(j + 1) * BS]))
            b = self.cache.get(key)
            if b is None:
                break
            hits.append(b)
            keys.append(key)
        return hits, keys
    monkeypatch.setattr(BlockManager, "_lookup", trusting)
    c = PCache(16)
    c.add_prompt(0, [5] + list(range(30)), 0)
    c.step()
    c.add_prompt(1, [5] + list(range(100, 130)), 0)       # same first token of block 0 only
    c.step()
    with pytest.raises(AssertionError):
        c.check()
