"""Pins of the reference block manager (oracle/block_manager.py) against what
the pages fix: on-demand blocks ("vLLM 基本原理", 按需分配), prompt blocks shared
by forked samples with private blocks for new tokens (内存共享), copy-on-write
through reference counts (intelliparadigm.com article, sections 2.2 and 3.3),
blocks returned when a sequence ends (xdnf.cn article, section 六.1).

The content pin simulates the KV cache: every appended token writes a unique
value into its slot (after the recorded copies are applied), and every
sequence, read back through its block table, must return exactly the values
of its own history -- the tokens it inherited at a fork included.  A manager
that writes into a shared block, loses a copy, or hands one slot to two
sequences fails it.
"""
import numpy as np
import pytest

from oracle.block_manager import BlockManager, OutOfBlocks, copy_blocks, swap_blocks

BS = 16


class Cache:
    """A pool with one value per token slot, driven by a block manager."""

    def __init__(self, bm):
        self.bm = bm
        self.pool = np.full((bm.num_blocks, BS), -1, dtype=np.int64)
        self.hist = {}
        self.next_val = 0

    def add(self, s):
        self.bm.add_sequence(s)
        self.hist[s] = []

    def fork(self, p, c):
        self.bm.fork(p, c)
        self.hist[c] = list(self.hist[p])

    def append(self, s, n):
        slots = self.bm.append_slots(s, n)
        self.pool = copy_blocks(self.pool, self.bm.take_copies())
        for slot in slots:
            self.pool[slot // BS, slot % BS] = self.next_val
            self.hist[s].append(self.next_val)
            self.next_val += 1
        return slots

    def free(self, s):
        self.bm.free_sequence(s)
        del self.hist[s]

    def read(self, s):
        t = self.bm.block_table(s)
        n = self.bm.num_tokens(s)
        return [int(self.pool[t[i // BS], i % BS]) for i in range(n)]

    def check(self):
        self.bm.check_invariants()
        for s in self.hist:
            assert self.read(s) == self.hist[s], s


def test_three_samples_share_prompt_blocks_and_get_private_new_blocks():
    # a prompt of two full blocks, three samples (the "3 different endings" example)
    c = Cache(BlockManager(16))
    c.add(0)
    c.append(0, 32)
    c.fork(0, 1)
    c.fork(0, 2)
    tables = [c.bm.block_table(s) for s in range(3)]
    assert tables[0] == tables[1] == tables[2] == [0, 1]
    assert c.bm.ref[0] == c.bm.ref[1] == 3
    for s in range(3):
        c.append(s, 1)
    assert c.bm.take_copies() == []                 # full shared blocks are never written
    lasts = [c.bm.block_table(s)[-1] for s in range(3)]
    assert len(set(lasts)) == 3 and not set(lasts) & {0, 1}
    assert all(c.bm.block_table(s)[:2] == [0, 1] for s in range(3))
    c.check()


def test_copy_on_write_of_a_partly_filled_shared_block():
    c = Cache(BlockManager(16))
    c.add(0)
    c.append(0, 20)                                 # block 1 holds 4 of 16 rows
    c.fork(0, 1)
    c.fork(0, 2)
    assert c.bm.ref[1] == 3
    c.append(1, 1)                                  # first writer copies
    assert c.bm.block_table(1)[-1] != 1 and c.bm.ref[1] == 2
    c.append(2, 1)                                  # second writer copies
    assert c.bm.block_table(2)[-1] != 1 and c.bm.ref[1] == 1
    c.append(0, 1)                                  # last owner writes in place
    assert c.bm.block_table(0)[-1] == 1
    c.check()


def test_blocks_are_taken_on_demand_only():
    c = Cache(BlockManager(64))
    c.add(0)
    for n in range(1, 100):
        c.append(0, 1)
        assert len(c.bm.block_table(0)) == -(-n // BS)
    assert c.bm.num_free() == 64 - 7
    c.check()


def test_free_returns_blocks_and_reuses_the_most_recent():
    bm = BlockManager(8)
    bm.add_sequence(0)
    bm.append_slots(0, 40)                          # blocks 0, 1, 2
    bm.add_sequence(1)
    bm.append_slots(1, 1)                           # block 3
    bm.free_sequence(0)
    assert bm.num_free() == 7
    bm.add_sequence(2)
    bm.append_slots(2, 17)
    assert bm.block_table(2) == [0, 1]              # LIFO: the freed table's first block first
    bm.check_invariants()


def test_out_of_blocks_changes_nothing():
    bm = BlockManager(4)
    bm.add_sequence(0)
    bm.append_slots(0, 50)                          # 4 blocks
    bm.fork(0, 1)
    before = (list(bm.free), list(bm.ref), bm.block_table(1), bm.num_tokens(1))
    with pytest.raises(OutOfBlocks):
        bm.append_slots(1, 1)                       # needs a copy, pool is empty
    assert (list(bm.free), list(bm.ref), bm.block_table(1), bm.num_tokens(1)) == before


@pytest.mark.parametrize("seed", range(6))
def test_random_workload_keeps_every_sequence_contents(seed):
    rng = np.random.default_rng(seed)
    c = Cache(BlockManager(96))
    live, nxt = [], 0
    for _ in range(400):
        op = rng.integers(0, 10)
        try:
            if op < 2 or not live:
                c.add(nxt)
                live.append(nxt)
                nxt += 1
            elif op < 4:
                p = int(rng.choice(live))
                c.fork(p, nxt)
                live.append(nxt)
                nxt += 1
            elif op < 9:
                c.append(int(rng.choice(live)), int(rng.integers(1, 40)))
            else:
                s = int(rng.choice(live))
                live.remove(s)
                c.free(s)
        except OutOfBlocks:
            pass
        c.check()


def test_planted_write_into_shared_block_is_caught(monkeypatch):
    """A manager without copy-on-write corrupts a sharer's contents."""
    def no_cow(self, seq, n):
        bs = self.block_size
        table = self.tables[seq]
        slots = []
        for _ in range(n):
            pos = self.ntok[seq]
            if pos % bs == 0:
                table.append(self._take())
            slots.append(table[-1] * bs + pos % bs)
            self.ntok[seq] = pos + 1
        return slots
    monkeypatch.setattr(BlockManager, "append_slots", no_cow)
    c = Cache(BlockManager(8))
    c.add(0)
    c.append(0, 5)
    c.fork(0, 1)
    c.append(0, 1)
    c.append(1, 1)
    with pytest.raises(AssertionError):
        c.check()


def test_copy_and_swap_are_plain_block_copies():
    rng = np.random.default_rng(3)
    pool = rng.standard_normal((10, 2, BS, 4)).astype(np.float32)
    out = copy_blocks(pool, [(1, 5), (5, 7), (2, 2)])
    assert np.array_equal(out[5], pool[1]) and np.array_equal(out[7], pool[1])
    assert np.array_equal(out[[0, 1, 2, 3, 4, 6, 8, 9]], pool[[0, 1, 2, 3, 4, 6, 8, 9]])
    host = np.zeros((4, 2, BS, 4), dtype=np.float32)
    h2 = swap_blocks(pool, host, [(9, 0), (3, 2)])
    assert np.array_equal(h2[0], pool[9]) and np.array_equal(h2[2], pool[3])
    assert not h2[[1, 3]].any()
