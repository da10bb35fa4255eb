"""Pins of the reference block manager (oracle/block_manager.py) against what
the pages fix: on-demand blocks ("vLLM 基本原理", 按需分配), prompt blocks shared
by forked samples with private blocks for new tokens (内存共享), copy-on-write
through reference counts (intelliparadigm.com article, sections 2.2 and 3.3),
the three sharing modes (same article, section 2.3), blocks returned when a
sequence ends (xdnf.cn article, section 六.1), swap space in host memory
(intelliparadigm.com article, section 5.1).

The content pin simulates the KV cache in steps: every appended token gets a
unique value; at the end of a step the recorded moves run (in a random order)
and then the reserved slots are written.  Every sequence, read back through
its block table from the pool it lives in, must return exactly the values of
its own history -- the tokens it inherited when it was forked or shared
included.  A manager that writes into a shared block, loses or misorders a
copy, reuses a block a pending move still needs, or hands one slot to two
sequences fails it.
"""
import copy

import numpy as np
import pytest

from oracle.block_manager import (BlockManager, Busy, OutOfBlocks, _Pool, copy_blocks,
                                  swap_blocks)

BS = 16


class Cache:
    """Device and host pools with one value per token slot, driven by a block
    manager step by step."""

    def __init__(self, bm, seed=0):
        self.bm = bm
        self.dev = np.full((bm.num_blocks, BS), -1, dtype=np.int64)
        self.host = np.full((max(bm.num_host_blocks, 1), BS), -1, dtype=np.int64)
        self.hist = {}
        self.writes = {}
        self.next_val = 0
        self.rng = np.random.default_rng(seed)

    def add(self, s):
        self.bm.add_sequence(s)
        self.hist[s] = []

    def fork(self, p, c):
        self.bm.fork(p, c)
        self.hist[c] = list(self.hist[p])

    def share(self, src, dst, idx):
        self.bm.share(src, dst, idx)
        self.hist[dst] = [v for i in idx for v in self.hist[src][i * BS:(i + 1) * BS]]

    def append(self, s, n):
        slots = self.bm.append_slots(s, n)
        for slot in slots:
            self.writes.setdefault(s, []).append((slot, self.next_val))
            self.hist[s].append(self.next_val)
            self.next_val += 1
        return slots

    def free(self, s):
        self.bm.free_sequence(s)
        del self.hist[s]
        self.writes.pop(s, None)

    def step(self):
        """Run the step's moves in a random order, then write the reserved slots."""
        copies, outs, ins = self.bm.take_moves()
        work = [("c", p) for p in copies] + [("o", p) for p in outs] + [("i", p) for p in ins]
        for k in self.rng.permutation(len(work)):
            kind, (src, dst) = work[k]
            if kind == "c":
                self.dev = copy_blocks(self.dev, [(src, dst)])
            elif kind == "o":
                self.host = swap_blocks(self.dev, self.host, [(src, dst)])
            else:
                self.dev = swap_blocks(self.host, self.dev, [(src, dst)])
        for s, ws in self.writes.items():
            for slot, v in ws:
                self.dev[slot // BS, slot % BS] = v
        self.writes = {}

    def read(self, s):
        pool = self.host if self.bm.is_swapped(s) else self.dev
        t = self.bm.block_table(s)
        return [int(pool[t[i // BS], i % BS]) for i in range(self.bm.num_tokens(s))]

    def check(self):
        self.bm.check_invariants()
        self.check_contents()

    def check_contents(self):
        for s in self.hist:
            assert self.read(s) == self.hist[s], s


def _data(d):
    return {k: v for k, v in d.items() if not callable(v)}


def _state(bm):
    return copy.deepcopy((_data(bm.dev.__dict__), _data(bm.host.__dict__), bm.tables, bm.ntok,
                          bm.on_host, bm.dirty, bm.copies, bm.swapped_out, bm.swapped_in,
                          bm.cache, bm.meta, bm.tok, bm.salt, bm.keys, bm.serial, bm.to_register))


def run_random_workload(seed, steps=120, num_blocks=96, num_host_blocks=48):
    rng = np.random.default_rng(seed)
    c = Cache(BlockManager(num_blocks, BS, num_host_blocks), seed)
    bm = c.bm
    nxt = 0
    refused = {"out": 0, "busy": 0}
    for _ in range(steps):
        for _ in range(int(rng.integers(1, 8))):
            live = sorted(c.hist)
            res = [s for s in live if not bm.is_swapped(s)]
            swapped = [s for s in live if bm.is_swapped(s)]
            clean = [s for s in res if s not in bm.dirty]
            op = int(rng.integers(0, 12))
            before = _state(bm)
            try:
                if op == 0 or not res:
                    c.add(nxt)
                    nxt += 1
                elif op == 1 and clean:
                    c.fork(int(rng.choice(clean)), nxt)
                    nxt += 1
                elif op == 2 and clean:
                    src = int(rng.choice(clean))
                    full = bm.num_tokens(src) // BS
                    if full:
                        if rng.integers(0, 2):
                            idx = list(range(int(rng.integers(1, full + 1))))
                        else:
                            idx = [int(i) for i in rng.choice(full, int(rng.integers(1, full + 1)))]
                        c.share(src, nxt, idx)
                        nxt += 1
                elif op < 8:
                    c.append(int(rng.choice(res)), int(rng.integers(1, 40)))
                elif op == 8:
                    c.free(int(rng.choice(live)))
                elif op == 9 and clean:
                    k = int(rng.integers(1, min(3, len(clean)) + 1))
                    bm.swap_out([int(x) for x in rng.choice(clean, k, replace=False)])
                elif op == 10 and swapped:
                    k = int(rng.integers(1, min(3, len(swapped)) + 1))
                    bm.swap_in([int(x) for x in rng.choice(swapped, k, replace=False)])
            except (OutOfBlocks, Busy) as e:
                refused["out" if isinstance(e, OutOfBlocks) else "busy"] += 1
                assert _state(bm) == before          # all-or-nothing
        c.step()
        c.check()
    return refused


def test_three_samples_share_prompt_blocks_and_get_private_new_blocks():
    # a prompt of two full blocks, three samples (the "3 different endings" example)
    c = Cache(BlockManager(16))
    c.add(0)
    c.append(0, 32)
    c.step()
    c.fork(0, 1)
    c.fork(0, 2)
    tables = [c.bm.block_table(s) for s in range(3)]
    assert tables[0] == tables[1] == tables[2] == [0, 1]
    assert c.bm.ref[0] == c.bm.ref[1] == 3
    assert [c.bm.shared_prefix_blocks(s) for s in range(3)] == [2, 2, 2]
    for s in range(3):
        c.append(s, 1)
    assert c.bm.take_copies() == []                 # full shared blocks are never written
    lasts = [c.bm.block_table(s)[-1] for s in range(3)]
    assert len(set(lasts)) == 3 and not set(lasts) & {0, 1}
    assert all(c.bm.block_table(s)[:2] == [0, 1] for s in range(3))
    c.step()
    c.check()


def test_copy_on_write_of_a_partly_filled_shared_block():
    c = Cache(BlockManager(16))
    c.add(0)
    c.append(0, 20)                                 # block 1 holds 4 of 16 rows
    c.step()
    c.fork(0, 1)
    c.fork(0, 2)
    assert c.bm.ref[1] == 3
    c.append(1, 1)                                  # first writer copies
    assert c.bm.block_table(1)[-1] != 1 and c.bm.ref[1] == 2
    c.append(2, 1)                                  # second writer copies
    assert c.bm.block_table(2)[-1] != 1 and c.bm.ref[1] == 1
    c.append(0, 1)                                  # last owner writes in place
    assert c.bm.block_table(0)[-1] == 1
    copies, _, _ = c.bm.take_moves()
    assert copies == [(1, c.bm.block_table(1)[-1]), (1, c.bm.block_table(2)[-1])]
    c.bm.copies = copies                            # hand them back to step()
    c.step()
    c.check()


def test_blocks_are_taken_on_demand_only():
    c = Cache(BlockManager(64))
    c.add(0)
    for n in range(1, 100):
        c.append(0, 1)
        assert len(c.bm.block_table(0)) == -(-n // BS)
    assert c.bm.num_free() == 64 - 7
    c.step()
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
    bm.take_moves()
    bm.fork(0, 1)
    before = _state(bm)
    with pytest.raises(OutOfBlocks):
        bm.append_slots(1, 1)                       # needs a copy, pool is empty
    assert _state(bm) == before


def test_prefix_and_selected_block_sharing():
    c = Cache(BlockManager(32))
    c.add(0)
    c.append(0, 6 * BS + 3)
    c.step()
    t0 = c.bm.block_table(0)
    c.share(0, 1, [0, 1, 2])                        # a prefix of three blocks
    c.share(0, 2, [0, 3, 5])                        # chosen logical blocks
    assert c.bm.block_table(1) == t0[:3] and c.bm.num_tokens(1) == 3 * BS
    assert c.bm.block_table(2) == [t0[0], t0[3], t0[5]] and c.bm.num_tokens(2) == 3 * BS
    assert c.bm.ref[t0[0]] == 3 and c.bm.ref[t0[4]] == 1
    assert c.bm.shared_prefix_blocks(2) == 3
    assert c.bm.shared_prefix_blocks(0) == 4        # t0[4] is its own; counting stops there
    with pytest.raises(ValueError):
        c.bm.share(0, 3, [6])                       # the partly filled last block
    c.append(2, 1)                                  # full last block: a new block, no copy
    assert c.bm.take_moves() == ([], [], [])
    c.step()
    c.check()


def test_reserved_slots_block_forks_until_moves_are_taken():
    bm = BlockManager(8)
    bm.add_sequence(0)
    bm.append_slots(0, 5)
    with pytest.raises(Busy):
        bm.fork(0, 1)
    with pytest.raises(Busy):
        bm.swap_out([0])
    bm.take_moves()
    bm.fork(0, 1)


def test_copy_source_still_arriving_is_refused():
    bm = BlockManager(8, BS, 4)
    bm.add_sequence(0)
    bm.append_slots(0, 5)
    bm.take_moves()
    bm.swap_out([0])
    bm.take_moves()
    bm.swap_in([0])                                 # its block is now a pending destination
    bm.fork(0, 1)
    before = _state(bm)
    with pytest.raises(Busy):
        bm.append_slots(1, 1)                       # would copy a block not yet filled
    assert _state(bm) == before
    bm.take_moves()
    bm.append_slots(1, 1)


def test_swap_keeps_sharing_inside_one_call():
    c = Cache(BlockManager(16, BS, 16))
    c.add(0)
    c.append(0, 40)
    c.step()
    c.fork(0, 1)
    c.fork(0, 2)
    c.bm.swap_out([0, 1])
    _, outs, _ = c.bm.take_moves()
    assert len(outs) == 3                           # each distinct block once
    assert c.bm.block_table(0) == c.bm.block_table(1)
    assert c.bm.ref[c.bm.block_table(2)[0]] == 1    # the device blocks stay with sample 2
    c.bm.swapped_out = outs
    c.step()
    c.check()
    c.bm.swap_in([1])
    c.step()
    c.check()


@pytest.mark.parametrize("seed", range(8))
def test_random_workload_keeps_every_sequence_contents(seed):
    run_random_workload(seed)


def test_random_workloads_reach_every_refusal():
    tot = {"out": 0, "busy": 0}
    for seed in range(8):
        r = run_random_workload(seed, steps=60, num_blocks=40, num_host_blocks=16)
        tot = {k: tot[k] + r[k] for k in tot}
    assert tot["out"] > 0 and tot["busy"] > 0


def test_planted_write_into_shared_block_is_caught(monkeypatch):
    """A manager without copy-on-write corrupts a sharer's contents."""
    def no_cow(self, seq, n):
        bs = self.block_size
        table = self.tables[seq]
        slots = []
        for _ in range(n):
            pos = self.ntok[seq]
            if pos % bs == 0:
                table.append(self.dev.take())
            slots.append(table[-1] * bs + pos % bs)
            self.ntok[seq] = pos + 1
        return slots
    monkeypatch.setattr(BlockManager, "append_slots", no_cow)
    c = Cache(BlockManager(8))
    c.add(0)
    c.append(0, 5)
    c.step()
    c.fork(0, 1)
    c.append(0, 1)
    c.append(1, 1)
    c.step()
    c.bm.check_invariants()                         # the bookkeeping alone looks fine
    with pytest.raises(AssertionError):
        c.check_contents()


def test_planted_early_release_is_caught(monkeypatch):
    """Without holding back blocks of pending moves, a later allocation in the
    same step reuses a block a move still reads or writes."""
    def eager(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)
    monkeypatch.setattr(_Pool, "release", eager)
    caught = 0
    for seed in range(8):
        try:
            run_random_workload(seed, steps=60)
        except AssertionError:
            caught += 1
    assert caught > 0


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


def test_prefix_groups_of_forked_samples_and_shared_prefixes():
    """Sharing groups for the grouped decode, worked by hand: seq 0 has three
    full blocks and two forked samples (one of which has moved on to a fourth,
    private block), seq 4 shares seq 3's first block, seq 5 shares nothing."""
    bm = BlockManager(32, 16)
    bm.add_sequence(0)
    bm.append_slots(0, 48)
    bm.take_moves()
    bm.fork(0, 1)
    bm.fork(0, 2)
    bm.take_moves()
    bm.append_slots(1, 1)                    # a fourth block, private to seq 1
    bm.add_sequence(3)
    bm.append_slots(3, 20)
    bm.take_moves()
    bm.share(3, 4, [0])
    bm.add_sequence(5)
    bm.append_slots(5, 5)
    bm.add_sequence(6)                       # no blocks yet
    bm.take_moves()
    t = {s: bm.block_table(s) for s in range(7) if s != 6}
    assert t[1][:3] == t[0] == t[2] and len(t[1]) == 4 and t[4] == t[3][:1]
    assert bm.prefix_groups([0, 1, 2, 3, 4, 5]) == ([0, 0, 0, 3, 3, 5], [3, 3, 3, 1, 1, 0], 3)
    # a group is a run of neighbours: seq 2 after seq 5 starts a run of its own
    assert bm.prefix_groups([1, 0, 5, 2]) == ([0, 0, 2, 3], [3, 3, 0, 0], 2)
    # an empty table leads nobody and joins nobody
    assert bm.prefix_groups([6, 0, 6]) == ([0, 1, 2], [0, 0, 0], 1)
    assert bm.prefix_groups([]) == ([], [], 0)
    with pytest.raises(KeyError):
        bm.prefix_groups([0, 99])
