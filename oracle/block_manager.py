"""Plain reference of the paged KV cache's block manager and its data movement.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the tests use it.  It shares no code with the native
block manager or the GPU kernels.

What it models, and the passages it follows (page titles as printed):

* A fixed pool of physical blocks of block_size token slots; each sequence owns
  a block table mapping its logical blocks to physical ones ("vLLM 基本原理",
  section "PagedAttention", items 1-3).
* On-demand allocation: a sequence takes a new physical block only when its
  last block is full, so only the last block may be partly filled ("vLLM
  基本原理", "按需分配").
* Sharing: samples forked from one prompt point at the prompt's physical
  blocks; new tokens go to private blocks ("vLLM 基本原理", "内存共享").
  Shared blocks carry a reference count, and a write into a shared block
  copies it first (intelliparadigm.com article, section 2.2: RefCounter for
  copy-on-write; section 3.3: with reference counts only a writer that still
  shares the block copies it -- the last owner writes in place).
* Three sharing modes (intelliparadigm.com article, section 2.3): a whole
  sequence (fork), its first n blocks (a prefix), or chosen logical blocks.
* A finished sequence returns its blocks at once (xdnf.cn article, section
  六.1).
* Swap space: a second pool in host memory (intelliparadigm.com article,
  section 5.1, the swap-space setting); a swapped-out sequence's blocks are
  copied there and its device blocks released, and swapping in reverses it.

Readings where the pages leave the policy open (the native manager follows the
same ones, so tables can be compared exactly; the invariants hold for any
policy):
* R1  Free blocks form a stack: allocation takes the most recently released
      block; initially blocks come out in increasing id order.
* R2  Releasing a table goes from its last entry to its first, so the first
      block is the next to be reused.
* R3  Every operation is all-or-nothing: if a pool cannot supply every block
      it needs, nothing changes and OutOfBlocks is raised.
* R4  Only a partly filled shared last block is copied on write; full shared
      blocks stay shared (nothing is written into them again).
* R5  Prefix and selected-block sharing take whole (full) blocks only -- a
      cached prefix is reused in whole blocks (xdnf.cn article, section 六.3)
      and only a last block may be partly filled.  The new sequence's table is
      the chosen blocks in the order given.
* R6  Data movement is recorded as (src, dst) pairs -- copies within the
      device pool, swap-outs device -> host, swap-ins host -> device -- and
      handed out by take_moves().  Until then, a block named by a pending pair
      that drops to reference count 0 is held back from its free stack and
      pushed (in release order) by take_moves().  So no destination of a batch
      is reused, and no source overwritten, before the batch has run.
* R7  An operation whose source block is the destination of a pending pair
      (its contents not there yet) is refused with Busy, changing nothing.
  With R6 and R7 the pairs of one batch have distinct destinations, none of
  them a source of the batch: they can run in any order, or all at once.
* R8  Swapping a list of sequences maps each distinct block once: sequences
      of the list that shared a block share its copy.  Only resident
      sequences fork, share, append or swap out; only swapped-out ones swap in.
* R9  The tokens reserved by append_slots are written by the caller after the
      batch's moves have run.  Until the next take_moves(), a sequence that
      reserved slots cannot be forked, shared from or swapped out (Busy): a
      copy of its blocks would miss those tokens.

Prefix caching (xdnf.cn article, section 六.3: a hash per KV block; a new
request whose prefix blocks hit reuses them and skips their prefill; a hit
needs the same model, precision, quantisation and adapter, the same tokens
from position 0, and whole blocks -- a partial tail is never reused):
* P1  A block's key is a chained hash: FNV-1a 64 over (the previous block's
      key, the cache salt, the block's 16 token ids), little-endian, with key
      0 before the first block.  The salt stands for everything besides the
      tokens that must match (model, precision, quantisation, adapter).
* P2  A sequence's full blocks enter the cache when they fill with known
      tokens (append_tokens) -- at the end of that batch (take_moves), once
      the caller is committed to writing them, and only if the sequence that
      filled the block still holds it (a sequence freed in the same batch
      never writes its tokens).  A hit is verified exactly, not by the key
      alone: same salt, same 16 tokens, and a parent that is the block the
      previous hit matched (none for the first), so a prefix is shared only if
      it is identical token for token.  A key whose entry fails that check is
      taken over by the newly filled block.
* P3  A prompt reuses at most the full blocks before its last token, which
      is always left to compute.
* P4  A cached block nobody holds stays cached.  Allocation takes blocks
      without cached contents first (R1); only when none is left it evicts
      the cached block released longest ago.
* P5  Only sequences created from a prompt (add_prompt) or forked from one
      know their tokens and fill the cache; shares of chosen blocks and blocks
      brought back by a swap-in are never entered.

Data movement: copy_blocks copies whole physical blocks within a pool (the
copy-on-write step); swap_blocks copies whole blocks between two pools (device
and host).  A physical block of a [num_blocks, num_heads, block_size,
head_dim] pool is one contiguous run of num_heads * block_size * head_dim
elements.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np


class OutOfBlocks(RuntimeError):
    pass


class Busy(RuntimeError):
    pass


FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3


def fnv1a64(data: bytes, h: int = FNV64_OFFSET) -> int:
    """FNV-1a, 64 bits: for each byte, xor it in, then multiply by the prime."""
    for byte in data:
        h ^= byte
        h = (h * FNV64_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def block_key(parent_key: int, salt: int, tokens) -> int:
    """Chained key of one full block (P1)."""
    data = (int(parent_key).to_bytes(8, "little") + (int(salt) & (2**64 - 1)).to_bytes(8, "little")
            + b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens))
    return fnv1a64(data)


def prefix_keys(tokens, salt: int = 0, block_size: int = 16) -> List[int]:
    """Keys of all full blocks of a token sequence."""
    keys, key = [], 0
    for j in range(len(tokens) // block_size):
        key = block_key(key, salt, tokens[j * block_size:(j + 1) * block_size])
        keys.append(key)
    return keys


class _Pool:
    """Free stack and reference counts of one pool."""

    def __init__(self, n: int):
        self.free: List[int] = list(range(n - 1, -1, -1))    # top = end of list
        self.lru: List[int] = []                             # idle cached blocks, oldest first (P4)
        self.ref = [0] * n
        self.held: List[int] = []                            # released while pending (R6)
        self.pending: set = set()                            # named by a pending pair
        self.pending_dst: set = set()
        self.is_cached = lambda b: False
        self.evict = lambda b: None

    def num_idle(self) -> int:
        return len(self.free) + len(self.lru)

    def take(self) -> int:
        if self.free:
            b = self.free.pop()
        else:
            b = self.lru.pop(0)
            self.evict(b)
        self.ref[b] = 1
        return b

    def park(self, b: int) -> None:
        """An unreferenced block that no pending move names goes idle."""
        (self.lru if self.is_cached(b) else self.free).append(b)

    def release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.pending:
                self.held.append(b)
            else:
                self.park(b)

    def revive(self, b: int) -> None:
        """An idle (or held-back) cached block is taken again by a cache hit."""
        (self.held if b in self.held else self.lru).remove(b)
        self.ref[b] = 1

    def settle(self) -> None:
        for b in self.held:
            self.park(b)
        self.held = []
        self.pending = set()
        self.pending_dst = set()


class BlockManager:
    """Reference block manager: free stacks, ref counts, block tables."""

    def __init__(self, num_blocks: int, block_size: int = 16, num_host_blocks: int = 0):
        self.block_size = block_size
        self.num_blocks = num_blocks
        self.num_host_blocks = num_host_blocks
        self.dev = _Pool(num_blocks)
        self.host = _Pool(num_host_blocks)
        self.tables: Dict[int, List[int]] = {}
        self.ntok: Dict[int, int] = {}
        self.on_host: Dict[int, bool] = {}
        self.dirty: set = set()                              # reserved slots this batch (R9)
        self.copies: List[Tuple[int, int]] = []
        self.swapped_out: List[Tuple[int, int]] = []
        self.swapped_in: List[Tuple[int, int]] = []
        # prefix cache (P1-P5)
        self.cache: Dict[int, int] = {}                      # key -> device block
        self.meta: Dict[int, tuple] = {}                     # block -> (key, parent, salt, tokens)
        self.tok: Dict[int, List[int]] = {}                  # seq -> token ids (cache-aware seqs)
        self.salt: Dict[int, int] = {}
        self.keys: Dict[int, List[int]] = {}                 # seq -> keys of its full blocks
        self.serial: Dict[int, int] = {}                     # seq -> creation number
        self.next_serial = 0
        self.to_register: List[tuple] = []                   # blocks filled in this batch (P2)
        self.dev.is_cached = lambda b: b in self.meta
        self.dev.evict = self._evict

    # convenience views of the device pool (tests read them)
    @property
    def free(self) -> List[int]:
        return self.dev.free

    @property
    def ref(self) -> List[int]:
        return self.dev.ref

    def _resident(self, seq: int) -> None:
        if seq not in self.tables:
            raise KeyError(f"no sequence {seq}")
        if self.on_host[seq]:
            raise KeyError(f"sequence {seq} is swapped out")

    def _clean(self, seq: int) -> None:
        if seq in self.dirty:
            raise Busy(f"sequence {seq} reserved slots since the last take_moves()")

    def _new(self, seq: int) -> None:
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        self.serial[seq] = self.next_serial
        self.next_serial += 1

    # ---- sequences ----
    def add_sequence(self, seq: int) -> None:
        self._new(seq)
        self.tables[seq] = []
        self.ntok[seq] = 0
        self.on_host[seq] = False

    def fork(self, parent: int, child: int) -> None:
        """Whole-sequence sharing: child starts with every token of parent, on
        the same physical blocks."""
        self._resident(parent)
        self._clean(parent)
        self._new(child)
        self.tables[child] = list(self.tables[parent])
        self.ntok[child] = self.ntok[parent]
        self.on_host[child] = False
        for b in self.tables[child]:
            self.dev.ref[b] += 1
        if parent in self.tok:
            self.tok[child] = list(self.tok[parent])
            self.salt[child] = self.salt[parent]
            self.keys[child] = list(self.keys[parent])

    def share(self, src: int, dst: int, logical_blocks) -> None:
        """New sequence dst made of the listed full logical blocks of src (R5):
        list(range(n)) shares a prefix of n blocks."""
        self._resident(src)
        self._clean(src)
        self._new(dst)
        full = self.ntok[src] // self.block_size
        idx = [int(i) for i in logical_blocks]
        if any(i < 0 or i >= full for i in idx):
            raise ValueError("only full logical blocks of the source can be shared")
        self.tables[dst] = [self.tables[src][i] for i in idx]
        self.ntok[dst] = len(idx) * self.block_size
        self.on_host[dst] = False
        for b in self.tables[dst]:
            self.dev.ref[b] += 1

    def free_sequence(self, seq: int) -> None:
        if seq not in self.tables:
            raise KeyError(f"no sequence {seq}")
        pool = self.host if self.on_host[seq] else self.dev
        for b in reversed(self.tables.pop(seq)):
            pool.release(b)
        del self.ntok[seq]
        del self.on_host[seq]
        self.dirty.discard(seq)
        for d in (self.tok, self.salt, self.keys, self.serial):
            d.pop(seq, None)

    # ---- allocation ----
    def _cow_needed(self, seq: int, n: int) -> bool:
        have = self.ntok[seq]
        return n > 0 and have % self.block_size != 0 and self.dev.ref[self.tables[seq][-1]] > 1

    def blocks_needed(self, seq: int, n: int) -> int:
        bs = self.block_size
        have = self.ntok[seq]
        new = -(-(have + n) // bs) - (-(-have // bs))
        return new + (1 if self._cow_needed(seq, n) else 0)

    def append_slots(self, seq: int, n: int) -> List[int]:
        """Reserve slots for n new tokens of seq; returns their physical slots
        (block * block_size + row), in token order."""
        self._resident(seq)
        if n < 0:
            raise ValueError("negative token count")
        if self._cow_needed(seq, n) and self.tables[seq][-1] in self.dev.pending_dst:
            raise Busy("the block to copy is the destination of a pending move")
        if self.blocks_needed(seq, n) > self.dev.num_idle():
            raise OutOfBlocks(f"sequence {seq} needs {self.blocks_needed(seq, n)} blocks, "
                              f"{self.dev.num_idle()} free")
        bs = self.block_size
        table = self.tables[seq]
        slots = []
        for _ in range(n):
            pos = self.ntok[seq]
            if pos % bs == 0:
                table.append(self.dev.take())
            elif self.dev.ref[table[-1]] > 1:
                old = table[-1]
                new = self.dev.take()
                self.copies.append((old, new))
                self.dev.pending |= {old, new}
                self.dev.pending_dst.add(new)
                self.dev.release(old)
                table[-1] = new
            slots.append(table[-1] * bs + pos % bs)
            self.ntok[seq] = pos + 1
        if n > 0:
            self.dirty.add(seq)
        return slots

    # ---- swapping ----
    def _swap(self, seqs, to_host: bool) -> None:
        src, dst = (self.dev, self.host) if to_host else (self.host, self.dev)
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise KeyError("a sequence is listed twice")
        for s in seqs:
            if s not in self.tables or self.on_host[s] == to_host:
                raise KeyError(f"sequence {s} cannot be swapped {'out' if to_host else 'in'}")
        for s in seqs:
            self._clean(s)
        distinct = []
        for s in seqs:
            for b in self.tables[s]:
                if b not in distinct:
                    distinct.append(b)
        if any(b in src.pending_dst for b in distinct):
            raise Busy("a block to move is the destination of a pending move")
        if len(distinct) > dst.num_idle():
            raise OutOfBlocks(f"{len(distinct)} blocks needed, {dst.num_idle()} free")
        moved = {}
        record = self.swapped_out if to_host else self.swapped_in
        for s in seqs:
            table = self.tables[s]
            for j, b in enumerate(table):
                if b in moved:
                    dst.ref[moved[b]] += 1
                else:
                    moved[b] = dst.take()
                    record.append((b, moved[b]))
                    src.pending.add(b)
                    dst.pending.add(moved[b])
                    dst.pending_dst.add(moved[b])
                src.release(b)
                table[j] = moved[b]
            self.on_host[s] = to_host

    def swap_out(self, seqs) -> None:
        self._swap(seqs, True)

    def swap_in(self, seqs) -> None:
        self._swap(seqs, False)

    # ---- pending data movement ----
    def take_moves(self):
        """(copies, swap_out, swap_in) recorded since the last call; releases
        the blocks held back for them (R6)."""
        out = (self.copies, self.swapped_out, self.swapped_in)
        self.copies, self.swapped_out, self.swapped_in = [], [], []
        self.dirty = set()
        self._commit_registrations()
        self.dev.settle()
        self.host.settle()
        return out

    def take_copies(self) -> List[Tuple[int, int]]:
        """Device copies only (for callers that never swap)."""
        return self.take_moves()[0]

    # ---- prefix cache ----
    def _evict(self, b: int) -> None:
        key = self.meta.pop(b)[0]
        del self.cache[key]

    def _uncache(self, b: int) -> None:
        """b loses its cache entry; if it is idle it moves to the plain free stack."""
        del self.meta[b]
        if b in self.dev.lru:
            self.dev.lru.remove(b)
            self.dev.free.append(b)

    def _lookup(self, tokens, salt: int, max_blocks: int):
        """Blocks of the longest verified cached prefix (P2, P3) and their keys."""
        bs = self.block_size
        hits, keys = [], []
        key, parent = 0, -1
        for j in range(max_blocks):
            blk = tuple(int(t) for t in tokens[j * bs:(j + 1) * bs])
            key = block_key(key, salt, blk)
            b = self.cache.get(key)
            if b is None or self.meta[b][1:] != (parent, salt, blk):
                break
            hits.append(b)
            keys.append(key)
            parent = b
        return hits, keys

    def add_prompt(self, seq: int, tokens, salt: int = 0) -> int:
        """New sequence for a prompt: it starts on the longest cached prefix of
        whole blocks (P3) and returns how many tokens that covers; the caller
        appends the rest with append_tokens."""
        self._new(seq)
        tokens = [int(t) for t in tokens]
        hits, keys = self._lookup(tokens, salt, max(0, (len(tokens) - 1) // self.block_size))
        for b in hits:
            if self.dev.ref[b] == 0:
                self.dev.revive(b)
            else:
                self.dev.ref[b] += 1
        n = len(hits) * self.block_size
        self.tables[seq] = hits
        self.ntok[seq] = n
        self.on_host[seq] = False
        self.tok[seq] = tokens[:n]
        self.salt[seq] = salt
        self.keys[seq] = keys
        return n

    def append_tokens(self, seq: int, tokens) -> List[int]:
        """append_slots for known tokens; blocks they fill enter the cache (P2)."""
        if seq not in self.tok:
            raise KeyError(f"sequence {seq} does not track its tokens")
        tokens = [int(t) for t in tokens]
        slots = self.append_slots(seq, len(tokens))
        self.tok[seq].extend(tokens)
        bs = self.block_size
        table, keys, salt = self.tables[seq], self.keys[seq], self.salt[seq]
        while (len(keys) + 1) * bs <= self.ntok[seq]:
            j = len(keys)
            blk = tuple(self.tok[seq][j * bs:(j + 1) * bs])
            parent = table[j - 1] if j else -1
            key = block_key(keys[-1] if keys else 0, salt, blk)
            keys.append(key)
            self.to_register.append((self.serial[seq], seq, j, table[j], key, parent, salt, blk))
        return slots

    def _commit_registrations(self) -> None:
        for serial, seq, j, b, key, parent, salt, blk in self.to_register:
            if self.serial.get(seq) != serial or self.on_host[seq] or self.tables[seq][j] != b:
                continue                      # freed (or moved) before its tokens were written
            old = self.cache.get(key)
            if old is not None and self.meta[old][1:] == (parent, salt, blk):
                continue                      # the same prefix is cached in another block
            if old is not None:
                self._uncache(old)            # a stale or colliding entry gives way
            self.cache[key] = b
            self.meta[b] = (key, parent, salt, blk)
        self.to_register = []

    def num_cached_blocks(self) -> int:
        return len(self.cache)

    # ---- queries ----
    def block_table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def num_tokens(self, seq: int) -> int:
        return self.ntok[seq]

    def is_swapped(self, seq: int) -> bool:
        return self.on_host[seq]

    def num_free(self, host: bool = False) -> int:
        """Blocks an allocation can take (idle cached blocks included)."""
        return (self.host if host else self.dev).num_idle()

    def shared_prefix_blocks(self, seq: int) -> int:
        """Leading table entries whose block another sequence also holds."""
        n = 0
        for b in self.tables[seq]:
            if self.dev.ref[b] < 2:
                break
            n += 1
        return n

    def prefix_groups(self, seqs):
        """Sharing groups of a decode batch in batch order: each run of consecutive
        entries whose tables start with the same physical block as the run's first
        entry ("vLLM 基本原理", 内存共享: samples of one prompt name its blocks) is a
        group led by that entry.  Returns (leader index per entry, count per entry,
        largest run): a member's count is its leading table entries equal to the
        leader's, the leader's the largest of its members' counts (0 alone)."""
        for s in seqs:
            self._resident(s)
        n = len(seqs)
        group, count = [0] * n, [0] * n
        largest = 1 if n else 0
        i = 0
        while i < n:
            lead = self.tables[seqs[i]]
            end = i + 1
            while end < n and lead and self.tables[seqs[end]] and \
                    self.tables[seqs[end]][0] == lead[0]:
                end += 1
            group[i] = i
            for m in range(i + 1, end):
                t = self.tables[seqs[m]]
                k = 0
                while k < len(t) and k < len(lead) and t[k] == lead[k]:
                    k += 1
                group[m], count[m] = i, k
            count[i] = max(count[i + 1:end], default=0)
            largest = max(largest, end - i)
            i = end
        return group, count, largest

    def check_invariants(self) -> None:
        """Reference counts equal table occurrences; free plus held-back blocks
        are exactly the unreferenced ones; only last blocks may be partly
        filled."""
        for host, pool, n in ((False, self.dev, self.num_blocks),
                              (True, self.host, self.num_host_blocks)):
            count = [0] * n
            for seq, t in self.tables.items():
                if self.on_host[seq] == host:
                    for b in t:
                        count[b] += 1
            assert count == pool.ref
            idle = pool.free + pool.lru + pool.held
            assert sorted(idle) == [b for b in range(n) if count[b] == 0]
            assert len(set(idle)) == len(idle)
        for key, b in self.cache.items():
            assert self.meta[b][0] == key
        assert len(self.meta) == len(self.cache)
        assert all(b in self.meta for b in self.dev.lru)
        assert not any(b in self.meta for b in self.dev.free)
        for seq, t in self.tables.items():
            assert len(t) == -(-self.ntok[seq] // self.block_size), seq


# --------------------------------------------------------------------------
# data movement on storage arrays (copies, bit for bit)
# --------------------------------------------------------------------------
def copy_blocks(pool: np.ndarray, pairs) -> np.ndarray:
    """Pool after copying whole physical block src onto dst for each (src, dst),
    in order."""
    out = np.array(pool, copy=True)
    for src, dst in pairs:
        out[int(dst)] = out[int(src)]
    return out


def swap_blocks(src_pool: np.ndarray, dst_pool: np.ndarray, pairs) -> np.ndarray:
    """dst_pool after copying block src of src_pool onto block dst of dst_pool."""
    out = np.array(dst_pool, copy=True)
    for src, dst in pairs:
        out[int(dst)] = src_pool[int(src)]
    return out
