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
* A finished sequence returns its blocks at once (xdnf.cn article, section
  六.1).

Readings where the pages leave the policy open (the same in the native
manager, so tables can be compared exactly; the invariants below hold for any
policy):
* Free blocks form a stack: allocation takes the most recently freed block;
  initially blocks come out in increasing id order.
* Freeing a sequence releases its table from the last entry to the first, so
  its first block is the next to be reused.
* Appending n tokens is all-or-nothing: if the pool cannot supply every block
  needed (copy-on-write included), nothing changes and OutOfBlocks is raised.
* Only a partly filled shared last block is copied on write; full shared
  blocks stay shared (nothing is ever written into them again).

Data movement: copy_blocks copies whole physical blocks within a pool (the
copy-on-write step); swap_blocks copies whole blocks between two pools (a
device pool and a host pool).  A physical block of a [num_blocks, num_heads,
block_size, head_dim] pool is one contiguous run of
num_heads * block_size * head_dim elements.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    """Reference block manager: free stack, ref counts, block tables."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        self.block_size = block_size
        self.num_blocks = num_blocks
        self.free: List[int] = list(range(num_blocks - 1, -1, -1))   # top = end of list
        self.ref = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.ntok: Dict[int, int] = {}
        self.copies: List[Tuple[int, int]] = []

    # ---- sequences ----
    def add_sequence(self, seq: int) -> None:
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.ntok[seq] = 0

    def fork(self, parent: int, child: int) -> None:
        """child starts with every token of parent, on the same physical blocks."""
        if child in self.tables:
            raise KeyError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.ntok[child] = self.ntok[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def free_sequence(self, seq: int) -> None:
        for b in reversed(self.tables.pop(seq)):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.ntok[seq]

    # ---- allocation ----
    def _take(self) -> int:
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def blocks_needed(self, seq: int, n: int) -> int:
        bs = self.block_size
        have = self.ntok[seq]
        new = -(-(have + n) // bs) - (-(-have // bs))
        cow = n > 0 and have % bs != 0 and self.ref[self.tables[seq][-1]] > 1
        return new + (1 if cow else 0)

    def append_slots(self, seq: int, n: int) -> List[int]:
        """Reserve slots for n new tokens of seq; returns their physical slots
        (block * block_size + row), in token order."""
        if self.blocks_needed(seq, n) > len(self.free):
            raise OutOfBlocks(f"sequence {seq} needs {self.blocks_needed(seq, n)} blocks, "
                              f"{len(self.free)} free")
        bs = self.block_size
        table = self.tables[seq]
        slots = []
        for _ in range(n):
            pos = self.ntok[seq]
            if pos % bs == 0:
                table.append(self._take())
            elif self.ref[table[-1]] > 1:
                old = table[-1]
                new = self._take()
                self.ref[old] -= 1
                self.copies.append((old, new))
                table[-1] = new
            slots.append(table[-1] * bs + pos % bs)
            self.ntok[seq] = pos + 1
        return slots

    def take_copies(self) -> List[Tuple[int, int]]:
        out, self.copies = self.copies, []
        return out

    # ---- queries ----
    def block_table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def num_tokens(self, seq: int) -> int:
        return self.ntok[seq]

    def num_free(self) -> int:
        return len(self.free)

    def check_invariants(self) -> None:
        """Reference counts equal table occurrences; free blocks are exactly the
        unreferenced ones; only last blocks may be partly filled."""
        count = [0] * self.num_blocks
        for seq, t in self.tables.items():
            for b in t:
                count[b] += 1
            assert len(t) == -(-self.ntok[seq] // self.block_size), seq
        assert count == self.ref
        assert sorted(self.free) == [b for b in range(self.num_blocks) if count[b] == 0]
        assert len(set(self.free)) == len(self.free)


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
