"""Reference model of the KV block manager (pure Python, integer only).

TEST INFRASTRUCTURE ONLY (see the package docstring).  It restates the
allocation rules of the pages so the product's C++ allocator can be compared
with it table for table, slot for slot:

* Free block queue: a new block is taken from the head of the queue, freed
  blocks go back immediately ("Life of a prompt", "Back to the queue, and into
  vLLM proper").  Freed blocks join the tail, in the sequence's logical order.
* A block is allocated only when the sequence's current block is full, so a
  sequence of L tokens owns ceil(L / 16) blocks ("PagedAttention in depth",
  vLLM Serving deep dive).
* Sharing and copy-on-write: several block tables may point at one physical
  block, with a reference count per block; appending into a shared block
  copies just that block and repoints only the appending sequence's table
  ("Sharing and copy-on-write", vLLM Serving deep dive).  A shared block that
  is full is never written, so appending after it takes a fresh block and no
  copy.
* Out of blocks: the pages' scheduler preempts instead of crashing ("The
  skeleton of a scheduler", LLM Serving from Scratch); here an append that
  cannot get all the blocks it needs changes nothing and reports the shortage,
  so the caller can preempt.
"""
from __future__ import annotations

from collections import deque


class OutOfBlocks(Exception):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int = 16, initial_order=None):
        self.num_blocks = int(num_blocks)
        self.bs = int(block_size)
        order = list(range(num_blocks)) if initial_order is None else [int(b) for b in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial order must be a permutation of the pool")
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self._next = 0

    # -- sequences -------------------------------------------------------
    def create(self) -> int:
        sid = self._next
        self._next += 1
        self.tables[sid] = []
        self.lens[sid] = 0
        return sid

    def fork(self, parent: int, n_prefix: int) -> int:
        """New sequence sharing the blocks of the parent's first n_prefix tokens."""
        if parent not in self.tables or not 0 <= n_prefix <= self.lens[parent]:
            raise ValueError("bad fork")
        nb = -(-n_prefix // self.bs)
        child = self.create()
        self.tables[child] = list(self.tables[parent][:nb])
        for b in self.tables[child]:
            self.ref[b] += 1
        self.lens[child] = n_prefix
        return child

    def _pop(self) -> int:
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def blocks_needed(self, sid: int, n: int) -> int:
        L = self.lens[sid]
        need = -(-(L + n) // self.bs) - (-(-L // self.bs))
        if n > 0 and L % self.bs != 0 and self.ref[self.tables[sid][L // self.bs]] > 1:
            need += 1
        return need

    def append(self, sid: int, n: int):
        """Make room for n new tokens; returns (slots, cow_pairs)."""
        if sid not in self.tables or n < 0:
            raise ValueError("bad append")
        if self.blocks_needed(sid, n) > len(self.free):
            raise OutOfBlocks()
        table = self.tables[sid]
        L = self.lens[sid]
        cow = []
        if n > 0 and L % self.bs != 0:
            last = table[L // self.bs]
            if self.ref[last] > 1:
                nb = self._pop()
                self.ref[last] -= 1
                table[L // self.bs] = nb
                cow.append((last, nb))
        slots = []
        for t in range(L, L + n):
            if t % self.bs == 0:
                table.append(self._pop())
            slots.append(table[t // self.bs] * self.bs + t % self.bs)
        self.lens[sid] = L + n
        return slots, cow

    def release(self, sid: int):
        """Finish a sequence: drop its references; blocks at zero rejoin the
        free queue's tail at once."""
        for b in self.tables.pop(sid):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[sid]

    # -- views -----------------------------------------------------------
    def table(self, sid: int) -> list[int]:
        return list(self.tables[sid])

    def num_free(self) -> int:
        return len(self.free)

    def free_queue(self) -> list[int]:
        return list(self.free)

    def padded_tables(self, sids, max_blocks: int, pad: int = -1):
        import numpy as np
        out = np.full((len(sids), max_blocks), pad, dtype=np.int32)
        lens = np.zeros(len(sids), dtype=np.int32)
        for i, s in enumerate(sids):
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("table wider than max_blocks")
            out[i, :len(t)] = t
            lens[i] = self.lens[s]
        return out, lens
