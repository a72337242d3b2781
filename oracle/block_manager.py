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
* Prefix caching ("Trick 3, Prefix caching", How AI actually answers you;
  "Prefix caching (automatic KV reuse)", vLLM Serving deep dive): a full
  block is labelled by its own tokens together with the label of the block
  before it, so equal labels mean equal text up to and including the block.
  Here a label is that exact pair (an interned tuple), not a hash.  Only full
  blocks are labelled; a new prompt reuses its leading labelled blocks (the
  prompt's last token always computed); unused labelled blocks are evicted
  least recently released first — a released block keeps its label in the
  free queue until the queue hands it out again.
* Swapping ("The scheduler: waiting, running, swapped", vLLM Serving deep
  dive; the CPU blocks of "Back to the queue, and into vLLM proper", Life of
  a prompt): a preempted sequence's blocks are parked in a pool of host
  ("CPU") blocks and restored later.  Here the CPU blocks have their own FIFO
  queue; swapping out gives each of the sequence's blocks, in logical order, a
  CPU block from the head of that queue (a private copy, also of blocks the
  sequence shares) and then releases the GPU blocks as a finished sequence
  would; swapping in gives each CPU block a GPU block from the head of the
  free queue and returns the CPU blocks to their queue's tail.  Both are all or
  nothing.  A swapped-out sequence can only be swapped in, freed or read
  back; anything else on it is a state error.
"""
from __future__ import annotations

from collections import deque


class OutOfBlocks(Exception):
    pass


class StateError(Exception):
    """An operation the sequence's state does not allow (swapped out)."""


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
        # prefix cache
        self.caching = False
        self.labels: dict[int, int] = {}        # label id -> block
        self.block_label = [None] * num_blocks  # block -> label id
        self._label_ids: dict[tuple, int] = {}  # (previous label id, tokens) -> label id
        self.tokens: dict[int, list[int] | None] = {}  # None: not known
        self.queried = 0
        self.hits = 0
        # swap space: host blocks with their own FIFO queue
        self.num_cpu_blocks = 0
        self.cpu_free: deque = deque()
        self.swapped: set[int] = set()

    def _label_id(self, prev: int, toks) -> int:
        key = (prev, tuple(int(t) for t in toks))
        if key not in self._label_ids:
            self._label_ids[key] = len(self._label_ids)
        return self._label_ids[key]

    def _seq_labels(self, sid: int) -> list[int]:
        toks = self.tokens[sid]
        out, prev = [], -1
        for i in range(self.lens[sid] // self.bs):
            prev = self._label_id(prev, toks[i * self.bs:(i + 1) * self.bs])
            out.append(prev)
        return out

    # -- sequences -------------------------------------------------------
    def create(self) -> int:
        sid = self._next
        self._next += 1
        self.tables[sid] = []
        self.lens[sid] = 0
        self.tokens[sid] = []
        return sid

    def enable_caching(self, on: bool = True):
        if not on:
            self.labels.clear()
            self.block_label = [None] * self.num_blocks
        self.caching = bool(on)

    def create_cached(self, tokens) -> tuple[int, int]:
        """New sequence for a prompt; reuses its leading labelled full blocks.
        Returns (sequence, reused tokens)."""
        tokens = [int(t) for t in tokens]
        sid = self.create()
        if self.caching and tokens:
            prev = -1
            for i in range((len(tokens) - 1) // self.bs):
                lab = self._label_id(prev, tokens[i * self.bs:(i + 1) * self.bs])
                self.queried += 1
                if lab not in self.labels:
                    break
                b = self.labels[lab]
                self.hits += 1
                if self.ref[b] == 0:
                    self.free.remove(b)
                self.ref[b] += 1
                self.tables[sid].append(b)
                prev = lab
        self.lens[sid] = len(self.tables[sid]) * self.bs
        self.tokens[sid] = tokens[:self.lens[sid]]
        return sid, self.lens[sid]

    def _label_new_full_blocks(self, sid: int, first: int):
        if not self.caching or self.tokens[sid] is None:
            return
        labs = self._seq_labels(sid)
        for i in range(first, len(labs)):
            b = self.tables[sid][i]
            if self.block_label[b] is not None or labs[i] in self.labels:
                continue
            self.labels[labs[i]] = b
            self.block_label[b] = labs[i]

    def cache_stats(self) -> dict:
        return {"cached_blocks": len(self.labels), "queried_blocks": self.queried, "hit_blocks": self.hits}

    def fork(self, parent: int, n_prefix: int) -> int:
        """New sequence sharing the blocks of the parent's first n_prefix tokens."""
        if parent in self.swapped:
            raise StateError("fork of a swapped-out sequence")
        if parent not in self.tables or not 0 <= n_prefix <= self.lens[parent]:
            raise ValueError("bad fork")
        nb = -(-n_prefix // self.bs)
        child = self.create()
        self.tables[child] = list(self.tables[parent][:nb])
        for b in self.tables[child]:
            self.ref[b] += 1
        self.lens[child] = n_prefix
        pt = self.tokens[parent]
        self.tokens[child] = None if pt is None else list(pt[:n_prefix])
        return child

    def _pop(self) -> int:
        b = self.free.popleft()
        lab = self.block_label[b]
        if lab is not None:  # evicted: it is about to hold new data
            if self.labels.get(lab) == b:
                del self.labels[lab]
            self.block_label[b] = None
        self.ref[b] = 1
        return b

    def blocks_needed(self, sid: int, n: int) -> int:
        if sid in self.swapped:
            raise StateError("swapped out")
        L = self.lens[sid]
        need = -(-(L + n) // self.bs) - (-(-L // self.bs))
        if n > 0 and L % self.bs != 0 and self.ref[self.tables[sid][L // self.bs]] > 1:
            need += 1
        return need

    def append_tokens(self, sid: int, tokens):
        """append() with the new tokens' ids, labelling the blocks they fill."""
        tokens = [int(t) for t in tokens]
        L = self.lens[sid] if sid in self.lens else 0
        slots, cow = self._append(sid, len(tokens))
        if self.tokens[sid] is not None:
            self.tokens[sid].extend(tokens)
            self._label_new_full_blocks(sid, L // self.bs)
        return slots, cow

    def append(self, sid: int, n: int):
        """Make room for n new tokens; returns (slots, cow_pairs).  The tokens
        are not known, so nothing of the sequence from here on is labelled."""
        slots, cow = self._append(sid, n)
        if n > 0:
            self.tokens[sid] = None
        return slots, cow

    def _append(self, sid: int, n: int):
        if sid in self.swapped:
            raise StateError("append to a swapped-out sequence")
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
        free queue's tail at once (a swapped-out sequence's CPU blocks rejoin
        theirs)."""
        if sid in self.swapped:
            self.cpu_free.extend(self.tables.pop(sid))
            self.swapped.discard(sid)
        else:
            for b in self.tables.pop(sid):
                self.ref[b] -= 1
                if self.ref[b] == 0:
                    self.free.append(b)
        del self.lens[sid]
        del self.tokens[sid]

    # -- swapping ----------------------------------------------------------
    def set_swap_space(self, n: int):
        """n host blocks, queued 0, 1, ..., n-1; only while nothing is swapped out."""
        if self.swapped:
            raise StateError("sequences are swapped out")
        if n < 0:
            raise ValueError("negative swap space")
        self.num_cpu_blocks = int(n)
        self.cpu_free = deque(range(self.num_cpu_blocks))

    def swap_out(self, sid: int) -> list[tuple[int, int]]:
        """Park sid's blocks in CPU blocks; returns (GPU block, CPU block)
        copies in logical order."""
        if sid in self.swapped:
            raise StateError("already swapped out")
        if sid not in self.tables:
            raise ValueError("unknown sequence")
        table = self.tables[sid]
        if len(table) > len(self.cpu_free):
            raise OutOfBlocks()
        pairs = [(b, self.cpu_free.popleft()) for b in table]
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        self.tables[sid] = [c for _, c in pairs]
        self.swapped.add(sid)
        return pairs

    def swap_in(self, sid: int) -> list[tuple[int, int]]:
        """Restore sid into fresh GPU blocks; returns (CPU block, GPU block)
        copies in logical order.  Its full blocks are labelled again when
        their text is known and not cached elsewhere."""
        if sid not in self.swapped:
            raise StateError("not swapped out")
        table = self.tables[sid]
        if len(table) > len(self.free):
            raise OutOfBlocks()
        pairs = [(c, self._pop()) for c in table]
        self.cpu_free.extend(table)
        self.tables[sid] = [g for _, g in pairs]
        self.swapped.discard(sid)
        self._label_new_full_blocks(sid, 0)
        return pairs

    def cpu_free_queue(self) -> list[int]:
        return list(self.cpu_free)

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
            if s in self.swapped:
                raise StateError("swapped out")
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("table wider than max_blocks")
            out[i, :len(t)] = t
            lens[i] = self.lens[s]
        return out, lens
