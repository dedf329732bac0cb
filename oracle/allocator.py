"""Host block allocator, plain Python.  TEST INFRASTRUCTURE ONLY.

What it does ([Serving] "PagedAttention: Virtual Memory for the KV Cache"; [Walkthrough]
"Step 7"): the KV cache is split into fixed-size blocks; each sequence sees contiguous logical
blocks; its block table maps them to physical blocks anywhere in the pool; a physical block is
taken only when the sequence's current block fills up.  Sharing ([Serving] "Sharing comes for
free"; [Walkthrough] "Step 8"): two sequences may point at the same physical block, which keeps a
reference count; a shared block is copied only when one of them writes into it.  Release
([Serving] "The Life of a Request"): a finished request's blocks drop their counts.

The pages fix no order in which free blocks are handed out; this policy (the one the library
follows too) makes every table unique:
  * the free list is FIFO, initialised from a given order of the block ids;
  * an allocation takes the head; a block whose count reaches zero goes to the tail, in the
    logical order of the table it is released from;
  * a batch step serves its sequences in the order given; the copy of a copy-on-write takes its
    block from the head like any other allocation;
  * sequence ids count up from 0 in creation order and are never reused;
  * a call that runs out of free blocks changes nothing and reports OOM.
"""
from __future__ import annotations

import collections
import copy
from typing import Dict, List, Optional, Sequence, Tuple


class OutOfBlocks(Exception):
    pass


class BadSequence(Exception):
    pass


class PyAllocator:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence] = None):
        if free_order is None:
            free_order = range(num_blocks)
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.free = collections.deque(int(b) for b in free_order)
        self.refcount = [0] * self.num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}
        self.next_id = 0

    # -- sequences ---------------------------------------------------------------------------
    def _check(self, seq: int) -> None:
        if seq not in self.tables:
            raise BadSequence(seq)

    def create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.lengths[sid] = 0
        return sid

    def fork(self, parent: int, n_tokens: int) -> int:
        """A new sequence whose first n_tokens are the parent's: it shares the parent's first
        ceil(n / bs) blocks, each gaining one reference."""
        self._check(parent)
        if n_tokens < 0 or n_tokens > self.lengths[parent]:
            raise ValueError("fork length out of range")
        nblk = -(-n_tokens // self.block_size)
        shared = self.tables[parent][:nblk]
        for blk in shared:
            self.refcount[blk] += 1
        sid = self.create()
        self.tables[sid] = list(shared)
        self.lengths[sid] = n_tokens
        return sid

    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks()
        blk = self.free.popleft()
        self.refcount[blk] = 1
        return blk

    def _append_one(self, seq: int) -> Tuple[int, int, int]:
        table = self.tables[seq]
        n = self.lengths[seq]
        j, off = divmod(n, self.block_size)
        src = dst = -1
        if off == 0:
            # the current block is full (or there is none): a new block is needed now
            table.append(self._take())
        elif self.refcount[table[j]] > 1:
            # writing into a block another sequence also uses: copy it first
            src = table[j]
            dst = self._take()
            self.refcount[src] -= 1
            table[j] = dst
        self.lengths[seq] = n + 1
        return table[j] * self.block_size + off, src, dst

    def _transaction(self, fn):
        saved = (copy.copy(self.free), list(self.refcount),
                 {k: list(v) for k, v in self.tables.items()}, dict(self.lengths))
        try:
            return fn()
        except OutOfBlocks:
            self.free, self.refcount, self.tables, self.lengths = saved
            raise

    def append_slot(self, seq: int) -> Tuple[int, int, int]:
        """Slot for the sequence's next token, and the (src, dst) block copy that must happen
        before the write (-1, -1 when none)."""
        self._check(seq)
        return self._transaction(lambda: self._append_one(seq))

    def reserve(self, seq: int, n: int):
        """n successive appends: (slots, list of (src, dst) copies)."""
        self._check(seq)

        def run():
            slots, cows = [], []
            for _ in range(n):
                s, a, b = self._append_one(seq)
                slots.append(s)
                if a >= 0:
                    cows.append((a, b))
            return slots, cows
        return self._transaction(run)

    def step(self, seqs: Sequence[int]):
        """One append per listed sequence, in list order: (slots, list of (src, dst) copies)."""
        for s in seqs:
            self._check(s)

        def run():
            slots, cows = [], []
            for s in seqs:
                slot, a, b = self._append_one(s)
                slots.append(slot)
                if a >= 0:
                    cows.append((a, b))
            return slots, cows
        return self._transaction(run)

    def release(self, seq: int) -> None:
        """Drop the sequence; each of its blocks loses a reference, and blocks left with none go
        to the tail of the free list in table order."""
        self._check(seq)
        for blk in self.tables.pop(seq):
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self.free.append(blk)
        del self.lengths[seq]

    # -- views -------------------------------------------------------------------------------
    def length(self, seq: int) -> int:
        self._check(seq)
        return self.lengths[seq]

    def table(self, seq: int) -> List[int]:
        self._check(seq)
        return list(self.tables[seq])

    def export(self, seqs: Sequence[int], max_blocks: int):
        """Block tables [B][max_blocks] padded with -1, and lengths [B]."""
        rows, lens = [], []
        for s in seqs:
            t = self.table(s)
            if len(t) > max_blocks:
                raise ValueError("table longer than max_blocks")
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lengths[s])
        return rows, lens

    def num_free(self) -> int:
        return len(self.free)

    def free_list(self) -> List[int]:
        return list(self.free)


def run_script(alloc: PyAllocator, ops) -> Dict[int, int]:
    """Apply a set-up script of ("create"|"reserve"|"fork"|"free", ...) ops; returns the map from
    script names to sequence ids."""
    ids: Dict[int, int] = {}
    for op in ops:
        if op[0] == "create":
            ids[op[1]] = alloc.create()
        elif op[0] == "reserve":
            alloc.reserve(ids[op[1]], op[2])
        elif op[0] == "fork":
            ids[op[3]] = alloc.fork(ids[op[1]], op[2])
        elif op[0] == "free":
            alloc.release(ids.pop(op[1]))
        else:
            raise ValueError(op)
    return ids
