"""Preemption by swapping, on the block allocator, plain Python.  TEST INFRASTRUCTURE ONLY.

What it does ("How LLM Inference Serving Works", section "When memory runs out anyway": when
the KV cache fills up, some requests are preempted to free their blocks; the preempted KV is
either dropped and recomputed later or swapped out to CPU memory and brought back).  Swapping:
  * a host swap pool of fixed size holds blocks in the device pool's layout;
  * swap-out gives each block of the sequence's table a swap block and releases the device
    blocks exactly as a finished request would (the copy device -> host is the caller's, one
    batched launch, enqueued before anything can write the released blocks);
  * swap-in takes fresh device blocks (as any allocation would, evicting cached blocks if it
    must) and returns the swap blocks; the copy host -> device is the caller's;
  * while swapped out the sequence keeps its length and token ids but owns no device blocks.
Readings where the pages leave a step open (the library follows the same ones): the swap pool
is a FIFO free list like the device one, swap blocks return to its tail in table order; every
block is swapped, shared or not (sharing with other sequences is lost: the swapped-in copy is
private); a swapped-in prompt sequence republishes its full blocks whose content is not cached.
"""
from __future__ import annotations

import collections
from typing import Dict, List, Optional, Sequence, Tuple

from oracle.allocator import BadSequence, OutOfBlocks
from oracle.prefix_cache import PrefixCachingAllocator


class SwapSpaceFull(Exception):
    pass


class SwappingAllocator(PrefixCachingAllocator):
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence] = None,
                 num_cpu_blocks: int = 0):
        super().__init__(num_blocks, block_size, free_order)
        self.cpu_free = collections.deque(range(num_cpu_blocks))
        self.swapped: Dict[int, Tuple[List[int], int]] = {}   # seq -> (swap blocks, length)

    def swap_out(self, seq: int) -> List[Tuple[int, int]]:
        """(device block, swap block) pairs in table order."""
        self._check(seq)
        table = self.tables[seq]
        if len(self.cpu_free) < len(table):
            raise SwapSpaceFull()
        cpu = [self.cpu_free.popleft() for _ in table]
        pairs = list(zip(table, cpu))
        length = self.lengths[seq]
        ids = self.ids.get(seq)
        salt = self.salt.get(seq)
        self.release(seq)            # device blocks go exactly as for a finished request
        if ids is not None:          # the sequence keeps its token ids, not its chain
            self.ids[seq], self.salt[seq], self.chain[seq] = ids, salt, []
        self.swapped[seq] = (cpu, length)
        return pairs

    def swap_in(self, seq: int) -> List[Tuple[int, int]]:
        """(swap block, device block) pairs in table order."""
        if seq not in self.swapped:
            raise BadSequence(seq)
        cpu, length = self.swapped[seq]

        def run():
            return [self._take() for _ in cpu]
        fresh = self._transaction(run)     # OutOfBlocks leaves everything as it was
        del self.swapped[seq]
        self.tables[seq] = fresh
        self.lengths[seq] = length
        self.cpu_free.extend(cpu)
        self._publish(seq)
        return list(zip(cpu, fresh))

    def release(self, seq: int) -> None:
        if seq in self.swapped:
            cpu, _ = self.swapped.pop(seq)
            self.cpu_free.extend(cpu)
            for d in (self.ids, self.salt, self.chain):
                d.pop(seq, None)
            return
        super().release(seq)

    def length(self, seq: int) -> int:
        if seq in self.swapped:
            return self.swapped[seq][1]
        return super().length(seq)

    def num_free_swap(self) -> int:
        return len(self.cpu_free)
