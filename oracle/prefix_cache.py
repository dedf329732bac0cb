"""Automatic prefix caching on the block allocator, plain Python.  TEST INFRASTRUCTURE ONLY.

What it does ("How LLM Inference Serving Works", section "Prefix Caching and Chunked Prefill",
"Automatic prefix caching"; section "Putting It Together: The Life of a Request"):
  * every KV block is identified by a hash of the tokens in the block and of all the tokens
    before it, so a block matches only if the whole prefix up to it is identical;
  * a table maps those hashes to cached physical blocks; a new request reuses its matching
    leading blocks and only the rest of its prompt needs prefill;
  * a block that no request uses any more is not freed at once: it stays matchable, and cached
    blocks are evicted in least-recently-used order when memory is needed;
  * an optional per-request salt enters the hash of a request's first block, which keeps
    requests with different salts from matching each other's cached blocks;
  * a finished request releases its blocks: their reference counts fall, and blocks left
    unreferenced stay cached until evicted.

Readings where the pages leave a step open (the library follows the same ones):
  * hash: 64-bit FNV-1a (offset basis 0xcbf29ce484222325, prime 0x100000001b3) over
    little-endian bytes; the chain starts at FNV-1a of the 8 salt bytes; a block's hash is
    FNV-1a of its parent hash's 8 bytes followed by its block_size int32 token ids.  A match
    also compares the stored ids and parent hash;
  * only full blocks whose ids are all known are published; when two blocks hold the same
    content the first one published keeps the hash;
  * a new request matches full blocks among its first n - 1 tokens only, so at least one prompt
    token is left to compute (generation needs its query);
  * "evicted when memory is needed": an allocation takes the free list's head first and evicts
    the least recently used cached block only when the free list is empty;
  * blocks released together join the LRU list last block first, so a prefix (which its
    extensions need in order to match at all) is evicted after them;
  * a hit on an evictable block takes it off the LRU list; a later release puts it at the end.
"""
from __future__ import annotations

import collections
import copy
from typing import Dict, List, Optional, Sequence, Tuple

from oracle.allocator import BadSequence, OutOfBlocks, PyAllocator

FNV_OFFSET = 0xcbf29ce484222325
FNV_PRIME = 0x100000001b3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """64-bit FNV-1a: for each byte, xor it in, then multiply by the prime (mod 2**64)."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def chain_root(salt: int) -> int:
    return fnv1a64((salt & MASK64).to_bytes(8, "little"))


def block_hash(parent: int, tokens: Sequence[int]) -> int:
    data = parent.to_bytes(8, "little") + b"".join(
        int(t).to_bytes(4, "little", signed=True) for t in tokens)
    return fnv1a64(data)


class PrefixCachingAllocator(PyAllocator):
    """PyAllocator plus the prefix cache.  Sequences made by create() behave exactly as in
    PyAllocator; sequences made by create_prefix() also publish their full blocks."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence] = None):
        super().__init__(num_blocks, block_size, free_order)
        self.cache: Dict[int, int] = {}                      # hash -> block
        self.info: Dict[int, Tuple[int, int, tuple]] = {}    # block -> (hash, parent, ids)
        self.evictable: "collections.OrderedDict[int, None]" = collections.OrderedDict()
        self.ids: Dict[int, List[int]] = {}                  # sequence -> known token ids
        self.salt: Dict[int, int] = {}
        self.chain: Dict[int, List[int]] = {}                # sequence -> hash of each block

    # -- allocation with eviction -----------------------------------------------------------
    def _take(self) -> int:
        if self.free:
            return super()._take()
        if not self.evictable:
            raise OutOfBlocks()
        blk, _ = self.evictable.popitem(last=False)          # least recently used
        del self.cache[self.info.pop(blk)[0]]
        self.refcount[blk] = 1
        return blk

    def _transaction(self, fn):
        saved = (dict(self.cache), dict(self.info), copy.copy(self.evictable))
        try:
            return super()._transaction(fn)
        except OutOfBlocks:
            self.cache, self.info, self.evictable = saved
            raise

    # -- publishing ---------------------------------------------------------------------------
    def _publish(self, seq: int) -> None:
        if seq not in self.ids:
            return
        bs = self.block_size
        ids, chain = self.ids[seq], self.chain[seq]
        full = min(self.lengths[seq], len(ids)) // bs
        while len(chain) < full:
            j = len(chain)
            parent = chain[-1] if chain else chain_root(self.salt[seq])
            toks = tuple(ids[j * bs:(j + 1) * bs])
            h = block_hash(parent, toks)
            chain.append(h)
            blk = self.tables[seq][j]
            if blk in self.info or h in self.cache:
                continue
            self.info[blk] = (h, parent, toks)
            self.cache[h] = blk

    # -- sequences ----------------------------------------------------------------------------
    def create_prefix(self, tokens: Sequence[int], salt: int = 0) -> Tuple[int, int]:
        """A sequence for this prompt: (id, number of leading tokens already cached)."""
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        sid = self.create()
        self.ids[sid] = list(tokens)
        self.salt[sid] = salt & MASK64
        chain, table = [], []
        parent = chain_root(salt)
        n_match = (len(tokens) - 1) // bs if tokens else 0
        for j in range(n_match):
            toks = tuple(tokens[j * bs:(j + 1) * bs])
            h = block_hash(parent, toks)
            blk = self.cache.get(h)
            if blk is None or self.info[blk][1:] != (parent, toks):
                break
            if self.refcount[blk] == 0:
                del self.evictable[blk]
            self.refcount[blk] += 1
            table.append(blk)
            chain.append(h)
            parent = h
        self.tables[sid] = table
        self.lengths[sid] = len(table) * bs
        self.chain[sid] = chain
        return sid, len(table) * bs

    def add_tokens(self, seq: int, tokens: Sequence[int]) -> None:
        self._check(seq)
        if seq not in self.ids:
            raise ValueError("sequence was not created with its token ids")
        self.ids[seq].extend(int(t) for t in tokens)
        self._publish(seq)

    def fork(self, parent: int, n_tokens: int) -> int:
        child = super().fork(parent, n_tokens)
        if parent in self.ids:
            self.ids[child] = self.ids[parent][:n_tokens]
            self.salt[child] = self.salt[parent]
            self.chain[child] = self.chain[parent][:n_tokens // self.block_size]
        return child

    def append_slot(self, seq: int):
        out = super().append_slot(seq)
        self._publish(seq)
        return out

    def reserve(self, seq: int, n: int):
        out = super().reserve(seq, n)
        self._publish(seq)
        return out

    def step(self, seqs: Sequence[int]):
        out = super().step(seqs)
        for s in seqs:
            self._publish(s)
        return out

    def release(self, seq: int) -> None:
        """Blocks left without references: private ones to the free list in table order, cached
        ones to the end of the LRU list, last block first."""
        self._check(seq)
        table = self.tables.pop(seq)
        del self.lengths[seq]
        for d in (self.ids, self.salt, self.chain):
            d.pop(seq, None)
        cached_zero = []
        for blk in table:
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                if blk in self.info:
                    cached_zero.append(blk)
                else:
                    self.free.append(blk)
        for blk in reversed(cached_zero):
            self.evictable[blk] = None

    # -- views --------------------------------------------------------------------------------
    def num_evictable(self) -> int:
        return len(self.evictable)

    def evictable_list(self) -> List[int]:
        return list(self.evictable)

    def block_hash(self, blk: int) -> Optional[int]:
        return self.info[blk][0] if blk in self.info else None


__all__ = ["PrefixCachingAllocator", "fnv1a64", "chain_root", "block_hash", "OutOfBlocks",
           "BadSequence"]
