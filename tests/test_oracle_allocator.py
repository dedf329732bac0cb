"""Pins for oracle.allocator: the pages' waste figures, hand-worked tables for the FIFO policy,
copy-on-write on a shared partial block, the strong guarantee on running out of blocks, and the
invariants that hold under any policy (checked after every op of random scripts)."""
import collections

import pytest
from hypothesis import given, settings, strategies as st

import inputs
from oracle import kvsize
from oracle.allocator import BadSequence, OutOfBlocks, PyAllocator, run_script
from tests.golden.load import load

WASTE = load("waste.txt")


def check_invariants(a: PyAllocator):
    held = collections.Counter(b for t in a.tables.values() for b in t)
    for blk in range(a.num_blocks):
        assert a.refcount[blk] == held.get(blk, 0)
    free = a.free_list()
    assert len(set(free)) == len(free)
    assert all(a.refcount[b] == 0 for b in free)
    assert len(free) + sum(1 for rc in a.refcount if rc > 0) == a.num_blocks
    for sid, t in a.tables.items():
        assert len(t) == kvsize.blocks_for(a.lengths[sid], a.block_size)


@pytest.mark.parametrize("S,key", [(100, "paged_bs16_S100"), (32, "paged_bs16_S32"),
                                   (1, "paged_bs16_S1")])
def test_waste_of_reserved_sequence(S, key):
    a = PyAllocator(64, 16)
    s = a.create()
    a.reserve(s, S)
    assert len(a.table(s)) * 16 - S == WASTE[key]


def test_fifo_policy_hand_worked():
    a = PyAllocator(6, 4, free_order=[5, 3, 1, 0, 2, 4])
    s0, s1 = a.create(), a.create()
    slots, cows = a.reserve(s0, 5)            # blocks 5 (4 tokens) then 3
    assert slots == [20, 21, 22, 23, 12] and cows == []
    slots, _ = a.step([s1, s0])               # s1 takes block 1, s0 writes 3 offset 1
    assert slots == [4, 13]
    assert a.table(s0) == [5, 3] and a.table(s1) == [1]
    a.release(s0)                             # 5 then 3 go to the tail
    assert a.free_list() == [0, 2, 4, 5, 3]
    s2 = a.create()
    assert s2 == 2                            # ids are never reused
    a.reserve(s2, 1)
    assert a.table(s2) == [0]


def test_copy_on_write_of_shared_partial_block():
    a = PyAllocator(8, 4, free_order=range(8))
    p = a.create()
    a.reserve(p, 6)                            # blocks 0, 1 (block 1 holds 2 tokens)
    c = a.fork(p, 6)
    assert a.table(c) == [0, 1] and a.refcount[0] == 2 and a.refcount[1] == 2
    slot, src, dst = a.append_slot(c)         # write into shared block 1 -> copy it
    assert (src, dst) == (1, 2) and slot == 2 * 4 + 2
    assert a.table(c) == [0, 2] and a.refcount[1] == 1 and a.refcount[2] == 1
    slot, src, dst = a.append_slot(p)         # the parent is now the only user of block 1
    assert (src, dst) == (-1, -1) and slot == 1 * 4 + 2
    check_invariants(a)


def test_fork_on_block_boundary_needs_no_copy():
    a = PyAllocator(8, 4)
    p = a.create()
    a.reserve(p, 8)
    c = a.fork(p, 8)
    slot, src, dst = a.append_slot(c)
    assert src == -1 and a.table(c) == [0, 1, 2] and slot == 8


def test_fork_shorter_than_parent_shares_partial_block():
    a = PyAllocator(8, 4)
    p = a.create()
    a.reserve(p, 7)
    c = a.fork(p, 5)                           # tokens 0..4: blocks 0 and 1 (partially)
    assert a.table(c) == [0, 1] and a.length(c) == 5
    _, src, dst = a.append_slot(c)
    assert (src, dst) == (1, 2)


def test_shared_prefix_counted_once():
    a = PyAllocator(64, 16)
    p = a.create()
    a.reserve(p, 100)
    kids = [a.fork(p, 100) for _ in range(3)]
    unique = {b for t in a.tables.values() for b in t}
    total = sum(len(t) for t in a.tables.values())
    assert len(unique) == 7 and total == 28
    assert a.num_free() == 64 - 7
    check_invariants(a)
    for k in kids:
        a.release(k)
    a.release(p)
    assert a.num_free() == 64


def test_out_of_blocks_changes_nothing():
    a = PyAllocator(3, 4, free_order=[2, 0, 1])
    s = a.create()
    a.reserve(s, 9)                            # 3 blocks, 9 tokens
    before = (a.free_list(), list(a.refcount), a.table(s), a.length(s))
    with pytest.raises(OutOfBlocks):
        a.reserve(s, 5)                        # 3 fit in place, then a 4th block is needed
    assert (a.free_list(), list(a.refcount), a.table(s), a.length(s)) == before
    t = a.create()
    with pytest.raises(OutOfBlocks):
        a.step([s, t])
    assert a.length(s) == 9 and a.length(t) == 0


def test_unknown_sequence():
    a = PyAllocator(4, 4)
    with pytest.raises(BadSequence):
        a.append_slot(7)
    s = a.create()
    a.release(s)
    with pytest.raises(BadSequence):
        a.release(s)


def test_tiny_workload_step_allocates_two_blocks():
    w = inputs.tiny_fp32()
    a = PyAllocator(w.NB, w.bs, inputs.free_order(w))
    ids = run_script(a, inputs.setup_script(w))
    seqs = [ids[b] for b in range(w.B)]
    assert [a.length(s) for s in seqs] == [0, 15, 16, 99]
    free_before = a.num_free()
    slots, cows = a.step(seqs)
    assert free_before - a.num_free() == 2 and cows == []
    assert [a.length(s) for s in seqs] == [1, 16, 17, 100]
    waste = [len(a.table(s)) * 16 - a.length(s) for s in seqs]
    assert waste == [15, 0, 15, 12]


def test_shared_prefix_workload_structure():
    w = inputs.small("shared_prefix_batch")
    a = PyAllocator(w.NB, w.bs, inputs.free_order(w))
    ids = run_script(a, inputs.setup_script(w))
    check_invariants(a)
    seqs = [ids[b] for b in range(w.B)]
    assert [a.length(s) for s in seqs] == list(w.cached_lengths)
    for g0 in range(0, w.B, w.group):
        grp = seqs[g0:g0 + w.group]
        shared = min(min(a.length(s) for s in grp), w.prefix_tokens) // 16
        first = [a.table(s)[:shared] for s in grp]
        assert all(f == first[0] for f in first)
    _, cows = a.step(seqs)
    check_invariants(a)
    for s in seqs:                              # no sequence writes into a shared block
        blk = a.table(s)[(a.length(s) - 1) // 16]
        assert a.refcount[blk] == 1


@settings(max_examples=60, deadline=None)
@given(ops=st.lists(st.tuples(st.sampled_from(["create", "reserve", "fork", "free", "step"]),
                              st.integers(0, 30), st.integers(0, 40)), max_size=40))
def test_invariants_random_scripts(ops):
    a = PyAllocator(24, 4, free_order=list(range(23, -1, -1)))
    live = []
    for op, x, n in ops:
        try:
            if op == "create" or not live:
                live.append(a.create())
            elif op == "reserve":
                a.reserve(live[x % len(live)], n % 9)
            elif op == "fork":
                p = live[x % len(live)]
                live.append(a.fork(p, n % (a.length(p) + 1)))
            elif op == "free":
                a.release(live.pop(x % len(live)))
            else:
                sel = live[x % len(live):][: 1 + n % 4]
                before = {s: (a.table(s), a.length(s)) for s in sel}
                slots, _ = a.step(sel)
                for s, slot in zip(sel, slots):
                    assert a.refcount[slot // 4] == 1       # written block is private
                    assert slot % 4 == before[s][1] % 4
        except OutOfBlocks:
            pass
        check_invariants(a)
