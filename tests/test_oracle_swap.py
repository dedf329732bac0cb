"""Pins for the swapping oracle: a swap-out releases exactly what freeing the sequence would,
a swap-out / swap-in round trip restores the length and gives a table of the same size, the
free counts of both pools add up, and running out of either pool changes nothing."""
import random

import pytest

from oracle.allocator import BadSequence, OutOfBlocks, PyAllocator
from oracle.swap import SwapSpaceFull, SwappingAllocator


def test_swap_out_releases_like_free():
    a = SwappingAllocator(20, 16, range(20), num_cpu_blocks=10)
    b = PyAllocator(20, 16, range(20))
    for al in (a, b):
        s = al.create()
        al.reserve(s, 50)
        c = al.fork(s, 20)
        al.reserve(c, 5)
    table = a.table(0)
    pairs = a.swap_out(0)
    b.release(0)
    assert a.free_list() == b.free_list() and a.refcount == b.refcount
    assert [p[0] for p in pairs] == table                     # shared blocks are copied too
    assert [p[1] for p in pairs] == [0, 1, 2, 3] and a.num_free_swap() == 6
    assert a.length(0) == 50
    with pytest.raises(BadSequence):
        a.reserve(0, 1)


def test_round_trip_restores_length_and_size():
    a = SwappingAllocator(16, 16, range(16), num_cpu_blocks=8)
    s = a.create()
    a.reserve(s, 70)
    out = a.swap_out(s)
    assert a.num_free() == 16 and len(out) == 5
    other = a.create()
    a.reserve(other, 16 * 10)                 # reuse the released blocks
    back = a.swap_in(s)
    assert a.length(s) == 70 and len(a.table(s)) == 5
    assert [p[0] for p in back] == [p[1] for p in out]
    assert [p[1] for p in back] == a.table(s)
    assert a.num_free_swap() == 8 and a.num_free() == 16 - 10 - 5
    slots, _ = a.reserve(s, 1)                # appends continue in the last block
    assert slots[0] == a.table(s)[4] * 16 + 70 % 16


def test_running_out_changes_nothing():
    a = SwappingAllocator(8, 16, range(8), num_cpu_blocks=2)
    s = a.create()
    a.reserve(s, 48)                          # 3 blocks, swap pool holds 2
    with pytest.raises(SwapSpaceFull):
        a.swap_out(s)
    assert a.table(s) == [0, 1, 2] and a.num_free_swap() == 2
    t = a.create()
    a.reserve(t, 32)
    out = a.swap_out(t)
    u = a.create()
    a.reserve(u, 16 * 5)                      # the device is full now
    state = (a.free_list(), a.num_free_swap(), a.refcount[:])
    with pytest.raises(OutOfBlocks):
        a.swap_in(t)
    assert (a.free_list(), a.num_free_swap(), a.refcount[:]) == state
    assert len(out) == 2


def test_pool_counts_add_up_on_random_scripts():
    rng = random.Random(3)
    a = SwappingAllocator(30, 16, rng.sample(range(30), 30), num_cpu_blocks=12)
    live = []
    for _ in range(400):
        op = rng.random()
        try:
            if op < 0.25 or not live:
                s = a.create()
                live.append(s)
                a.reserve(s, rng.randrange(1, 40))
            elif op < 0.45:
                s = rng.choice(live)
                if s in a.swapped:
                    a.swap_in(s)
                else:
                    a.swap_out(s)
            elif op < 0.75:
                res = [s for s in live if s not in a.swapped]
                if res:
                    a.step(rng.sample(res, min(3, len(res))))
            else:
                a.release(live.pop(rng.randrange(len(live))))
        except (OutOfBlocks, SwapSpaceFull):
            pass
        used_cpu = sum(len(c) for c, _ in a.swapped.values())
        assert used_cpu + a.num_free_swap() == 12
        in_use = sum(1 for r in a.refcount if r > 0)
        assert in_use + a.num_free() + a.num_evictable() == 30
        for s, (c, n) in a.swapped.items():
            assert len(c) == -(-n // 16)
