"""Pins for the prefix-cache oracle: the published FNV-1a vectors, the figures the page gives
(tests/golden/prefix_cache.txt), brute force on the matching rule, and the state invariants."""
import random

import pytest

from oracle.allocator import OutOfBlocks, PyAllocator
from oracle.prefix_cache import PrefixCachingAllocator, block_hash, chain_root, fnv1a64
from tests.golden.load import load

G = load("prefix_cache.txt")
BS = G["block_size"]


def test_fnv1a64_published_vectors():
    # reference values of 64-bit FNV-1a
    assert fnv1a64(b"") == 0xcbf29ce484222325
    assert fnv1a64(b"a") == 0xaf63dc4c8601ec8c
    assert fnv1a64(b"foobar") == 0x85944171f73967e8


def test_block_hash_is_fnv_of_parent_then_ids():
    # the byte string is spelled out here, independently of block_hash's own packing
    parent = 0x0123456789ABCDEF
    ids = [1, -2, 300, 7] + [0] * 12
    data = bytes([0xEF, 0xCD, 0xAB, 0x89, 0x67, 0x45, 0x23, 0x01])
    data += bytes([1, 0, 0, 0]) + bytes([0xFE, 0xFF, 0xFF, 0xFF]) + bytes([44, 1, 0, 0])
    data += bytes([7, 0, 0, 0]) + bytes(4 * 12)
    assert block_hash(parent, ids) == fnv1a64(data)
    assert chain_root(5) == fnv1a64(bytes([5, 0, 0, 0, 0, 0, 0, 0]))


def _prompt(rng, n, vocab=50000):
    return [rng.randrange(vocab) for _ in range(n)]


def _prefill(a, tokens, salt=0):
    sid, cached = a.create_prefix(tokens, salt)
    a.reserve(sid, len(tokens) - cached)
    return sid, cached


def test_page_example_3000_shared_tokens():
    rng = random.Random(1)
    n = G["shared_prefix_tokens"]
    shared = _prompt(rng, n)
    a = PrefixCachingAllocator(1024, BS)
    first, cached0 = _prefill(a, shared + _prompt(rng, 500))
    assert cached0 == 0
    second, cached = _prefill(a, shared + _prompt(rng, 40))
    assert cached == G["reused_tokens_3000"]
    assert a.table(second)[:G["reused_blocks_3000"]] == a.table(first)[:G["reused_blocks_3000"]]
    # block 187 holds tokens 2992..3007: the two prompts differ inside it, so it is not shared
    assert a.table(second)[187] != a.table(first)[187]


def test_page_example_early_change_breaks_the_chain():
    rng = random.Random(2)
    p = _prompt(rng, 2000)
    a = PrefixCachingAllocator(512, BS)
    _prefill(a, p)
    q = list(p)
    q[G["changed_token_index"]] += 1
    _, cached = _prefill(a, q)
    assert cached == G["reused_tokens_change_at_100"]


def test_salt_isolates_tenants():
    rng = random.Random(3)
    p = _prompt(rng, 700)
    a = PrefixCachingAllocator(512, BS)
    _prefill(a, p, salt=11)
    assert _prefill(a, p, salt=12)[1] == 0
    assert _prefill(a, p, salt=0)[1] == 0
    assert _prefill(a, p, salt=11)[1] == (700 - 1) // BS * BS


def test_at_least_one_prompt_token_is_left_to_compute():
    rng = random.Random(4)
    p = _prompt(rng, 4 * BS)          # exactly four full blocks
    a = PrefixCachingAllocator(64, BS)
    _prefill(a, p)
    assert _prefill(a, p)[1] == 3 * BS
    assert _prefill(a, p + [5])[1] == 4 * BS
    assert a.create_prefix([])[1] == 0


def test_released_cached_blocks_stay_matchable_until_evicted():
    rng = random.Random(5)
    a = PrefixCachingAllocator(8, BS, free_order=range(8))
    p = _prompt(rng, 3 * BS + 5)      # 3 full blocks published, a 4th partial one private
    sid, _ = _prefill(a, p)
    table = a.table(sid)
    a.release(sid)
    # the partial block is freed; the three published ones become evictable, last first
    assert a.free_list() == [4, 5, 6, 7, table[3]]
    assert a.evictable_list() == [table[2], table[1], table[0]]
    # a hit revives them
    sid2, cached = _prefill(a, p)
    assert cached == 3 * BS and a.table(sid2)[:3] == table[:3] and a.num_evictable() == 0
    a.release(sid2)
    # use up the free list, then each allocation evicts the least recently used cached block
    other = a.create()
    a.reserve(other, 5 * BS)
    assert a.num_free() == 0 and a.num_evictable() == 3
    a.reserve(other, 1)
    assert a.table(other)[-1] == table[2] and a.block_hash(table[2]) is None
    assert a.evictable_list() == [table[1], table[0]]
    # the chain now stops at the evicted block... which was the last; the first two still match
    assert a.create_prefix(p)[1] == 2 * BS


def test_out_of_blocks_rolls_back_evictions():
    rng = random.Random(6)
    a = PrefixCachingAllocator(6, BS)
    p = _prompt(rng, 2 * BS + 1)
    sid, _ = _prefill(a, p)
    a.release(sid)
    before = (a.free_list(), a.evictable_list(), dict(a.cache), a.refcount[:])
    other = a.create()
    with pytest.raises(OutOfBlocks):
        a.reserve(other, 7 * BS)       # needs 7 blocks, 6 exist
    assert (a.free_list(), a.evictable_list(), dict(a.cache), a.refcount[:]) == before


def _longest_cached_prefix(prompts_cached, tokens):
    """Brute force: the longest run of whole blocks that some earlier published prompt shares
    with `tokens`, capped so that one token is left to compute."""
    best = 0
    cap = (len(tokens) - 1) // BS
    for q in prompts_cached:
        k = 0
        while (k < cap and (k + 1) * BS <= len(q)
               and q[k * BS:(k + 1) * BS] == tokens[k * BS:(k + 1) * BS]):
            k += 1
        best = max(best, k)
    return best * BS


def test_matching_rule_by_brute_force():
    rng = random.Random(7)
    a = PrefixCachingAllocator(4096, BS)     # big enough that nothing is evicted
    roots = [_prompt(rng, 200, vocab=7) for _ in range(4)]
    seen = []
    for _ in range(60):
        r = rng.choice(roots)
        cut = rng.randrange(0, 201)
        tokens = r[:cut] + _prompt(rng, rng.randrange(0, 60), vocab=7)
        if not tokens:
            continue
        expect = _longest_cached_prefix(seen, tokens)
        sid, cached = _prefill(a, tokens)
        assert cached == expect
        seen.append(tokens)
        if rng.random() < 0.3:
            a.release(sid)


def _check_invariants(a: PrefixCachingAllocator):
    in_use = {b for b in range(a.num_blocks) if a.refcount[b] > 0}
    free, ev = set(a.free_list()), set(a.evictable_list())
    assert len(free) == a.num_free() and len(ev) == a.num_evictable()
    assert not (free & ev) and not (free & in_use) and not (ev & in_use)
    assert len(free) + len(ev) + len(in_use) == a.num_blocks
    assert all(a.block_hash(b) is not None for b in ev)
    assert all(a.block_hash(b) is None for b in free)
    for h, b in a.cache.items():
        assert a.info[b][0] == h
    # refcount = number of tables holding the block
    held = [0] * a.num_blocks
    for t in a.tables.values():
        for b in t:
            held[b] += 1
    assert held == a.refcount
    # every published block a live prompt-sequence holds carries that sequence's own ids
    for sid, t in a.tables.items():
        if sid not in a.ids:
            continue
        full = min(a.lengths[sid], len(a.ids[sid])) // BS
        for j in range(full):
            info = a.info.get(t[j])
            if info is not None:
                assert list(info[2]) == a.ids[sid][j * BS:(j + 1) * BS]


def test_invariants_on_random_scripts():
    rng = random.Random(8)
    for trial in range(20):
        a = PrefixCachingAllocator(40, BS, free_order=rng.sample(range(40), 40))
        roots = [_prompt(rng, 120, vocab=5) for _ in range(3)]
        live = []
        for _ in range(80):
            op = rng.random()
            try:
                if op < 0.35 or not live:
                    tokens = rng.choice(roots)[:rng.randrange(1, 121)]
                    sid, cached = a.create_prefix(tokens)
                    live.append(sid)
                    a.reserve(sid, len(tokens) - cached)
                elif op < 0.6:
                    a.step(rng.sample(live, min(len(live), 3)))
                elif op < 0.7:
                    s = rng.choice(live)
                    a.add_tokens(s, [rng.randrange(5)])
                elif op < 0.8:
                    s = rng.choice(live)
                    live.append(a.fork(s, rng.randrange(0, a.length(s) + 1)))
                else:
                    a.release(live.pop(rng.randrange(len(live))))
            except OutOfBlocks:
                pass
            _check_invariants(a)


def test_plain_sequences_behave_as_before():
    """Without create_prefix nothing is ever published: the same script leaves the same state
    as in the plain allocator."""
    rng = random.Random(9)
    order = rng.sample(range(30), 30)
    a, b = PrefixCachingAllocator(30, BS, order), PyAllocator(30, BS, order)
    ids = []
    for _ in range(300):
        op = rng.random()
        if op < 0.2 or not ids:
            ids.append((a.create(), b.create()))
        elif op < 0.5:
            x, y = rng.choice(ids)
            n = rng.randrange(1, 20)
            ra = rb = None
            try:
                ra = a.reserve(x, n)
            except OutOfBlocks:
                ra = "oom"
            try:
                rb = b.reserve(y, n)
            except OutOfBlocks:
                rb = "oom"
            assert ra == rb
        elif op < 0.7:
            x, y = rng.choice(ids)
            k = rng.randrange(0, a.length(x) + 1)
            ids.append((a.fork(x, k), b.fork(y, k)))
        else:
            x, y = ids.pop(rng.randrange(len(ids)))
            a.release(x)
            b.release(y)
        assert a.free_list() == b.free_list() and a.refcount == b.refcount
        assert a.num_evictable() == 0 and not a.cache
    assert [a.table(x) for x, _ in ids] == [b.table(y) for _, y in ids]


def test_a_block_matches_only_after_an_identical_prefix():
    """Block contents that were cached after a different prefix are not reused: the K/V of a
    token depends on everything before it."""
    rng = random.Random(10)
    A, B, X, C = (_prompt(rng, BS) for _ in range(4))
    a = PrefixCachingAllocator(64, BS)
    _prefill(a, A + B + [1])
    _prefill(a, X + C + [1])
    sid, cached = a.create_prefix(A + C + [1])
    assert cached == BS                  # A matches; C after A was never computed
    sid, cached = a.create_prefix(X + C + [2])
    assert cached == 2 * BS
