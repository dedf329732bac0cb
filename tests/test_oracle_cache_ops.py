"""Pins for oracle.cache_ops: each write is checked through flat byte offsets of the pool, a
second reading of the layout that does not use the oracle's multi-index assignment."""
import numpy as np

from oracle import cache_ops

NB, H, BS, D = 7, 3, 16, 8


def _pools(rng):
    return (rng.standard_normal((NB, H, BS, D)).astype(np.float32),
            rng.standard_normal((NB, H, D, BS)).astype(np.float32))


def test_append_writes_only_its_slots():
    rng = np.random.default_rng(1)
    k, v = _pools(rng)
    kn = rng.standard_normal((4, H, D)).astype(np.float32)
    vn = rng.standard_normal((4, H, D)).astype(np.float32)
    slots = np.array([5 * BS + 3, -1, 0, 6 * BS + 15])
    k2, v2 = cache_ops.append(k, v, kn, vn, slots, BS)
    kf, vf = k.reshape(-1).copy(), v.reshape(-1).copy()
    for b, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = s // BS, s % BS
        for g in range(H):
            for d in range(D):
                kf[((blk * H + g) * BS + off) * D + d] = kn[b, g, d]
                vf[((blk * H + g) * D + d) * BS + off] = vn[b, g, d]
    assert np.array_equal(k2.reshape(-1), kf)
    assert np.array_equal(v2.reshape(-1), vf)
    assert np.array_equal(k, _pools(np.random.default_rng(1))[0])  # input untouched


def test_copy_blocks_whole_tiles_in_order():
    rng = np.random.default_rng(2)
    k, v = _pools(rng)
    ks = rng.random((NB, H)).astype(np.float32)
    vs = rng.random((NB, H)).astype(np.float32)
    pairs = [(1, 4), (4, 6)]  # chained: block 6 gets block 1's content
    k2, v2, ks2, vs2 = cache_ops.copy_blocks(k, v, pairs, ks, vs)
    tile = H * BS * D
    kf = k.reshape(-1).copy()
    for src, dst in pairs:
        kf[dst * tile:(dst + 1) * tile] = kf[src * tile:(src + 1) * tile]
    assert np.array_equal(k2.reshape(-1), kf)
    assert np.array_equal(v2[6], v[1]) and np.array_equal(v2[4], v[1])
    assert np.array_equal(ks2[6], ks[1]) and np.array_equal(vs2[4], vs[1])
    for blk in (0, 2, 3, 5):
        assert np.array_equal(k2[blk], k[blk]) and np.array_equal(v2[blk], v[blk])
