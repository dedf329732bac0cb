"""Pins for the int4 layout and the int4 parts of the oracle: a hand-packed row, the device
packer (inputs) against the oracle's reader, the quantiser at 4 bits, decode over a packed pool
against the same decode over the dequantised contiguous values, and the quantising append at
4 bits (fresh block = the absmax quantiser; scale rule; bounds)."""
import numpy as np

import inputs
from oracle import attention, int4
from oracle.cache_ops import append_int4


def test_hand_packed_row():
    codes = np.array([[-7, -6, -5, -4, -3, -2, -1, 0, 1, 2, 3, 4, 5, 6, 7, 7]])
    # elements 0..3 -> low nibbles of bytes 0..3, elements 4..7 -> their high nibbles
    want = np.array([[0x51, 0x62, 0x73, 0x84, 0xD9, 0xEA, 0xFB, 0xFC]], np.uint8)
    assert np.array_equal(inputs.pack_int4(codes), want)
    assert np.array_equal(int4.unpack_rows(want), codes)
    assert np.array_equal(int4.pack_rows(codes), want)
    for e in range(16):
        assert int4.code_at(want[0], e) == codes[0, e]


def test_packer_and_reader_agree_on_random_pools():
    rng = np.random.default_rng(0)
    c = rng.integers(-7, 8, (3, 2, 16, 64))
    assert np.array_equal(int4.unpack_rows(inputs.pack_int4(c)), c)
    row = inputs.pack_int4(c)[1, 1, 5]
    assert [int4.code_at(row, e) for e in range(64)] == c[1, 1, 5].tolist()


def test_quantiser_at_four_bits():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 2, 16, 32)).astype(np.float32)
    codes, s = inputs.quantize_int8_pool(x, qmax=7)
    assert np.abs(codes).max() == 7
    assert np.all(np.abs(codes.astype(np.float64) * s[:, :, None, None] - x)
                  <= s[:, :, None, None] / 2 + 1e-7)


def test_decode_over_packed_pool_equals_dequantised_contiguous():
    w = inputs.small("int4_mha")
    w.B = 3
    w.lengths = w.lengths[:3]
    pool = inputs.pool(w)
    rng = np.random.default_rng(2)
    order = rng.permutation(w.NB)
    lens = [int(x) for x in w.lengths]
    tables, used = [], 0
    for L in lens:
        n = -(-L // 16)
        tables.append(np.concatenate([order[used:used + n], -np.ones(4, int)]))
        used += n
    q = inputs.queries(w, 0)
    out = attention.decode_paged(q, "bf16", pool["k"], pool["v"], "i4", tables, lens, 16,
                                 w.scale, pool["k_scale"], pool["v_scale"])
    kc, vc = int4.unpack_pool(pool["k"], pool["v"])
    kd = kc.astype(np.float64) * pool["k_scale"][:, :, None, None]
    vd = vc.astype(np.float64) * pool["v_scale"][:, :, None, None]
    qf = attention.to_f64(q, "bf16")
    for b, L in enumerate(lens):
        t = np.arange(L)
        blk = np.asarray(tables[b])[t // 16]
        for h in range(w.Hq):
            K = kd[blk, h, t % 16, :]
            V = vd[blk, h, :, t % 16]
            s = w.scale * (K @ qf[b, h])
            p = np.exp(s - s.max())
            assert np.max(np.abs(out[b, h] - (p @ V) / p.sum())) <= 1e-12


def test_quantising_append_at_four_bits():
    rng = np.random.default_rng(3)
    Hkv, D, bs = 2, 32, 16
    kp = np.zeros((2, Hkv, bs, D // 2), np.uint8)
    vp = np.zeros((2, Hkv, D, bs // 2), np.uint8)
    ks = np.zeros((2, Hkv), np.float32)
    vs = np.zeros((2, Hkv), np.float32)
    state = (kp, vp, ks, vs)
    toks = []
    for off in range(bs):
        x = (rng.standard_normal((1, Hkv, D)) * rng.uniform(0.2, 3)).astype(np.float32)
        toks.append(x[0])
        state = append_int4(*state, x, x, [bs + off], bs)
        kc, vc = int4.unpack_pool(state[0], state[1])
        amax = np.max(np.abs(np.stack(toks)), axis=(0, 2)).astype(np.float32)
        assert np.array_equal(state[2][1], amax / np.float32(7))
        if off == 0:
            ref, ref_s = inputs.quantize_int8_pool(x[0][:, None, :], tile_axes=(1, 2), qmax=7)
            assert np.array_equal(kc[1, :, 0, :], ref[:, 0, :])
            assert np.array_equal(vc[1, :, :, 0], ref[:, 0, :])
        assert np.all(np.abs(kc[1, :, :off + 1, :]) <= 7)     # written slots (0x00 is -8)
        newest = kc[1, :, off, :].astype(np.float64) * state[2][1][:, None]
        assert np.all(np.abs(newest - x[0]) <= state[2][1][:, None] / 2 + 1e-9)
    assert np.all(state[0][0] == 0) and np.all(state[1][0] == 0)   # block 0 untouched
