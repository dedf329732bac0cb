"""Pins for the quantising int8 append: a fresh one-token block equals the harness's absmax
quantiser on that token; the block scale always equals the absmax rule over the block's valid
tokens; rounding bounds, also on hypothesis-random token streams; blocks whose scale did not
grow keep their codes."""

import numpy as np
from hypothesis import given, settings, strategies as st

import inputs
from oracle.cache_ops import append_int8


def _empty(NB, Hkv, D, bs=16):
    return (np.zeros((NB, Hkv, bs, D), np.int8), np.zeros((NB, Hkv, D, bs), np.int8),
            np.zeros((NB, Hkv), np.float32), np.zeros((NB, Hkv), np.float32))


def test_fresh_block_equals_the_absmax_quantiser():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 2, 64)).astype(np.float32)
    kc, vc, ks, vs = append_int8(*_empty(4, 2, 64), x, x * 2, [3 * 16], 16)
    ref_codes, ref_scale = inputs.quantize_int8_pool(x[0][:, None, :], tile_axes=(1, 2))
    assert np.array_equal(kc[3, :, 0, :], ref_codes[:, 0, :])
    assert np.array_equal(ks[3], ref_scale)
    ref_v, ref_vs = inputs.quantize_int8_pool((2 * x[0])[:, None, :], tile_axes=(1, 2))
    assert np.array_equal(vc[3, :, :, 0], ref_v[:, 0, :]) and np.array_equal(vs[3], ref_vs)


def test_scale_is_the_block_absmax_rule_and_codes_are_bounded():
    rng = np.random.default_rng(1)
    Hkv, D, bs = 2, 32, 16
    state = _empty(2, Hkv, D)
    toks = []
    growths = np.zeros((bs, Hkv))        # scale growths each token has been re-rounded through
    for off in range(bs):
        x = (rng.standard_normal((1, Hkv, D)) * rng.uniform(0.1, 3)).astype(np.float32)
        toks.append(x[0])
        before = state[2][1].copy()
        state = append_int8(*state, x, x, [16 + off], bs)
        kc, vc, ks, vs = state
        if off:
            growths[:off] += (ks[1] > before)[None, :]
        allx = np.stack(toks)                                   # [off+1][Hkv][D]
        amax = np.max(np.abs(allx), axis=(0, 2)).astype(np.float32)
        assert np.array_equal(ks[1], amax / np.float32(127))    # the absmax rule, exactly
        assert np.array_equal(vs[1], ks[1])
        # the newest token is within half a step; each re-rounding adds at most half a step
        # of a scale no larger than the current one
        deq = kc[1, :, :off + 1, :].astype(np.float64) * ks[1][:, None, None]
        err = np.abs(deq - np.transpose(allx, (1, 0, 2)))          # [Hkv][off+1][D]
        assert np.all(err[:, off, :] <= ks[1][:, None] / 2 + 1e-12)
        bound = (growths[:off + 1].T + 1) * ks[1][:, None] / 2    # [Hkv][off+1]
        assert np.all(err <= bound[:, :, None] + 1e-12)
        assert np.all(np.abs(kc) <= 127)


def test_no_growth_leaves_codes_alone_and_growth_rerounds():
    Hkv, D = 1, 8
    big = np.full((1, Hkv, D), 4.0, np.float32)
    small = np.full((1, Hkv, D), 1.0, np.float32)
    s = append_int8(*_empty(1, Hkv, D), big, big, [0], 16)
    s2 = append_int8(*s, small, small, [1], 16)
    assert np.array_equal(s2[0][0, 0, 0], s[0][0, 0, 0]) and s2[2][0, 0] == s[2][0, 0]
    assert np.all(s2[0][0, 0, 1] == np.rint(np.float32(1.0) / s[2][0, 0]))
    # growth: 1.0 first, then 4.0 -> the first row is re-rounded by 1/4
    t = append_int8(*_empty(1, Hkv, D), small, small, [0], 16)
    t2 = append_int8(*t, big, big, [1], 16)
    assert np.all(t[0][0, 0, 0] == 127) and np.all(t2[0][0, 0, 1] == 127)
    r = np.float32(t[2][0, 0]) / np.float32(t2[2][0, 0])
    assert np.all(t2[0][0, 0, 0] == np.rint(np.float32(127) * r))     # 31.75 -> 32


def test_zero_tokens_keep_scale_zero_until_data_arrives():
    z = np.zeros((1, 1, 8), np.float32)
    s = append_int8(*_empty(1, 1, 8), z, z, [0], 16)
    assert s[2][0, 0] == 0 and np.all(s[0][0, 0, 0] == 0)
    x = np.linspace(-1, 1, 8, dtype=np.float32).reshape(1, 1, 8)
    s2 = append_int8(*s, x, x, [1], 16)
    assert s2[2][0, 0] == np.float32(1) / np.float32(127)
    assert np.all(s2[0][0, 0, 0] == 0) and s2[0][0, 0, 1, -1] == 127


def test_batch_order_and_skips():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 1, 8)).astype(np.float32)
    both = append_int8(*_empty(2, 1, 8), x, x, [0, -1, 1], 16)
    one = append_int8(*_empty(2, 1, 8), x[:1], x[:1], [0], 16)
    two = append_int8(*one, x[2:], x[2:], [1], 16)
    for a, b in zip(both, two):
        assert np.array_equal(a, b)


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 2**31 - 1), st.integers(1, 40),
       st.lists(st.sampled_from([0.0, 1e-3, 0.25, 1.0, 4.0, 100.0]), min_size=1, max_size=40),
       st.integers(1, 2))
def test_growth_keeps_every_token_within_its_accumulated_half_steps(seed, n, mags, Hkv):
    """Random token streams spread over three blocks in interleaved order (magnitudes from 0 to
    100, so scales grow, stay, and start from zero): after every append each block's scale is the
    absmax rule over its tokens so far, and every earlier token decodes to within
    (1 + the growths since it was written) half-steps of the final scale (each rounding, the
    first and every re-rounding, is off by at most half a step of a scale no larger than the
    current one).  The quotient x / s and the product code * ratio are float32 values before
    they are rounded to a code: each is off by at most 127 units of 2^-24 of a step, and a
    ratio s_old / s_new rounded to float32 adds as much again, so a rounding's bound is
    (1/2 + 2^-15) steps.  A wrong growth ratio, a missing re-rounding or a truncating rounding
    breaks it."""
    rng = np.random.default_rng(seed)
    D, bs, nblk = 8, 16, 3
    state = _empty(nblk, Hkv, D)
    toks = {k: [] for k in range(nblk)}          # block -> [(x [Hkv][D], growths so far)]
    for i in range(min(n, nblk * bs)):
        blk = int(rng.integers(nblk))
        if len(toks[blk]) == bs:
            continue
        off = len(toks[blk])
        x = (rng.standard_normal((1, Hkv, D)) * mags[i % len(mags)]).astype(np.float32)
        before = state[2][blk].copy()
        state = append_int8(*state, x, -x, [blk * bs + off], bs)
        kc, vc, ks, vs = state
        grew = ks[blk] > before if off else np.zeros(Hkv, bool)
        toks[blk] = [(t, g + grew) for t, g in toks[blk]] + [(x[0], np.zeros(Hkv))]
        allx = np.stack([t for t, _ in toks[blk]])                       # [n][Hkv][D]
        amax = np.max(np.abs(allx), axis=(0, 2)).astype(np.float32)
        assert np.array_equal(ks[blk], amax / np.float32(127))
        assert np.array_equal(vs[blk], ks[blk])
        assert np.all(np.abs(kc) <= 127) and np.all(np.abs(vc) <= 127)
        for j, (t, g) in enumerate(toks[blk]):
            bound = (1 + g) * ks[blk].astype(np.float64) * (0.5 + 2.0**-15) + 1e-12  # [Hkv]
            kd = kc[blk, :, j, :].astype(np.float64) * ks[blk][:, None]
            vd = vc[blk, :, :, j].astype(np.float64) * vs[blk][:, None]
            assert np.all(np.abs(kd - t) <= bound[:, None])
            assert np.all(np.abs(vd + t) <= bound[:, None])
