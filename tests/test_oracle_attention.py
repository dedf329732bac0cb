"""Pins for oracle.attention, each against something other than the oracle itself:

* closed forms: one token returns its V exactly; identical keys or a zero query give the mean of V;
* paging invariance: attention through a shuffled pool and its block tables equals attention on
  the logically contiguous K/V, bit for bit (the pages: paging changes where bytes are, not the
  arithmetic);
* scalar brute force with math.exp / math.fsum over Python lists read from the pool by a
  pure-Python reading of the layout;
* grouped-query attention reduces to multi-head attention on repeated KV: torch's fp64
  scaled_dot_product_attention;
* the log-sum-exp merge of partition states equals the direct softmax.
A few planted mistakes (a transposed V read, a dropped max shift that overflows, an off-by-one
group mapping) are shown to fail these pins.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import inputs
from oracle import attention as A

BS = 16


# ---- helpers that build pools from logical K/V (test scaffolding, pure Python loops) -----------
def scatter_pool(Klog, Vlog, lens, NB, rng, poison=np.nan):
    """Place logical K/V [B][Hkv][Lmax][D] into a shuffled pool; unused slots hold `poison`."""
    B, Hkv, _, D = Klog.shape
    kp = np.full((NB, Hkv, BS, D), poison)
    vp = np.full((NB, Hkv, D, BS), poison)
    order = list(rng.permutation(NB))
    nblk = [-(-int(L) // BS) for L in lens]
    MB = max(max(nblk), 1)
    tables = np.full((B, MB), -1, np.int64)
    for b in range(B):
        for j in range(nblk[b]):
            tables[b, j] = order.pop()
        for t in range(int(lens[b])):
            blk, off = int(tables[b, t // BS]), t % BS
            for g in range(Hkv):
                for d in range(D):
                    kp[blk, g, off, d] = Klog[b, g, t, d]
                    vp[blk, g, d, off] = Vlog[b, g, t, d]
    return kp, vp, tables


def scalar_read(pool_k, pool_v, table, L, g, to_float, ks=None, vs=None):
    Kl, Vl = [], []
    D = pool_k.shape[-1]
    for t in range(L):
        blk = int(table[t // BS])
        off = t % BS
        sk = 1.0 if ks is None else float(ks[blk][g])
        sv = 1.0 if vs is None else float(vs[blk][g])
        Kl.append([to_float(pool_k[blk][g][off][d]) * sk for d in range(D)])
        Vl.append([to_float(pool_v[blk][g][d][off]) * sv for d in range(D)])
    return Kl, Vl


def bf16_to_float(bits):
    return float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0])


# ---- closed forms ------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_single_token_returns_its_value(dtype):
    rng = np.random.default_rng(5)
    D, Hkv, NB = 64, 2, 5
    raw_k = rng.standard_normal((NB, Hkv, BS, D)).astype(np.float32)
    raw_v = rng.standard_normal((NB, Hkv, D, BS)).astype(np.float32)
    ks = vs = None
    if dtype == "f32":
        kp, vp = raw_k, raw_v
    elif dtype == "bf16":
        kp, vp = inputs.bf16_bits(raw_k), inputs.bf16_bits(raw_v)
    else:
        kp, ks = inputs.quantize_int8_pool(raw_k)
        vp, vs = inputs.quantize_int8_pool(raw_v)
    q = rng.standard_normal((1, 4, D)).astype(np.float32)
    tables = np.array([[3]])
    out = A.decode_paged(q, "f32", kp, vp, dtype, tables, [1], BS, 0.125, ks, vs)
    for h in range(4):
        g = h // 2
        expect = A.to_f64(vp[3, g, :, 0], dtype)
        if dtype == "i8":
            expect = expect * float(vs[3, g])
        assert np.array_equal(out[0, h], expect)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(6)
    L, D = 37, 16
    k = rng.standard_normal(D)
    K = np.tile(k, (L, 1))
    V = rng.standard_normal((L, D))
    out = A.attend(rng.standard_normal(D), K, V, 0.3)
    mean = np.array([math.fsum(V[:, d]) / L for d in range(D)])
    assert np.max(np.abs(out - mean)) <= 1e-15 * 4


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(7)
    L, D = 50, 8
    K = rng.standard_normal((L, D)) * 10
    V = rng.standard_normal((L, D))
    out = A.attend(np.zeros(D), K, V, 1.0)
    mean = np.array([math.fsum(V[:, d]) / L for d in range(D)])
    assert np.max(np.abs(out - mean)) <= 4e-15


def test_empty_context_is_zero():
    out = A.decode_paged(np.ones((1, 2, 4), np.float32), "f32", np.zeros((2, 1, BS, 4), np.float32),
                         np.zeros((2, 1, 4, BS), np.float32), "f32", np.array([[-1]]), [0], BS, 1.0)
    assert np.array_equal(out, np.zeros((1, 2, 4)))


# ---- paging invariance -------------------------------------------------------------------------
@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), B=st.integers(1, 3), G=st.sampled_from([1, 2, 4]),
       maxlen=st.integers(1, 70))
def test_paging_invariance(seed, B, G, maxlen):
    rng = np.random.default_rng(seed)
    Hkv, D = 2, 8
    lens = rng.integers(0, maxlen, size=B, endpoint=True)
    Lmax = max(int(lens.max()), 1)
    Klog = rng.standard_normal((B, Hkv, Lmax, D))
    Vlog = rng.standard_normal((B, Hkv, Lmax, D))
    NB = sum(-(-int(L) // BS) for L in lens) + 3
    kp, vp, tables = scatter_pool(Klog, Vlog, lens, NB, rng)
    q = rng.standard_normal((B, Hkv * G, D))
    # fp64 pools and queries: treat them as already-widened values
    paged = A.decode_paged(q.astype(np.float32), "f32", kp.astype(np.float32),
                           vp.astype(np.float32), "f32", tables, lens, BS, 0.35)
    contig = A.decode_contiguous(q.astype(np.float32).astype(np.float64),
                                 Klog.astype(np.float32).astype(np.float64),
                                 Vlog.astype(np.float32).astype(np.float64), lens, 0.35)
    assert np.array_equal(paged, contig)


def test_paging_invariance_catches_transposed_v_read(monkeypatch):
    """Planted mistake: reading V token-major from a dim-major pool breaks the invariance."""
    rng = np.random.default_rng(11)
    lens = [40, 23]
    Klog = rng.standard_normal((2, 1, 40, BS))
    Vlog = rng.standard_normal((2, 1, 40, BS))
    kp, vp, tables = scatter_pool(Klog, Vlog, lens, 8, rng, poison=0.0)
    q = rng.standard_normal((2, 1, BS)).astype(np.float32)
    good = A.decode_contiguous(q.astype(np.float64), Klog, Vlog, lens, 0.2)

    def wrong_gather(k_pool, v_pool, kv_dtype, k_scale, v_scale, table, L, g, bs):
        t = np.arange(L)
        blk = np.asarray(table)[t // bs]
        return (A.to_f64(k_pool[blk, g, t % bs, :], kv_dtype),
                A.to_f64(v_pool[blk, g, t % bs, :], kv_dtype))  # token-major read
    monkeypatch.setattr(A, "gather_sequence", wrong_gather)
    bad = A.decode_paged(q, "f32", kp, vp, "f32", tables, lens, BS, 0.2)
    assert not np.allclose(bad, good)


# ---- scalar brute force ------------------------------------------------------------------------
def _brute_force_check(w, tol):
    pool = inputs.pool(w)
    q = inputs.queries(w)
    rng = np.random.default_rng(99)
    order = rng.permutation(w.NB)
    nblk = [-(-int(L) // BS) for L in w.lengths]
    tables = np.full((w.B, max(nblk)), -1)
    i = 0
    for b in range(w.B):
        for j in range(nblk[b]):
            tables[b, j] = order[i]
            i += 1
    ks, vs = pool.get("k_scale"), pool.get("v_scale")
    out = A.decode_paged(q, w.q_dtype, pool["k"], pool["v"], w.kv_dtype, tables, w.lengths, BS,
                         w.scale, ks, vs)
    kv_float = {"f32": float, "bf16": bf16_to_float, "i8": float}[w.kv_dtype]
    q_float = {"f32": float, "bf16": bf16_to_float}[w.q_dtype]
    worst = 0.0
    for b in range(w.B):
        for h in range(w.Hq):
            g = h // w.G
            Kl, Vl = scalar_read(pool["k"], pool["v"], tables[b], int(w.lengths[b]), g, kv_float,
                                 ks, vs)
            ref = A.decode_scalar([q_float(x) for x in q[b, h]], Kl, Vl, w.scale)
            worst = max(worst, float(np.max(np.abs(out[b, h] - np.array(ref)))))
    assert worst <= tol, worst


def test_brute_force_tiny_fp32():
    _brute_force_check(inputs.tiny_fp32(), 1e-13)


def test_brute_force_bf16_gqa():
    w = inputs.llama8b_decode(B=2, lo=1, hi=40, cid=90, name="bf")
    w.Hq, w.Hkv = 4, 1
    _brute_force_check(w, 1e-13)


def test_brute_force_int8():
    w = inputs.int8_mha(B=2, lo=1, hi=40, Hq=2, cid=91)
    _brute_force_check(w, 1e-13)


def test_brute_force_peaked_keys():
    w = inputs.long_context(lengths=(33, 7), cid=92)
    w.Hq, w.Hkv, w.peak_fraction, w.peak_factor = 2, 1, 0.2, 8.0
    _brute_force_check(w, 1e-13)


@settings(max_examples=20, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), L=st.integers(1, 40))
def test_brute_force_random(seed, L):
    rng = np.random.default_rng(seed)
    D = 6
    K = rng.standard_normal((L, D)) * 3
    V = rng.standard_normal((L, D))
    q = rng.standard_normal(D)
    ref = A.decode_scalar(list(q), K.tolist(), V.tolist(), 0.7)
    assert np.max(np.abs(A.attend(q, K, V, 0.7) - np.array(ref))) <= 1e-13


def test_unshifted_softmax_overflows_where_oracle_does_not():
    """Planted mistake: dropping the max shift overflows on large logits; the shifted oracle
    stays finite and matches brute force."""
    K = np.array([[800.0], [790.0]])
    V = np.array([[1.0], [2.0]])
    q = np.array([1.0])
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.exp(K @ q)
        naive = (w @ V) / w.sum()
    assert not np.all(np.isfinite(naive))
    ref = A.decode_scalar([1.0], K.tolist(), V.tolist(), 1.0)
    assert abs(A.attend(q, K, V, 1.0)[0] - ref[0]) <= 1e-13


# ---- grouped-query attention against torch's fp64 SDPA ----------------------------------------
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gqa_equals_mha_on_repeated_kv(G):
    rng = np.random.default_rng(20 + G)
    B, Hkv, D, L = 2, 2, 16, 45
    lens = [L, L]
    Klog = rng.standard_normal((B, Hkv, L, D))
    Vlog = rng.standard_normal((B, Hkv, L, D))
    q = rng.standard_normal((B, Hkv * G, D))
    kp, vp, tables = scatter_pool(Klog, Vlog, lens, 20, rng)
    ours = A.decode_paged(q.astype(np.float32), "f32", kp.astype(np.float32),
                          vp.astype(np.float32), "f32", tables, lens, BS, 0.25)
    qt = torch.from_numpy(q.astype(np.float32).astype(np.float64))[:, :, None, :]
    Kt = torch.from_numpy(Klog.astype(np.float32).astype(np.float64)).repeat_interleave(G, dim=1)
    Vt = torch.from_numpy(Vlog.astype(np.float32).astype(np.float64)).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=0.25)[:, :, 0, :]
    assert np.max(np.abs(ours - ref.numpy())) <= 1e-12


def test_gqa_pin_catches_wrong_group_mapping():
    """Planted mistake: query head h reading KV head h % Hkv instead of h // G."""
    rng = np.random.default_rng(3)
    Hkv, G, D, L = 2, 2, 8, 20
    K = rng.standard_normal((1, Hkv, L, D))
    V = rng.standard_normal((1, Hkv, L, D))
    q = rng.standard_normal((1, Hkv * G, D))
    right = A.decode_contiguous(q, K, V, [L], 0.5)
    wrong = np.stack([A.attend(q[0, h], K[0, h % Hkv], V[0, h % Hkv], 0.5)
                      for h in range(Hkv * G)])[None]
    qt = torch.from_numpy(q)[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, torch.from_numpy(K).repeat_interleave(G, 1), torch.from_numpy(V).repeat_interleave(G, 1),
        scale=0.5)[:, :, 0, :].numpy()
    assert np.max(np.abs(right - ref)) <= 1e-12
    assert np.max(np.abs(wrong - ref)) > 1e-3


# ---- split-K algebra ---------------------------------------------------------------------------
@settings(max_examples=30, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), L=st.integers(2, 300), parts=st.integers(1, 9))
def test_lse_combine_equals_direct_softmax(seed, L, parts):
    rng = np.random.default_rng(seed)
    D = 8
    K = rng.standard_normal((L, D)) * rng.choice([1.0, 8.0])
    V = rng.standard_normal((L, D))
    q = rng.standard_normal(D)
    cuts = sorted(set([0, L] + list(rng.integers(1, L, size=parts - 1))))
    states = [A.partition_state(q, K, V, 0.5, lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:])]
    ref = A.decode_scalar(list(q), K.tolist(), V.tolist(), 0.5)
    assert np.max(np.abs(A.combine_partitions(states) - np.array(ref))) <= 1e-13
