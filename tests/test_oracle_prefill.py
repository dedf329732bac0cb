"""Pins for the chunked-prefill oracle: a library routine (torch's causal scaled-dot-product
attention in float64 on the CPU, with the KV heads repeated for GQA), the defining properties of
causal attention (a chunked prefill equals the same rows of the whole prefill; the first token
attends only to itself), paging invariance, and brute force."""
import math

import numpy as np
import pytest
import torch

from oracle import attention
from oracle.prefill import prefill_paged


def _paged(rng, L, Hkv, D, bs, NB, shuffle=True):
    """A contiguous K, V [Hkv][L][D] float64 (bf16-representable) and a pool holding it."""
    K = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    V = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    nblk = -(-L // bs)
    perm = rng.permutation(NB)[:nblk]
    blocks = perm if shuffle else np.arange(nblk)
    kp = np.zeros((NB, Hkv, bs, D), np.float32)
    vp = np.zeros((NB, Hkv, D, bs), np.float32)
    for t in range(L):
        kp[blocks[t // bs], :, t % bs, :] = K[:, t, :]
        vp[blocks[t // bs], :, :, t % bs] = V[:, t, :]
    table = np.full(8 + nblk, -1, np.int64)
    table[:nblk] = blocks
    return K.astype(np.float64), V.astype(np.float64), kp, vp, table


@pytest.mark.parametrize("G", [1, 4])
def test_whole_prompt_equals_torch_causal_sdpa(G):
    rng = np.random.default_rng(0)
    L, Hkv, D, bs = 37, 2, 16, 16
    K, V, kp, vp, table = _paged(rng, L, Hkv, D, bs, 16)
    q = rng.standard_normal((L, Hkv * G, D)).astype(np.float32)
    scale = 1 / math.sqrt(D)
    out = prefill_paged(q, "f32", kp, vp, "f32", [table], [L], [0, L], bs, scale)
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)          # [Hq][L][D]
    kt = torch.from_numpy(K).repeat_interleave(G, dim=0)                  # [Hq][L][D]
    vt = torch.from_numpy(V).repeat_interleave(G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    assert np.max(np.abs(out - ref.permute(1, 0, 2).numpy())) <= 1e-12


def test_chunks_equal_rows_of_the_whole_prefill():
    rng = np.random.default_rng(1)
    L, Hkv, G, D, bs = 70, 2, 2, 8, 16
    _, _, kp, vp, table = _paged(rng, L, Hkv, D, bs, 12)
    q = rng.standard_normal((L, Hkv * G, D)).astype(np.float32)
    whole = prefill_paged(q, "f32", kp, vp, "f32", [table], [L], [0, L], bs, 0.3)
    for start in (0, 5, 33, 69):
        # the chunk is rows start..L-1; its context is the whole sequence
        chunk = prefill_paged(q[start:], "f32", kp, vp, "f32", [table], [L], [0, L - start], bs,
                              0.3)
        assert np.array_equal(chunk, whole[start:])
        # and the same chunk as of an earlier step: context cut at end
        end = min(start + 7, L)
        part = prefill_paged(q[start:end], "f32", kp, vp, "f32", [table], [end],
                             [0, end - start], bs, 0.3)
        assert np.array_equal(part, whole[start:end])


def test_first_token_attends_only_to_itself():
    rng = np.random.default_rng(2)
    L, Hkv, D, bs = 20, 1, 8, 16
    K, V, kp, vp, table = _paged(rng, L, Hkv, D, bs, 4)
    q = rng.standard_normal((L, 3, D)).astype(np.float32)
    out = prefill_paged(q, "f32", kp, vp, "f32", [table], [L], [0, L], bs, 0.5)
    for h in range(3):
        assert np.array_equal(out[0, h], V[0, 0])


def test_last_row_is_a_decode_step():
    rng = np.random.default_rng(3)
    L, Hkv, G, D, bs = 45, 2, 4, 16, 16
    _, _, kp, vp, table = _paged(rng, L, Hkv, D, bs, 8)
    q = rng.standard_normal((9, Hkv * G, D)).astype(np.float32)
    out = prefill_paged(q, "f32", kp, vp, "f32", [table], [L], [0, 9], bs, 0.25)
    dec = attention.decode_paged(q[-1:], "f32", kp, vp, "f32", [table], [L], bs, 0.25)
    assert np.array_equal(out[-1], dec[0])


def test_paging_invariance_and_batching():
    rng = np.random.default_rng(4)
    Hkv, G, D, bs = 2, 2, 8, 16
    lens, chunks = [30, 64, 5], [30, 17, 5]
    cu = np.concatenate([[0], np.cumsum(chunks)])
    q = rng.standard_normal((int(cu[-1]), Hkv * G, D)).astype(np.float32)
    outs = []
    for shuffle in (False, True):
        rng2 = np.random.default_rng(5)
        tabs, kps, vps = [], [], []
        # one pool per sequence, concatenated: tables offset into it
        NB_each = 8
        kp = np.zeros((NB_each * 3, Hkv, bs, D), np.float32)
        vp = np.zeros((NB_each * 3, Hkv, D, bs), np.float32)
        for b, L in enumerate(lens):
            _, _, k1, v1, t1 = _paged(rng2, L, Hkv, D, bs, NB_each, shuffle)
            kp[b * NB_each:(b + 1) * NB_each] = k1
            vp[b * NB_each:(b + 1) * NB_each] = v1
            tabs.append(np.where(t1 >= 0, t1 + b * NB_each, -1))
        outs.append(prefill_paged(q, "f32", kp, vp, "f32", tabs, lens, cu, bs, 0.4))
    assert np.array_equal(outs[0], outs[1])
    # each sequence alone gives the same rows
    for b in range(3):
        alone = prefill_paged(q[cu[b]:cu[b + 1]], "f32", kp, vp, "f32", [tabs[b]], [lens[b]],
                              [0, chunks[b]], bs, 0.4)
        assert np.array_equal(alone, outs[1][cu[b]:cu[b + 1]])


def test_chunk_longer_than_context_gives_zero_rows():
    rng = np.random.default_rng(6)
    _, _, kp, vp, table = _paged(rng, 3, 1, 4, 16, 2)
    q = rng.standard_normal((5, 1, 4)).astype(np.float32)
    out = prefill_paged(q, "f32", kp, vp, "f32", [table], [3], [0, 5], 16, 1.0)
    assert np.all(out[:2] == 0) and np.all(np.isfinite(out))


def test_brute_force_scalar():
    rng = np.random.default_rng(7)
    L, D, bs = 19, 5, 16
    K, V, kp, vp, table = _paged(rng, L, 1, D, bs, 3)
    q = rng.standard_normal((6, 1, D)).astype(np.float32)
    out = prefill_paged(q, "f32", kp, vp, "f32", [table], [L], [0, 6], bs, 0.7)
    for i in range(6):
        p = L - 6 + i
        s = [0.7 * math.fsum(float(q[i, 0, d]) * K[0, t, d] for d in range(D)) for t in range(p + 1)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        Z = math.fsum(w)
        ref = [math.fsum(w[t] * V[0, t, d] for t in range(p + 1)) / Z for d in range(D)]
        assert np.max(np.abs(out[i, 0] - np.array(ref))) <= 1e-13
