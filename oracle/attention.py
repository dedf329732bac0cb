"""Decode attention over a paged KV cache, in float64.  TEST INFRASTRUCTURE ONLY.

What is computed ([Serving] "What the KV Cache Is, and How Big It Gets"; [Walkthrough]
"Step 2"): to produce the next token, the query of the new token is compared against the key of
every earlier token and the values are mixed by those weights,

    s_t = scale * <q_h, K_t>,   out_h = sum_t softmax(s)_t * V_t,    t = 0 .. L-1.

Where the keys and values live ([Serving] "PagedAttention: Virtual Memory for the KV Cache";
[Walkthrough] "Step 7"): token t of a sequence sits in logical block t // bs at offset t % bs,
and the sequence's block table maps that logical block to a physical block of the pool.  The
attention kernel follows the table to gather K and V.  Paging changes only where the bytes are,
not the arithmetic ([Walkthrough] "Quick self-check": the FLOPs are unchanged).

Grouped-query attention ([Serving] "What the KV Cache Is": the Llama 3.1 8B example has four
query heads per KV head): query head h reads KV head h // G with G = Hq / Hkv (contiguous
groups; the pages do not say which query heads share a KV head, contiguous groups are the plain
reading).

Physical layout (the pages fix none; this is the layout both sides use):
    K pool [NB][Hkv][bs][D], V pool [NB][Hkv][D][bs], int8 scales [NB][Hkv] (K and V apart).
An int8 element dequantises to float64(code) * float64(scale of its (block, KV head)); the
product of an 8-bit integer and a 24-bit significand is exact in float64.  int4 caches hold
packed nibbles (layout in oracle.int4) and dequantise the same way.

An empty context (L = 0) has no keys; its output is defined as zero.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of one stored dtype to float64 ("f32", "bf16" bit patterns, "i8" codes)."""
    if dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "i8":
        return np.asarray(x, np.int8).astype(np.float64)
    raise ValueError(dtype)


def gather_sequence(k_pool, v_pool, kv_dtype, k_scale, v_scale, table, L, g, bs):
    """Keys and values of KV head g for logical tokens 0..L-1 of one sequence: two [L][D] f64.

    Token t lives in physical block table[t // bs] at offset t % bs.
    """
    t = np.arange(L)
    blk = np.asarray(table)[t // bs].astype(np.int64)   # physical block of each token
    off = t % bs                                        # slot inside that block
    if kv_dtype == "i4":                                # packed nibbles (oracle.int4)
        from oracle import int4
        K = int4.k_codes(k_pool, blk, g, off).astype(np.float64)
        V = int4.v_codes(v_pool, blk, g, off).astype(np.float64)
        K = K * np.asarray(k_scale, np.float32)[blk, g].astype(np.float64)[:, None]
        V = V * np.asarray(v_scale, np.float32)[blk, g].astype(np.float64)[:, None]
        return K, V
    K = to_f64(k_pool[blk, g, off, :], kv_dtype)        # [L][D]
    V = to_f64(v_pool[blk, g, :, off], kv_dtype)        # [L][D]
    if kv_dtype == "i8":
        K = K * np.asarray(k_scale, np.float32)[blk, g].astype(np.float64)[:, None]
        V = V * np.asarray(v_scale, np.float32)[blk, g].astype(np.float64)[:, None]
    return K, V


def attend(qh: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) weighted sum of V rows, one query vector; zeros when K is empty."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], np.float64)
    s = scale * (K @ qh)
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def decode_paged(q, q_dtype, k_pool, v_pool, kv_dtype, tables, lens, bs, scale,
                 k_scale=None, v_scale=None, heads: Sequence[Tuple[int, int]] = None):
    """Paged decode attention for a batch: out [B][Hq][D] float64.

    q [B][Hq][D] (f32 or bf16 bits), pools in the layout above, tables [B][max_blocks] int,
    lens [B].  With ``heads`` (a list of (b, h)) only those rows are computed and the rest of
    the output is NaN, for sampled checks of large batches.
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    qf = to_f64(q, q_dtype)
    out = np.full((B, Hq, D), np.nan)
    want = None if heads is None else set((int(b), int(h)) for b, h in heads)
    for b in range(B):
        L = int(lens[b])
        for g in range(Hkv):
            hs = [h for h in range(g * G, (g + 1) * G) if want is None or (b, h) in want]
            if not hs:
                continue
            K, V = gather_sequence(k_pool, v_pool, kv_dtype, k_scale, v_scale, tables[b], L, g,
                                   bs)
            for h in hs:
                out[b, h] = attend(qf[b, h], K, V, scale)
    return out


def decode_contiguous(q, K, V, lens, scale):
    """The same attention over logically contiguous float64 K/V [B][Hkv][Lmax][D] (no table)."""
    B, Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            out[b, h] = attend(q[b, h], K[b, h // G, :L], V[b, h // G, :L], scale)
    return out


def decode_scalar(q: List, K: List, V: List, scale: float) -> List[float]:
    """Scalar brute force for one query vector over Python lists (math.exp and math.fsum only).

    q: D floats; K, V: L lists of D floats.  Returns D floats.
    """
    L = len(K)
    if L == 0:
        return [0.0] * len(q)
    s = [scale * math.fsum(qd * kd for qd, kd in zip(q, K[t])) for t in range(L)]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    Z = math.fsum(w)
    return [math.fsum(w[t] * V[t][d] for t in range(L)) / Z for d in range(len(q))]


# ---- split-K algebra (the pages are silent; this is the log-sum-exp identity the kernel uses) --
def partition_state(qh, K, V, scale, lo, hi):
    """Softmax state of tokens [lo, hi): (m, l, o) with m = max score, l = sum exp(s - m) and
    o = sum exp(s - m) V / l (a normalised partial output)."""
    s = scale * (K[lo:hi] @ qh)
    m = s.max()
    w = np.exp(s - m)
    l = w.sum()
    return m, l, (w @ V[lo:hi]) / l


def combine_partitions(states):
    """Merge normalised partial states: M = max m_p, w_p = l_p exp(m_p - M),
    out = sum w_p o_p / sum w_p."""
    M = max(m for m, _, _ in states)
    w = [l * math.exp(m - M) for m, l, _ in states]
    num = sum(wp * o for wp, (_, _, o) in zip(w, states))
    return num / sum(w)
