"""Chunked-prefill attention over a paged KV cache, in float64.  TEST INFRASTRUCTURE ONLY.

What is computed ("How LLM Inference Serving Works", section "Two Phases: Prefill and Decode":
prefill runs all prompt tokens through the model at once, each token depending on all the ones
before it; section "Prefix Caching and Chunked Prefill" / "Chunked prefill": a long prefill is
split into pieces that run in successive steps).  A step gives sequence b a chunk of n_b new
query tokens, the last n_b of its L_b cached tokens (their K and V are already in the pool).
Query i of the chunk sits at position p = L_b - n_b + i and attends to every token up to and
including itself:

    out[i, h] = sum_{t <= p} softmax_t(scale * <q[i, h], K_t>) V_t,   K, V of KV head h // G.

A query attends exactly as a decode step would over the first p + 1 tokens, so the decode
oracle (attention.attend over the gathered prefix) is this computation's building block; the
chunk adds nothing but the per-query prefix length.  Queries are packed [T][Hq][D] with the
chunk of sequence b in rows cu_q[b] .. cu_q[b+1]-1.  A query whose position would be negative
(a chunk longer than its context) has no keys; its output is zero.
"""
from __future__ import annotations

import numpy as np

from oracle.attention import attend, gather_sequence, to_f64


def prefill_paged(q, q_dtype, k_pool, v_pool, kv_dtype, tables, seq_lens, cu_q, bs, scale,
                  k_scale=None, v_scale=None, rows=None):
    """out [T][Hq][D] float64.  With ``rows`` (a list of (query row, head)) only those are
    computed and the rest is NaN, for sampled checks of large chunks."""
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    qf = to_f64(q, q_dtype)
    out = np.full((T, Hq, D), np.nan if rows is not None else 0.0, np.float64)
    want = None if rows is None else set(rows)
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        r0, r1 = int(cu_q[b]), int(cu_q[b + 1])
        n = r1 - r0
        for g in range(Hkv):
            K, V = gather_sequence(k_pool, v_pool, kv_dtype, k_scale, v_scale, tables[b], L, g,
                                   bs)
            for i in range(n):
                p = L - n + i
                for h in range(g * G, (g + 1) * G):
                    if want is not None and (r0 + i, h) not in want:
                        continue
                    if p < 0:
                        out[r0 + i, h] = 0.0
                    else:
                        out[r0 + i, h] = attend(qf[r0 + i, h], K[:p + 1], V[:p + 1], scale)
    return out
