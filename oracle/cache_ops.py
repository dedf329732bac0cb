"""Writes into the paged KV cache, defined by their effect on the pool.  TEST INFRASTRUCTURE ONLY.

Append ([Serving] "What the KV Cache Is": each decode step appends one more token's K and V;
"The Life of a Request": the token goes into the request's current block).  The new token of
sequence b goes to slot s_b = physical_block * bs + offset chosen by the allocator; a slot of -1
means "no write".  Every other byte of the pool is left as it was.

Copy-on-write ([Serving] "Sharing comes for free": a shared block is copied only when one
branch needs to write to it; [Walkthrough] "Step 8").  The whole physical block is copied
(all bs slots, K, V and, for int8 caches, both scales); the allocator then points the writer's
table at the copy.

Layouts: K pool [NB][Hkv][bs][D], V pool [NB][Hkv][D][bs], scales [NB][Hkv].
"""
from __future__ import annotations

import numpy as np


def append(k_pool, v_pool, k_new, v_new, slots, bs):
    """Return copies of the pools with token b's K/V [Hkv][D] written at slots[b] (>= 0)."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for b, s in enumerate(np.asarray(slots).tolist()):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        k_out[blk, :, off, :] = k_new[b]
        v_out[blk, :, :, off] = v_new[b]
    return k_out, v_out


def copy_blocks(k_pool, v_pool, pairs, k_scale=None, v_scale=None):
    """Return copies of the pools (and scales) with block dst := block src for each pair, in
    order."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    ks = None if k_scale is None else k_scale.copy()
    vs = None if v_scale is None else v_scale.copy()
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        k_out[dst] = k_out[src]
        v_out[dst] = v_out[src]
        if ks is not None:
            ks[dst] = ks[src]
            vs[dst] = vs[src]
    return k_out, v_out, ks, vs
