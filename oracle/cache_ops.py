"""Writes into the paged KV cache, defined by their effect on the pool.  TEST INFRASTRUCTURE ONLY.

Append ([Serving] "What the KV Cache Is": the cache grows by one token's K and V per decode
step; "The Life of a Request": that token lands in the last block of the request).  The new token of
sequence b goes to slot s_b = physical_block * bs + offset chosen by the allocator; a slot of -1
means "no write".  Every other byte of the pool is left as it was.

Copy-on-write ([Serving] "Sharing comes for free": a block held by several sequences is
duplicated at the moment one of them must write into it; [Walkthrough] "Step 8").  The whole physical block is copied
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


def append_int4(k_pool, v_pool, k_scale, v_scale, k_new, v_new, slots, bs):
    """The quantising append of append_int8 with 4-bit codes: 7 in place of 127 (scale =
    max|x| / 7, codes in [-7, 7]), on packed pools (layout in oracle.int4).  Returns copies of
    (k_pool, v_pool, k_scale, v_scale)."""
    from oracle import int4
    kc, vc = int4.unpack_pool(k_pool, v_pool)
    kc, vc, ks, vs = _append_quant(kc, vc, k_scale, v_scale, k_new, v_new, slots, bs, 7)
    kp, vp = int4.pack_pool(kc, vc)
    return kp, vp, ks, vs


def append_int8(k_codes, v_codes, k_scale, v_scale, k_new, v_new, slots, bs):
    """Quantising append into an int8 cache (the write side of a quantised cache, "LLM serving
    (vLLM, quantized inference): Visual walkthrough": KV kept as int8 with a scale per block).
    Returns copies of (k_codes, v_codes, k_scale, v_scale).

    k_new / v_new: [B][Hkv][D] float32 (bf16 inputs widen exactly).  Entries are applied in
    batch order; for entry b with slot s >= 0 (block blk, offset off) and every KV head g, for K
    and V alike, with x the new vector and all arithmetic in float32 (IEEE division,
    round-half-to-even):
      * c = max|x| / 127 is the scale the token alone would need;
      * off == 0 (a fresh block): scale := c;
      * otherwise, with the block's scale s: if c > s, the scale grows to c and the codes of
        the block's first off slots are re-rounded to it, code := clamp(rint(code * (s / c)),
        -127, 127); else the scale stays;
      * the new slot gets clamp(rint(x / scale), -127, 127), or 0 when the scale is 0.
    The scale of a block thus stays max over its tokens of max|x| / 127 (the absmax scale of the
    whole block's valid slots); a block with only zeros so far has scale 0 (it dequantises to
    zeros).  Earlier tokens' codes are re-rounded from their codes: the originals are gone.
    """
    return _append_quant(k_codes, v_codes, k_scale, v_scale, k_new, v_new, slots, bs, 127)


def _append_quant(k_codes, v_codes, k_scale, v_scale, k_new, v_new, slots, bs, qmax):
    """append_int8's rule with codes in [-qmax, qmax] (scale = max|x| / qmax)."""
    kc, vc = k_codes.copy(), v_codes.copy()
    ks, vs = k_scale.copy(), v_scale.copy()
    f32 = np.float32
    qm = f32(qmax)
    k_new = np.asarray(k_new, f32)
    v_new = np.asarray(v_new, f32)
    Hkv = kc.shape[1]
    for b, s in enumerate(np.asarray(slots).tolist()):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        for g in range(Hkv):
            for x, codes, scales, token_major in ((k_new[b, g], kc, ks, True),
                                                  (v_new[b, g], vc, vs, False)):
                cand = f32(np.max(np.abs(x))) / qm
                if off == 0:
                    scale = cand
                else:
                    old = scales[blk, g]
                    scale = old
                    if cand > old:
                        r = f32(old) / f32(cand)
                        tile = codes[blk, g]
                        prev = tile[:off, :] if token_major else tile[:, :off]
                        new_prev = np.clip(np.rint(prev.astype(f32) * r), -qm, qm)
                        if token_major:
                            tile[:off, :] = new_prev.astype(np.int8)
                        else:
                            tile[:, :off] = new_prev.astype(np.int8)
                        scale = cand
                if scale > 0:
                    q = np.clip(np.rint(x / f32(scale)), -qm, qm).astype(np.int8)
                else:
                    q = np.zeros_like(x, dtype=np.int8)
                if token_major:
                    codes[blk, g, off, :] = q
                else:
                    codes[blk, g, :, off] = q
                scales[blk, g] = scale
    return kc, vc, ks, vs
