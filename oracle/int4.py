"""The packed int4 KV layout, read and written element by element.  TEST INFRASTRUCTURE ONLY.

INT4 keeps half a byte per element ([W] "Step 1": the KV bytes per element set the cache size,
so four bits halve INT8's cache again).  A (block, KV head) tile holds codes c in
[-7, 7] stored as the nibble u = c + 8, one fp32 scale per tile (K and V apart), x = c * scale.

Packing (the pages fix none): every group of 4 bytes holds 8 consecutive elements of a row --
elements 0..3 in the low nibbles of bytes 0..3, elements 4..7 in their high nibbles.
  K tile [bs][D/2] bytes: row = token, elements = dims (D/8 groups per row);
  V tile [D][bs/2] bytes: row = dim, elements = tokens (2 groups per row for bs = 16).
"""
from __future__ import annotations

import numpy as np


def _element_byte(e: int):
    """(byte offset inside the row, shift) of element e."""
    group, j = divmod(e, 8)
    return 4 * group + (j % 4), 4 * (j // 4)


def code_at(row_bytes, e: int) -> int:
    off, shift = _element_byte(e)
    return int((int(row_bytes[off]) >> shift) & 0xF) - 8


def unpack_rows(rows: np.ndarray) -> np.ndarray:
    """Codes of packed rows [..., n/2] -> int8 [..., n]: each 4-byte group gives its low nibbles
    (elements 0..3) then its high nibbles (elements 4..7)."""
    rows = np.asarray(rows, np.uint8)
    n = rows.shape[-1] * 2
    g = rows.reshape(rows.shape[:-1] + (n // 8, 4))
    lo = (g & 0xF).astype(np.int8) - 8
    hi = (g >> 4).astype(np.int8) - 8
    return np.concatenate([lo, hi], axis=-1).reshape(rows.shape[:-1] + (n,))


def pack_rows(codes: np.ndarray) -> np.ndarray:
    """Inverse of unpack_rows: int codes [..., n] in [-7, 7] -> packed bytes [..., n/2]."""
    codes = np.asarray(codes).astype(np.int16)
    n = codes.shape[-1]
    g = (codes + 8).astype(np.uint8).reshape(codes.shape[:-1] + (n // 8, 8))
    packed = (g[..., :4] & 0xF) | ((g[..., 4:] & 0xF) << 4)
    return packed.astype(np.uint8).reshape(codes.shape[:-1] + (n // 2,))


def unpack_pool(k_pool, v_pool):
    """Whole packed pools -> code pools K [NB][Hkv][bs][D], V [NB][Hkv][D][bs]."""
    return unpack_rows(k_pool), unpack_rows(v_pool)


def pack_pool(k_codes, v_codes):
    return pack_rows(k_codes), pack_rows(v_codes)


def k_codes(k_pool: np.ndarray, blk, g, off) -> np.ndarray:
    """K codes [L][D] of tokens at (blk[t], off[t]) of KV head g."""
    return unpack_rows(np.asarray(k_pool)[blk, g, off, :])


def v_codes(v_pool: np.ndarray, blk, g, off) -> np.ndarray:
    """V codes [L][D] of tokens at (blk[t], off[t]): element off[t] of every dim row."""
    rows = unpack_rows(np.asarray(v_pool)[blk, g])      # [L][D][bs]
    return rows[np.arange(len(blk)), :, np.asarray(off)]
