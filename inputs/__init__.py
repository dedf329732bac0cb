"""Seeded synthetic inputs for the paged-KV decode path.

This module is shared by the CPU oracle tests, the GPU parity tests and the benchmark.  It only
*draws numbers* and states workload shapes: context lengths, the free-list permutation, query and
key/value values, the new tokens of each step, the int8 codes of the quantised-cache workload and
the script of allocator calls that builds each workload's sequences.  It holds none of the
method's arithmetic: no attention, no block-table gather, no allocation policy and no dequantised
product.  Both sides (oracle and HIP library) consume the exact bytes produced here.

Seeds follow ``numpy.random.default_rng([284, config_id, stream, ...])`` with the streams

    0 lengths, 1 free-list permutation, 2 queries, 3 K pool, 4 V pool,
    5 new-token K/V of a step, 6 peak mask (long-context workload),
    7 prompt token ids, 8 K/V of the tokens a request writes (prompt / prefill),
    9 chunk sizes of a chunked prefill, 10 the chunk's queries.

Physical layouts produced here (the library and the oracle document the same layouts):

    K pool  [NB][Hkv][bs][D]   token-major inside a (block, KV head) tile
    V pool  [NB][Hkv][D][bs]   dim-major inside a (block, KV head) tile
    scales  [NB][Hkv] fp32     int8 workloads only, one for K and one for V
    q       [B][Hq][D]
    k_new / v_new [B][Hkv][D]

Floating data is drawn as fp32 N(0, 1).  bf16 data is the fp32 draw rounded to nearest even and
is carried on the host as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np

SEED_ROOT = 284

KV_F32, KV_BF16, KV_I8, KV_I4 = "f32", "bf16", "i8", "i4"


# --------------------------------------------------------------------------------------------
# workload shapes
# --------------------------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    """One synthetic decode workload.

    ``lengths`` are the context lengths the *first* decode step attends over.  When the workload
    appends (``append`` is True, every float cache), the cache holds ``lengths - 1`` tokens after
    set-up and the first step writes token ``lengths - 1`` before attention; every later step
    appends one more token per sequence.  The int8 workload has no append: its cache is written
    once by :func:`quantize_int8_pool` and holds ``lengths`` tokens.
    """

    name: str
    cid: int                 # seed id
    B: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    kv_dtype: str            # "f32" | "bf16" | "i8"
    q_dtype: str             # "f32" | "bf16"
    lengths: np.ndarray      # int64 [B], context length seen by the first decode step
    NB: int                  # physical pool size in blocks
    append: bool
    steps: int = 1           # decode steps in one pass of the workload
    group: int = 0           # >0: sequences come in groups of this size sharing a prefix
    prefix_tokens: int = 0   # shared-prefix length of each group (tokens)
    peak_fraction: float = 0.0  # fraction of K tokens scaled by peak_factor
    peak_factor: float = 8.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def cached_lengths(self) -> np.ndarray:
        return self.lengths - 1 if self.append else self.lengths.copy()

    def max_len_after(self, steps: Optional[int] = None) -> int:
        s = self.steps if steps is None else steps
        return int(self.lengths.max()) + (s - 1 if self.append else 0)

    def describe(self) -> str:
        L = self.lengths
        return (f"{self.name}: B={self.B} Hq={self.Hq} Hkv={self.Hkv} D={self.D} bs={self.bs} "
                f"kv={self.kv_dtype} q={self.q_dtype} NB={self.NB} steps={self.steps} "
                f"L[min/mean/max]={L.min()}/{L.mean():.1f}/{L.max()} sumL={int(L.sum())}")


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([SEED_ROOT, *key])


def _blocks(n: np.ndarray, bs: int) -> np.ndarray:
    return (n + bs - 1) // bs


def _pool_with_slack(needed_blocks: int) -> int:
    return int(math.ceil(1.1 * needed_blocks))


def _group_unique_blocks(cached: np.ndarray, group: int, prefix: int, bs: int) -> int:
    """Blocks held once a prefix-sharing workload is set up (sizing only)."""
    total = 0
    for g0 in range(0, len(cached), group):
        c = cached[g0:g0 + group]
        shared = np.minimum(c, prefix)
        total += int(_blocks(np.array([shared.max()]), bs)[0])
        total += int(_blocks(np.maximum(c - prefix, 0), bs).sum())
    return total


def tiny_fp32() -> Workload:
    """B=4, lengths {1, 16, 17, 100} after one append, 4/2 heads, D=64, fp32, 64-block pool."""
    return Workload("tiny_fp32", 1, B=4, Hq=4, Hkv=2, D=64, bs=16, kv_dtype=KV_F32,
                    q_dtype=KV_F32, lengths=np.array([1, 16, 17, 100], np.int64), NB=64,
                    append=True)


def llama8b_decode(B: int = 64, lo: int = 512, hi: int = 4096, steps: int = 1,
                   cid: int = 2, name: str = "llama8b_decode") -> Workload:
    """Llama-3.1-8B single-layer decode shape: 32 Q / 8 KV heads, D=128, bf16, L ~ U{lo..hi}."""
    L = _rng(cid, 0).integers(lo, hi, size=B, endpoint=True).astype(np.int64)
    need = int(_blocks(L - 1, 16).sum())
    extra = B * (1 + (steps + 15) // 16)
    return Workload(name, cid, B=B, Hq=32, Hkv=8, D=128, bs=16, kv_dtype=KV_BF16,
                    q_dtype=KV_BF16, lengths=L, NB=_pool_with_slack(need) + extra, append=True,
                    steps=steps)


def llama8b_decode_tp8(steps: int = 1, cid: int = 2, name: str = "llama8b_decode_tp8") -> Workload:
    """One GPU's share of the Llama-3.1-8B decode layer split by KV head over 8 GPUs: the same
    batch and lengths (same seed), 4 query heads on its one KV head."""
    w = llama8b_decode(steps=steps, cid=cid, name=name)
    w.Hq, w.Hkv = w.Hq // 8, w.Hkv // 8
    return w


def long_context(lengths=(8192, 32768, 65536, 131072), cid: int = 3,
                 name: str = "long_context") -> Workload:
    """Split-K stress: Llama-3.1-8B layer shape, few very long sequences, peaked softmax."""
    L = np.asarray(lengths, np.int64)
    need = int(_blocks(L - 1, 16).sum())
    return Workload(name, cid, B=len(L), Hq=32, Hkv=8, D=128, bs=16, kv_dtype=KV_BF16,
                    q_dtype=KV_BF16, lengths=L, NB=_pool_with_slack(need) + 2 * len(L),
                    append=True, peak_fraction=0.01)


def shared_prefix_batch(B: int = 256, group: int = 8, prefix_tokens: int = 1024,
                        median: float = 1000.0, sigma: float = 1.0, lo: int = 1,
                        hi: int = 8192, steps: int = 16, cid: int = 4,
                        name: str = "shared_prefix_batch") -> Workload:
    """Continuous-batching mix: lognormal lengths, groups sharing a copy-on-write prefix."""
    x = _rng(cid, 0).lognormal(mean=math.log(median), sigma=sigma, size=B)
    L = np.clip(np.rint(x), lo, hi).astype(np.int64)
    cached = L - 1
    unique = _group_unique_blocks(cached, group, prefix_tokens, 16)
    extra = B * (2 + (steps + 15) // 16)
    return Workload(name, cid, B=B, Hq=32, Hkv=8, D=128, bs=16, kv_dtype=KV_BF16,
                    q_dtype=KV_BF16, lengths=L, NB=_pool_with_slack(unique) + extra,
                    append=True, steps=steps, group=group, prefix_tokens=prefix_tokens)


def int4_mha(B: int = 32, lo: int = 1, hi: int = 2048, Hq: int = 40, cid: int = 6,
             name: str = "int4_mha") -> Workload:
    """The int8_mha layer shape with a packed int4 cache (half a byte per element)."""
    w = int8_mha(B=B, lo=lo, hi=hi, Hq=Hq, cid=cid, name=name)
    w.kv_dtype = KV_I4
    return w


def int8_mha(B: int = 32, lo: int = 1, hi: int = 2048, Hq: int = 40, cid: int = 5,
             name: str = "int8_mha") -> Workload:
    """LLaMA-13B-like MHA layer (40/40 heads, D=128) with an int8 cache and fp32 scales."""
    L = _rng(cid, 0).integers(lo, hi, size=B, endpoint=True).astype(np.int64)
    need = int(_blocks(L, 16).sum())
    return Workload(name, cid, B=B, Hq=Hq, Hkv=Hq, D=128, bs=16, kv_dtype=KV_I8,
                    q_dtype=KV_BF16, lengths=L, NB=_pool_with_slack(need), append=False)


FULL = {
    "tiny_fp32": tiny_fp32,
    "llama8b_decode": llama8b_decode,
    "llama8b_decode_tp8": llama8b_decode_tp8,
    "long_context": long_context,
    "shared_prefix_batch": shared_prefix_batch,
    "int8_mha": int8_mha,
    "int4_mha": int4_mha,
}


def small(name: str) -> Workload:
    """Reduced versions of the full workloads: same head shapes and structure, lengths that the
    fp64 oracle finishes in seconds while still spanning several partitions and ragged tails."""
    if name == "tiny_fp32":
        return tiny_fp32()
    if name == "llama8b_decode":
        return llama8b_decode(B=8, lo=1, hi=1200, steps=3, cid=12, name="llama8b_small")
    if name == "long_context":
        return long_context(lengths=(700, 5000), cid=13, name="long_context_small")
    if name == "shared_prefix_batch":
        return shared_prefix_batch(B=16, group=8, prefix_tokens=96, median=80.0, sigma=1.0,
                                   lo=1, hi=400, steps=4, cid=14, name="shared_prefix_small")
    if name == "int8_mha":
        return int8_mha(B=6, lo=1, hi=700, cid=15, name="int8_mha_small")
    if name == "int4_mha":
        return int4_mha(B=6, lo=1, hi=700, cid=16, name="int4_mha_small")
    raise KeyError(name)


def full(name: str) -> Workload:
    return FULL[name]()


# --------------------------------------------------------------------------------------------
# allocator set-up script (what to call, not how the allocator answers)
# --------------------------------------------------------------------------------------------
def setup_script(w: Workload) -> List[Tuple]:
    """Allocator calls that build the workload's sequences, in order.

    Ops (sequence names are small integers local to the script; the batch order is 0..B-1):
      ("create", name)                 new empty sequence
      ("reserve", name, n)             n successive slot appends to that sequence
      ("fork", parent, n, child)       child shares the first n tokens of parent
      ("free", name)                   release a sequence
    Plain workloads create sequence b and reserve its cached length, in batch order.  Prefix
    workloads build, per group, a holder that reserves the longest shared prefix, fork each
    member from it with min(cached, prefix) tokens, reserve each member's private tokens, and
    release the holder.
    """
    cached = w.cached_lengths
    ops: List[Tuple] = []
    if w.group <= 0:
        for b in range(w.B):
            ops.append(("create", b))
            ops.append(("reserve", b, int(cached[b])))
        return ops
    holder_base = w.B
    for gi, g0 in enumerate(range(0, w.B, w.group)):
        members = list(range(g0, min(g0 + w.group, w.B)))
        shared = [int(min(cached[m], w.prefix_tokens)) for m in members]
        h = holder_base + gi
        ops.append(("create", h))
        ops.append(("reserve", h, max(shared)))
        for m, s in zip(members, shared):
            ops.append(("fork", h, s, m))
            ops.append(("reserve", m, int(cached[m]) - s))
        ops.append(("free", h))
    return ops


def free_order(w: Workload) -> np.ndarray:
    """Initial free-list order: a seeded permutation of the physical blocks (int32)."""
    return _rng(w.cid, 1).permutation(w.NB).astype(np.int32)


# --------------------------------------------------------------------------------------------
# numbers
# --------------------------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.  Finite inputs only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    xf, of = x.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for i in range(0, xf.size, step):
        u = xf[i:i + step].view(np.uint32)
        r = ((u >> 16) & 1) + np.uint32(0x7FFF)
        of[i:i + step] = ((u + r) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    out = np.empty(shape, np.float32)
    rng.standard_normal(dtype=np.float32, out=out)
    return out


def _cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == KV_F32:
        return x32
    if dtype == KV_BF16:
        return bf16_bits(x32)
    raise ValueError(dtype)


def queries(w: Workload, step: int = 0) -> np.ndarray:
    """q [B][Hq][D]: fp32 array or bf16 bits."""
    return _cast(_normal(_rng(w.cid, 2, step), (w.B, w.Hq, w.D)), w.q_dtype)


def _peak_rows(w: Workload, key, n: int) -> np.ndarray:
    return _rng(w.cid, 6, *key).random(n) < w.peak_fraction


def pool_f32(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Raw fp32 pool draws: K [NB][Hkv][bs][D], V [NB][Hkv][D][bs].

    With a peak fraction, each physical slot is picked independently with that probability and
    its K vector is multiplied by ``peak_factor`` in every KV head.
    """
    k = _normal(_rng(w.cid, 3), (w.NB, w.Hkv, w.bs, w.D))
    v = _normal(_rng(w.cid, 4), (w.NB, w.Hkv, w.D, w.bs))
    if w.peak_fraction > 0:
        m = _peak_rows(w, (0,), w.NB * w.bs).reshape(w.NB, w.bs)
        blk, slot = np.nonzero(m)
        k[blk, :, slot, :] *= np.float32(w.peak_factor)
    return k, v


def quantize_int8_pool(x: np.ndarray, tile_axes=(2, 3), qmax: int = 127
                       ) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric absmax codes with one fp32 scale per (block, head) tile.

    scale = absmax / qmax in fp32 (1.0 for an all-zero tile); code = clamp(rint(x / scale),
    -qmax, qmax) with fp32 division and round-half-to-even.  The absmax runs over every slot of
    the physical tile.  qmax = 127 gives int8 codes, 7 the int4 codes.  Returns (codes int8 same
    shape as x, scales fp32 [NB][Hkv]).
    """
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=tile_axes).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(qmax), np.float32(1.0)).astype(np.float32)
    s = np.expand_dims(scale, tile_axes)
    codes = np.clip(np.rint(x / s), -qmax, qmax).astype(np.int8)
    return codes, scale


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Device bytes of int4 codes in [-7, 7] along the last axis (n elements -> n/2 bytes):
    byte 4m + j holds element 8m + j in its low nibble and element 8m + j + 4 in its high
    nibble, each nibble being code + 8.  Applied to a K pool [NB][Hkv][bs][D] (rows of dims) or
    a V pool [NB][Hkv][D][bs] (rows of tokens)."""
    c = np.asarray(codes, np.int16) + 8
    n = c.shape[-1]
    out = np.zeros(c.shape[:-1] + (n // 2,), np.uint8)
    for m in range(n // 8):
        for j in range(4):
            out[..., 4 * m + j] = (c[..., 8 * m + j] | (c[..., 8 * m + j + 4] << 4)).astype(np.uint8)
    return out


def pool(w: Workload) -> dict:
    """Device-ready pool contents: {"k", "v"} in the cache dtype (+ "k_scale", "v_scale")."""
    k, v = pool_f32(w)
    if w.kv_dtype == KV_I8:
        kq, ks = quantize_int8_pool(k)
        vq, vs = quantize_int8_pool(v)
        return {"k": kq, "v": vq, "k_scale": ks, "v_scale": vs}
    if w.kv_dtype == KV_I4:
        kq, ks = quantize_int8_pool(k, qmax=7)
        vq, vs = quantize_int8_pool(v, qmax=7)
        return {"k": pack_int4(kq), "v": pack_int4(vq), "k_scale": ks, "v_scale": vs}
    return {"k": _cast(k, w.kv_dtype), "v": _cast(v, w.kv_dtype)}


def prompt_tokens(cid: int, request: int, n: int, vocab: int = 32000) -> np.ndarray:
    """Token ids of a synthetic prompt, int32 [n] (stream 7)."""
    return _rng(cid, 7, request).integers(0, vocab, n, dtype=np.int64).astype(np.int32)


def token_kv(cid: int, request: int, n: int, Hkv: int, D: int, dtype: str):
    """K and V [n][Hkv][D] of n tokens written by one request, in the cache dtype (stream 8)."""
    rng = _rng(cid, 8, request)
    k = _normal(rng, (n, Hkv, D))
    v = _normal(rng, (n, Hkv, D))
    return _cast(k, dtype), _cast(v, dtype)


def chunk_sizes(w: Workload, lo: int, hi: int) -> np.ndarray:
    """Chunked prefill: the number of new query tokens of each sequence, U{lo..hi} capped at its
    context length (stream 9)."""
    n = _rng(w.cid, 9).integers(lo, hi, size=w.B, endpoint=True).astype(np.int64)
    return np.minimum(n, w.lengths)


def chunk_queries(w: Workload, T: int) -> np.ndarray:
    """q [T][Hq][D] of a prefill chunk (stream 10): fp32 array or bf16 bits."""
    return _cast(_normal(_rng(w.cid, 10), (T, w.Hq, w.D)), w.q_dtype)


def new_tokens(w: Workload, step: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """The K and V vectors appended in a step: [B][Hkv][D] each, in the cache dtype."""
    if not w.append:
        raise ValueError(f"{w.name} has no append step")
    rng = _rng(w.cid, 5, step)
    k = _normal(rng, (w.B, w.Hkv, w.D))
    v = _normal(rng, (w.B, w.Hkv, w.D))
    if w.peak_fraction > 0:
        m = _peak_rows(w, (1, step), w.B)
        k[m] *= np.float32(w.peak_factor)
    return _cast(k, w.kv_dtype), _cast(v, w.kv_dtype)


POISON_BF16 = np.uint16(0x7FC0)   # quiet NaN
POISON_I8 = np.int8(-128)         # never produced by the symmetric quantiser
