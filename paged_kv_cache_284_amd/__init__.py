"""Python binding of libpagedkv (PagedAttention decode for MI355X).

Argument marshalling only: every computation runs in the C-ABI library (host allocator in C++,
device work in HIP kernels).  torch is used for device memory and streams; tensors are passed by
data pointer and the current HIP stream.  There is no fallback: if the library is not built,
every call raises.

    import paged_kv_cache_284_amd as pkv
    a = pkv.Allocator(num_blocks, 16, free_order)
    ...
    pkv.kv_append(k_new, v_new, slots, k_cache, v_cache)
    out = pkv.decode(q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale)

Layouts: k_cache [NB][Hkv][16][D], v_cache [NB][Hkv][D][16], scales [NB][Hkv] fp32,
q [B][Hq][D] (float32 or bfloat16), out [B][Hq][D] float32.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PA_OK, PA_ERR_INVALID, PA_ERR_OOM, PA_ERR_DEVICE, PA_ERR_UNSUPPORTED, PA_ERR_STATE = \
    0, -1, -2, -3, -4, -5
PA_ERR_TOO_LARGE = -6
DECODE_SCRATCH_BYTES = 16 << 20
PA_F32, PA_BF16, PA_I8, PA_I4 = 0, 1, 2, 3
BLOCK_SIZE = 16

_i32, _i64, _sz, _vp, _f32 = C.c_int32, C.c_int64, C.c_size_t, C.c_void_p, C.c_float
_pi32, _pi64 = C.POINTER(C.c_int32), C.POINTER(C.c_int64)

# name -> (restype, argtypes); kept in the order of include/pagedkv.h
_SIGNATURES = {
    "pa_status_string": (C.c_char_p, [C.c_int]),
    "pa_abi_version": (C.c_int, []),
    "pa_alloc_create": (C.c_int, [_i32, _i32, _pi32, C.POINTER(_vp)]),
    "pa_alloc_destroy": (None, [_vp]),
    "pa_seq_create": (C.c_int, [_vp, _pi32]),
    "pa_seq_fork": (C.c_int, [_vp, _i32, _i32, _pi32]),
    "pa_seq_append_slot": (C.c_int, [_vp, _i32, _pi64, _pi32, _pi32]),
    "pa_seq_reserve": (C.c_int, [_vp, _i32, _i32, _pi64, _pi32, _pi32]),
    "pa_step": (C.c_int, [_vp, _pi32, _i32, _pi64, _pi32, _pi32, _pi32, _pi32]),
    "pa_seq_free": (C.c_int, [_vp, _i32]),
    "pa_seq_len": (C.c_int, [_vp, _i32, _pi32]),
    "pa_seq_table": (C.c_int, [_vp, _i32, _pi32, _i32, _pi32]),
    "pa_export_block_tables": (C.c_int, [_vp, _pi32, _i32, _i32, _pi32, _pi32]),
    "pa_block_refcount": (C.c_int, [_vp, _i32, _pi32]),
    "pa_num_free": (C.c_int, [_vp, _pi32]),
    "pa_free_list": (C.c_int, [_vp, _pi32, _i32, _pi32]),
    "pa_seq_create_prefix": (C.c_int, [_vp, _pi32, _i32, C.c_uint64, _pi32, _pi32]),
    "pa_seq_add_tokens": (C.c_int, [_vp, _i32, _pi32, _i32]),
    "pa_num_evictable": (C.c_int, [_vp, _pi32]),
    "pa_alloc_set_swap": (C.c_int, [_vp, _i32]),
    "pa_seq_swap_out": (C.c_int, [_vp, _i32, _pi32, _i32, _pi32]),
    "pa_seq_swap_in": (C.c_int, [_vp, _i32, _pi32, _i32, _pi32]),
    "pa_num_free_swap": (C.c_int, [_vp, _pi32]),
    "pa_swap_blocks": (C.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                 _i32, _i32, _i32, _i32, _vp]),
    "pa_evictable_list": (C.c_int, [_vp, _pi32, _i32, _pi32]),
    "pa_block_hash": (C.c_int, [_vp, _i32, C.POINTER(C.c_uint64), _pi32]),
    "pa_kv_append": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_kv_append_int8": (C.c_int, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                    _i32, _i32, _vp]),
    "pa_kv_append_int4": (C.c_int, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                    _i32, _i32, _vp]),
    "pa_copy_blocks": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                 _vp]),
    "pa_update_block_tables": (C.c_int, [_vp, _i32, _vp, _vp, _i32, _i32, _vp]),
    "pa_append_step": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                 _i32, _i32, _i32, _i32, _vp]),
    "pa_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_prefill": (C.c_int, [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp,
                             _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp]),
    "pa_decode": (C.c_int, [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32,
                            _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_no_alloc": (C.c_int, [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp,
                                     _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp]),
    "pa_decode_shared_prefix_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_shared_prefix": (C.c_int, [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i32,
                                          _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                          _vp, _sz, _vp]),
}

_lib_handle = None


class PagedKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class OutOfBlocks(PagedKVError):
    pass


_host_only = False


def use_host_library(path: str) -> None:
    """Bind `path`, a build of the host allocator alone (no device entry points, e.g. the
    sanitized build of paged_kv_cache_284_amd.build.build_host_sanitized), instead of
    libpagedkv.so.  Only the symbols it exports are bound and torch is not imported; the device
    calls are then missing (an AttributeError).  Must come before the first lib() call."""
    global LIB_PATH, _host_only
    if _lib_handle is not None:
        raise RuntimeError("the library is already loaded")
    LIB_PATH = os.path.abspath(path)
    _host_only = True


def lib() -> C.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_284_amd.build`")
        if not _host_only:
            try:  # let torch bring in its HIP runtime first, so the process holds exactly one
                import torch  # noqa: F401
            except ImportError:
                pass
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            if _host_only and not hasattr(h, name):
                continue
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib_handle = h
    return _lib_handle


def status_string(status: int) -> str:
    return lib().pa_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != PA_OK:
        if status == PA_ERR_OOM:
            raise OutOfBlocks(status, what)
        raise PagedKVError(status, what)


def _i32_array(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(_pi32)


def _p64(a: np.ndarray):
    return a.ctypes.data_as(_pi64)


# ------------------------------------------------------------------------------------------
# host allocator
# ------------------------------------------------------------------------------------------
class Allocator:
    """Handle on the library's block allocator (FIFO free list, refcounts, copy-on-write)."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE,
                 free_order: Optional[Sequence[int]] = None):
        self._h = _vp()
        order = None if free_order is None else _i32_array(free_order)
        if order is not None and order.size != num_blocks:
            raise ValueError("free_order must list every block once")
        _check(lib().pa_alloc_create(num_blocks, block_size,
                                     None if order is None else _p32(order), C.byref(self._h)),
               "pa_alloc_create")
        self.num_blocks, self.block_size = num_blocks, block_size

    def close(self) -> None:
        if self._h:
            lib().pa_alloc_destroy(self._h)
            self._h = _vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def create(self) -> int:
        s = _i32()
        _check(lib().pa_seq_create(self._h, C.byref(s)), "pa_seq_create")
        return s.value

    def fork(self, parent: int, n_tokens: int) -> int:
        c = _i32()
        _check(lib().pa_seq_fork(self._h, parent, n_tokens, C.byref(c)), "pa_seq_fork")
        return c.value

    def append_slot(self, seq: int) -> Tuple[int, int, int]:
        slot, src, dst = _i64(), _i32(), _i32()
        _check(lib().pa_seq_append_slot(self._h, seq, C.byref(slot), C.byref(src), C.byref(dst)),
               "pa_seq_append_slot")
        return slot.value, src.value, dst.value

    def reserve(self, seq: int, n: int):
        slots = np.zeros(max(n, 1), np.int64)
        pairs = np.zeros((max(n, 1), 2), np.int32)
        k = _i32()
        _check(lib().pa_seq_reserve(self._h, seq, n, _p64(slots), _p32(pairs), C.byref(k)),
               "pa_seq_reserve")
        return slots[:n].tolist(), [tuple(p) for p in pairs[:k.value].tolist()]

    def step_arrays(self, seqs):
        """One append per listed sequence: (slots int64 [B], lengths after the append int32 [B],
        table_index int32 [B] (-1 = no table change), cow pairs int32 [n][2])."""
        s = _i32_array(seqs)
        B = s.size
        slots = np.zeros(max(B, 1), np.int64)
        lens = np.zeros(max(B, 1), np.int32)
        tidx = np.zeros(max(B, 1), np.int32)
        pairs = np.zeros((max(B, 1), 2), np.int32)
        k = _i32()
        _check(lib().pa_step(self._h, _p32(s), B, _p64(slots), _p32(lens), _p32(tidx), _p32(pairs),
                             C.byref(k)), "pa_step")
        return slots[:B], lens[:B], tidx[:B], pairs[:k.value]

    def step(self, seqs):
        slots, _, _, pairs = self.step_arrays(seqs)
        return slots.tolist(), [tuple(p) for p in pairs.tolist()]

    def release(self, seq: int) -> None:
        _check(lib().pa_seq_free(self._h, seq), "pa_seq_free")

    def length(self, seq: int) -> int:
        n = _i32()
        _check(lib().pa_seq_len(self._h, seq, C.byref(n)), "pa_seq_len")
        return n.value

    def table(self, seq: int) -> List[int]:
        n = _i32()
        _check(lib().pa_seq_table(self._h, seq, None, 0, C.byref(n)), "pa_seq_table")
        out = np.zeros(max(n.value, 1), np.int32)
        _check(lib().pa_seq_table(self._h, seq, _p32(out), n.value, C.byref(n)), "pa_seq_table")
        return out[:n.value].tolist()

    def export(self, seqs, max_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
        s = _i32_array(seqs)
        tables = np.zeros((s.size, max(max_blocks, 1)), np.int32)[:, :max_blocks].copy()
        lens = np.zeros(max(s.size, 1), np.int32)
        _check(lib().pa_export_block_tables(self._h, _p32(s), s.size, max_blocks,
                                            _p32(tables) if tables.size else None, _p32(lens)),
               "pa_export_block_tables")
        return tables, lens[:s.size]

    def refcount(self, block: int) -> int:
        rc = _i32()
        _check(lib().pa_block_refcount(self._h, block, C.byref(rc)), "pa_block_refcount")
        return rc.value

    def num_free(self) -> int:
        n = _i32()
        _check(lib().pa_num_free(self._h, C.byref(n)), "pa_num_free")
        return n.value

    def free_list(self) -> List[int]:
        n = _i32()
        _check(lib().pa_free_list(self._h, None, 0, C.byref(n)), "pa_free_list")
        out = np.zeros(max(n.value, 1), np.int32)
        _check(lib().pa_free_list(self._h, _p32(out), n.value, C.byref(n)), "pa_free_list")
        return out[:n.value].tolist()

    # -- preemption by swapping -----------------------------------------------------------------
    def set_swap(self, num_cpu_blocks: int) -> None:
        _check(lib().pa_alloc_set_swap(self._h, num_cpu_blocks), "pa_alloc_set_swap")

    def _swap(self, fn, name, seq):
        m = -(-self.length(seq) // self.block_size)    # the table's length
        n = _i32()
        out = np.zeros((max(m, 1), 2), np.int32)
        _check(fn(self._h, seq, _p32(out), m, C.byref(n)), name)
        return [tuple(p) for p in out[:n.value].tolist()]

    def swap_out(self, seq: int) -> List[Tuple[int, int]]:
        """(device block, swap block) pairs in table order; the device blocks are released."""
        return self._swap(lib().pa_seq_swap_out, "pa_seq_swap_out", seq)

    def swap_in(self, seq: int) -> List[Tuple[int, int]]:
        """(swap block, device block) pairs in table order."""
        return self._swap(lib().pa_seq_swap_in, "pa_seq_swap_in", seq)

    def num_free_swap(self) -> int:
        n = _i32()
        _check(lib().pa_num_free_swap(self._h, C.byref(n)), "pa_num_free_swap")
        return n.value

    # -- automatic prefix caching --------------------------------------------------------------
    def create_prefix(self, tokens, salt: int = 0) -> Tuple[int, int]:
        """A sequence for a prompt of token ids, reusing matching cached blocks: (id, tokens
        already cached)."""
        t = _i32_array(tokens)
        s, n = _i32(), _i32()
        _check(lib().pa_seq_create_prefix(self._h, _p32(t) if t.size else None, t.size,
                                          C.c_uint64(salt & (2**64 - 1)), C.byref(s),
                                          C.byref(n)), "pa_seq_create_prefix")
        return s.value, n.value

    def add_tokens(self, seq: int, tokens) -> None:
        t = _i32_array(tokens)
        _check(lib().pa_seq_add_tokens(self._h, seq, _p32(t) if t.size else None, t.size),
               "pa_seq_add_tokens")

    def num_evictable(self) -> int:
        n = _i32()
        _check(lib().pa_num_evictable(self._h, C.byref(n)), "pa_num_evictable")
        return n.value

    def evictable_list(self) -> List[int]:
        n = _i32()
        _check(lib().pa_evictable_list(self._h, None, 0, C.byref(n)), "pa_evictable_list")
        out = np.zeros(max(n.value, 1), np.int32)
        _check(lib().pa_evictable_list(self._h, _p32(out), n.value, C.byref(n)),
               "pa_evictable_list")
        return out[:n.value].tolist()

    def block_hash(self, block: int) -> Optional[int]:
        """The block's published hash, or None when it is not cached."""
        h, c = C.c_uint64(), _i32()
        _check(lib().pa_block_hash(self._h, block, C.byref(h), C.byref(c)), "pa_block_hash")
        return h.value if c.value else None


def run_script(alloc: Allocator, ops) -> dict:
    """Apply a set-up script of ("create"|"reserve"|"fork"|"free", ...) ops (see
    inputs.setup_script); returns the map from script names to sequence ids."""
    ids = {}
    for op in ops:
        if op[0] == "create":
            ids[op[1]] = alloc.create()
        elif op[0] == "reserve":
            alloc.reserve(ids[op[1]], op[2])
        elif op[0] == "fork":
            ids[op[3]] = alloc.fork(ids[op[1]], op[2])
        elif op[0] == "free":
            alloc.release(ids.pop(op[1]))
        else:
            raise ValueError(op)
    return ids


# ------------------------------------------------------------------------------------------
# device entry points (torch tensors in, nothing computed here)
# ------------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    """Element type code of a tensor: uint8 caches hold packed int4 codes (two per byte)."""
    torch = _torch()
    m = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.int8: PA_I8, torch.uint8: PA_I4}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _readable(t, name, dtype=None):
    """A device-readable array: a device tensor or a pinned host tensor."""
    if t is None:
        return None
    if not t.is_cuda and not t.is_pinned():
        raise ValueError(f"{name} must be a device tensor or pinned host memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """Write each sequence's new K/V [B][Hkv][D] at its slot (int64 [B], -1 skips)."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    B = k_new.shape[0]
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new/v_new must be [B][Hkv][D]")
    if tuple(v_cache.shape) != (NB, Hkv, D, bs) or tuple(slot_mapping.shape) != (B,):
        raise ValueError("v_cache must be [NB][Hkv][D][bs], slot_mapping [B]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("k_new, v_new, k_cache and v_cache must share one dtype")
    _check(lib().pa_kv_append(_dev(k_new, "k_new"), _dev(v_new, "v_new"),
                              _readable(slot_mapping, "slot_mapping", torch.int64),
                              _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), B, Hkv, D, bs,
                              NB, _dtype_code(k_cache), _stream(stream)), "pa_kv_append")


def kv_append_int8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                   stream=None) -> None:
    """Quantising append into an int8 cache: k_new/v_new [B][Hkv][D] bf16 or fp32."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    B = k_new.shape[0]
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new/v_new must be [B][Hkv][D]")
    if k_cache.dtype != torch.int8 or v_cache.dtype != torch.int8:
        raise TypeError("caches must be int8")
    if tuple(v_cache.shape) != (NB, Hkv, D, bs) or tuple(k_scale.shape) != (NB, Hkv):
        raise ValueError("v_cache must be [NB][Hkv][D][bs], scales [NB][Hkv]")
    if k_new.dtype != v_new.dtype:
        raise TypeError("k_new and v_new must share a dtype")
    _check(lib().pa_kv_append_int8(_dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                   _dtype_code(k_new),
                                   _readable(slot_mapping, "slot_mapping", torch.int64),
                                   _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                   _dev(k_scale, "k_scale", torch.float32),
                                   _dev(v_scale, "v_scale", torch.float32), B, Hkv, D, bs, NB,
                                   _stream(stream)), "pa_kv_append_int8")


def cache_geometry(k_cache, v_cache):
    """(NB, Hkv, bs, D) of a K/V pool pair, checking that the layouts agree; packed int4 pools
    (uint8) hold K [NB][Hkv][bs][D/2] and V [NB][Hkv][D][bs/2]."""
    NB, Hkv, bs, last = k_cache.shape
    packed = k_cache.dtype == _torch().uint8
    D = 2 * last if packed else last
    want_v = (NB, Hkv, D, bs // 2 if packed else bs)
    if tuple(v_cache.shape) != want_v or v_cache.dtype != k_cache.dtype:
        raise ValueError(f"v_cache must be {want_v} of {k_cache.dtype}")
    return NB, Hkv, bs, D


def kv_append_int4(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                   stream=None) -> None:
    """Quantising append into a packed int4 cache (uint8 pools): k_new/v_new [B][Hkv][D] bf16
    or fp32."""
    torch = _torch()
    if k_cache.dtype != torch.uint8:
        raise TypeError("int4 caches are uint8 (two codes per byte)")
    NB, Hkv, bs, D = cache_geometry(k_cache, v_cache)
    B = k_new.shape[0]
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new/v_new must be [B][Hkv][D]")
    if tuple(k_scale.shape) != (NB, Hkv) or k_new.dtype != v_new.dtype:
        raise ValueError("scales must be [NB][Hkv]; k_new and v_new share a dtype")
    _check(lib().pa_kv_append_int4(_dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                   _dtype_code(k_new),
                                   _readable(slot_mapping, "slot_mapping", torch.int64),
                                   _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                   _dev(k_scale, "k_scale", torch.float32),
                                   _dev(v_scale, "v_scale", torch.float32), B, Hkv, D, bs, NB,
                                   _stream(stream)), "pa_kv_append_int4")


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs, src_scales=(None, None),
                dst_scales=(None, None), stream=None) -> None:
    """Copy whole blocks between two pools of one layout (device and pinned host swap pool):
    dst block pairs[i][1] := src block pairs[i][0]."""
    torch = _torch()
    NBs, Hkv, bs, D = cache_geometry(src_k, src_v)
    NBd = dst_k.shape[0]
    n = pairs.shape[0]
    if tuple(dst_k.shape[1:]) != tuple(src_k.shape[1:]) or src_k.dtype != dst_k.dtype:
        raise ValueError("pools must share a layout and dtype")
    for t, nm in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v")):
        _readable(t, nm)
    sp = [_readable(x, "scale", torch.float32) for x in src_scales]
    dp = [_readable(x, "scale", torch.float32) for x in dst_scales]
    _check(lib().pa_swap_blocks(src_k.data_ptr(), src_v.data_ptr(), sp[0], sp[1], NBs,
                                dst_k.data_ptr(), dst_v.data_ptr(), dp[0], dp[1], NBd,
                                _readable(pairs, "pairs", torch.int32) if n else None, n, Hkv, D,
                                bs, _dtype_code(src_k), _stream(stream)), "pa_swap_blocks")


def copy_blocks(k_cache, v_cache, pairs, k_scale=None, v_scale=None, stream=None) -> None:
    """Copy whole blocks (K, V and int8 scales) for each (src, dst) row of pairs int32 [n][2]."""
    torch = _torch()
    NB, Hkv, bs, D = cache_geometry(k_cache, v_cache)
    n = pairs.shape[0]
    if n and tuple(pairs.shape) != (n, 2):
        raise ValueError("pairs must be [n][2]")
    _check(lib().pa_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                _dev(k_scale, "k_scale", torch.float32),
                                _dev(v_scale, "v_scale", torch.float32),
                                _readable(pairs, "pairs", torch.int32) if n else None, n, Hkv, D, bs,
                                NB, _dtype_code(k_cache), _stream(stream)), "pa_copy_blocks")


def update_block_tables(block_tables, slots, table_index, stream=None) -> None:
    """For every i with table_index[i] >= 0: block_tables[i][table_index[i]] = slots[i] // 16."""
    torch = _torch()
    B, MB = block_tables.shape
    if tuple(slots.shape) != (B,) or tuple(table_index.shape) != (B,):
        raise ValueError("slots and table_index must be [B]")
    _check(lib().pa_update_block_tables(_dev(block_tables, "block_tables", torch.int32), MB,
                                        _readable(slots, "slots", torch.int64),
                                        _readable(table_index, "table_index", torch.int32), B,
                                        BLOCK_SIZE, _stream(stream)), "pa_update_block_tables")


def append_step(k_new, v_new, slot_mapping, table_index, k_cache, v_cache, block_tables,
                seq_lens=None, seq_lens_out=None, stream=None) -> None:
    """kv_append, update_block_tables and (with seq_lens / seq_lens_out) a copy of the new
    lengths in one launch.  slot_mapping, table_index and seq_lens may be pinned host tensors."""
    torch = _torch()
    NB, Hkv, bs, D = k_cache.shape
    B = k_new.shape[0]
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new/v_new must be [B][Hkv][D]")
    if tuple(v_cache.shape) != (NB, Hkv, D, bs) or tuple(slot_mapping.shape) != (B,):
        raise ValueError("v_cache must be [NB][Hkv][D][bs], slot_mapping [B]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B][max_blocks]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("k_new, v_new, k_cache and v_cache must share one dtype")
    for t, n in ((table_index, "table_index"), (seq_lens, "seq_lens"), (seq_lens_out, "seq_lens_out")):
        if t is not None and tuple(t.shape) != (B,):
            raise ValueError(f"{n} must be [B]")
    _check(lib().pa_append_step(_dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                _readable(slot_mapping, "slot_mapping", torch.int64),
                                _readable(table_index, "table_index", torch.int32),
                                _readable(seq_lens, "seq_lens", torch.int32),
                                _dev(seq_lens_out, "seq_lens_out", torch.int32),
                                _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                _dev(block_tables, "block_tables", torch.int32),
                                block_tables.shape[1], B, Hkv, D, bs, NB, _dtype_code(k_cache),
                                _stream(stream)), "pa_append_step")


def decode_workspace_size(B: int, Hq: int, Hkv: int, D: int, max_seq_len: int,
                          partition_tokens: int = 0) -> int:
    return int(lib().pa_decode_workspace_size(B, Hq, Hkv, D, max_seq_len, partition_tokens))


def decode(q, k_cache, v_cache, block_tables, seq_lens, max_seq_len: int, scale: float,
           k_scale=None, v_scale=None, out=None, workspace=None, partition_tokens: int = 0,
           stream=None):
    """Paged decode attention; returns out [B][Hq][D] float32."""
    torch = _torch()
    B, Hq, D = q.shape
    NB, Hkv, bs, Dk = cache_geometry(k_cache, v_cache)
    if Dk != D:
        raise ValueError("cache shapes do not match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_tables must be [B][max_blocks] and seq_lens [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B][Hq][D]")
    need = decode_workspace_size(B, Hq, Hkv, D, max_seq_len, partition_tokens)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().pa_decode(_dev(out, "out", torch.float32), _dev(q, "q"), _dtype_code(q),
                           _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dtype_code(k_cache), _dev(k_scale, "k_scale", torch.float32),
                           _dev(v_scale, "v_scale", torch.float32),
                           _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
                           _dev(seq_lens, "seq_lens", torch.int32), max_seq_len, B, Hq, Hkv, D,
                           bs, NB, float(scale), partition_tokens, _dev(workspace, "workspace"),
                           workspace.numel() * workspace.element_size(), _stream(stream)),
           "pa_decode")
    return out


def decode_no_alloc(q, k_cache, v_cache, block_tables, seq_lens, max_seq_len: int, scale: float,
                    out, k_scale=None, v_scale=None, partition_tokens: int = 0, stream=None):
    """pa_decode_no_alloc: decode into the caller's ``out`` with the library's fixed device
    scratch instead of a workspace; allocates nothing."""
    B, Hq, D = q.shape
    NB, Hkv, bs, Dk = cache_geometry(k_cache, v_cache)
    if Dk != D:
        raise ValueError("cache shapes do not match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_tables must be [B][max_blocks] and seq_lens [B]")
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B][Hq][D]")
    torch = _torch()
    _check(lib().pa_decode_no_alloc(_dev(out, "out", torch.float32), _dev(q, "q"), _dtype_code(q),
                                    _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                    _dtype_code(k_cache), _dev(k_scale, "k_scale", torch.float32),
                                    _dev(v_scale, "v_scale", torch.float32),
                                    _dev(block_tables, "block_tables", torch.int32),
                                    block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32),
                                    max_seq_len, B, Hq, Hkv, D, bs, NB, float(scale),
                                    partition_tokens, _stream(stream)), "pa_decode_no_alloc")
    return out


def decode_shared_prefix_workspace_size(B: int, Hq: int, Hkv: int, D: int,
                                        max_seq_len: int) -> int:
    return int(lib().pa_decode_shared_prefix_workspace_size(B, Hq, Hkv, D, max_seq_len))


def decode_shared_prefix(q, k_cache, v_cache, block_tables, seq_lens, max_seq_len: int,
                         scale: float, k_scale=None, v_scale=None, out=None, workspace=None,
                         stream=None):
    """pa_decode_shared_prefix: decode that reads the blocks a run of adjacent sequences
    shares at the start of their tables once per group; returns out [B][Hq][D] float32."""
    torch = _torch()
    B, Hq, D = q.shape
    NB, Hkv, bs, Dk = cache_geometry(k_cache, v_cache)
    if Dk != D:
        raise ValueError("cache shapes do not match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_tables must be [B][max_blocks] and seq_lens [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [B][Hq][D]")
    if workspace is None:
        need = decode_shared_prefix_workspace_size(B, Hq, Hkv, D, max_seq_len)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().pa_decode_shared_prefix(
        _dev(out, "out", torch.float32), _dev(q, "q"), _dtype_code(q), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dtype_code(k_cache), _dev(k_scale, "k_scale", torch.float32),
        _dev(v_scale, "v_scale", torch.float32), _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32), max_seq_len, B, Hq, Hkv,
        D, bs, NB, float(scale), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)), "pa_decode_shared_prefix")
    return out


def prefill(q, k_cache, v_cache, block_tables, seq_lens, cu_q, max_seq_len: int, scale: float,
            k_scale=None, v_scale=None, out=None, stream=None):
    """Chunked-prefill attention: q [T][Hq][D] bf16 packed by cu_q [B+1]; each sequence's chunk
    is the last cu_q[b+1]-cu_q[b] of its seq_lens[b] cached tokens.  The cache is bf16, int8 or
    packed int4 (uint8 bytes; then k_scale / v_scale [NB][Hkv] float32).  Returns out [T][Hq][D]
    float32."""
    torch = _torch()
    T, Hq, D = q.shape
    NB, Hkv, bs, Dk = cache_geometry(k_cache, v_cache)
    B = seq_lens.shape[0]
    if Dk != D:
        raise ValueError("cache shapes do not match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or tuple(cu_q.shape) != (B + 1,):
        raise ValueError("block_tables must be [B][max_blocks] and cu_q [B+1]")
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    elif tuple(out.shape) != (T, Hq, D):
        raise ValueError("out must be [T][Hq][D]")
    _check(lib().pa_prefill(_dev(out, "out", torch.float32), _dev(q, "q"), _dtype_code(q),
                            _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                            _dtype_code(k_cache), _dev(k_scale, "k_scale", torch.float32),
                            _dev(v_scale, "v_scale", torch.float32),
                            _dev(block_tables, "block_tables", torch.int32),
                            block_tables.shape[1], _dev(seq_lens, "seq_lens", torch.int32),
                            _dev(cu_q, "cu_q", torch.int32), max_seq_len, B, T, Hq, Hkv, D, bs,
                            NB, float(scale), _stream(stream)), "pa_prefill")
    return out
