"""Paged KV-cache decode for AMD MI355X (gfx950): Python binding of ``libpa.so``.

This module marshals arguments only.  Every step of the path runs in the
library: the block pool (C++) and the HIP kernels.  PyTorch supplies device
memory and the stream; nothing here computes on tensors.  When ``libpa.so`` is
missing every call raises -- there is no fallback.

The names follow the C ABI of ``include/pa.h`` without its ``pa_`` prefix:
``reshape_and_cache``, ``copy_blocks``, ``paged_attention_decode``,
``paged_attention_prefill`` (chunked prefill), their INT8
cache forms ``reshape_and_cache_int8`` and ``paged_attention_decode_int8``, the pool
calls on :class:`Pool` (``alloc``, ``free``, ``incref``, ``fork``,
``free_table``, ``append_slots``, ``prefix_match``, ``prefix_register``,
``refcount``, ``num_free``, ``stats``), ``swap_blocks`` and
``transfer_blocks`` (the host tier) and ``blocks_for_bytes``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "BLOCK_SIZE", "PARTITION_NONE", "PARTITION_AUTO", "PAError", "load", "lib_path",
    "Pool", "BlockManager", "blocks_for_bytes", "reshape_and_cache", "copy_blocks",
    "paged_attention_decode", "paged_attention_decode_noalloc", "DECODE_SCRATCH_BYTES",
    "shared_prefix_groups", "paged_attention_decode_shared", "decode_step_shared",
    "decode_shared_workspace_bytes",
    "decode_workspace_bytes", "decode_auto_partition", "last_plan_partition",
    "reshape_and_cache_int8", "paged_attention_decode_int8", "paged_attention_decode_int8_shared",
    "decode_step_int8_shared",
    "swap_blocks", "transfer_blocks", "release_finished_transfers", "new_host_kv_cache",
    "paged_attention_prefill",
    "decode_step", "decode_step_int8",
    "new_kv_cache", "new_kv_cache_int8", "logical_view", "timing_begin", "timing_end", "timing_launches", "status_string",
]

BLOCK_SIZE = 16
DECODE_SCRATCH_BYTES = 128 << 20  # PA_DECODE_SCRATCH_BYTES
PARTITION_NONE = 0
PARTITION_AUTO = -1
KERNEL_KINDS = ("decode", "decode_reduce", "reshape_and_cache", "copy_blocks", "decode_plan",
                "transfer_blocks", "prefill")

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpa.so")
_lib = None

_c_i32, _c_i64, _c_sz, _c_p, _c_f = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                     ctypes.c_void_p, ctypes.c_float)
_P_I32 = ctypes.POINTER(ctypes.c_int32)
_P_I64 = ctypes.POINTER(ctypes.c_int64)


class _Stats(ctypes.Structure):
    _fields_ = [("num_blocks", _c_i32), ("num_free", _c_i32), ("num_used", _c_i32),
                ("num_shared", _c_i32), ("copies", _c_i64), ("num_cached", _c_i32),
                ("num_evictable", _c_i32), ("prefix_hits", _c_i64)]


_SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [_c_i32]),
    "pa_pool_create": (_c_i32, [_c_i32, _P_I32, ctypes.POINTER(_c_p)]),
    "pa_pool_destroy": (None, [_c_p]),
    "pa_alloc": (_c_i32, [_c_p, _P_I32]),
    "pa_incref": (_c_i32, [_c_p, _c_i32]),
    "pa_free": (_c_i32, [_c_p, _c_i32]),
    "pa_fork": (_c_i32, [_c_p, _P_I32, _c_i32]),
    "pa_free_table": (_c_i32, [_c_p, _P_I32, _c_i32]),
    "pa_append_slots": (_c_i32, [_c_p, _P_I32, _P_I32, _c_i32, _c_i32, _c_i32, _P_I64,
                                 _P_I32, _P_I32]),
    "pa_refcount": (_c_i32, [_c_p, _c_i32]),
    "pa_num_free": (_c_i32, [_c_p]),
    "pa_pool_stats": (_c_i32, [_c_p, ctypes.POINTER(_Stats)]),
    "pa_prefix_match": (_c_i32, [_c_p, _P_I32, _c_i32, _P_I32, _c_i32, _P_I32]),
    "pa_swap_blocks": (_c_i32, [_c_p, _c_p, _P_I32, _c_i32, _P_I64]),
    "pa_transfer_blocks": (_c_i32, [_c_p, _c_p, _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_i32, _c_i32,
                                    _c_i32, _c_i32, _c_p]),
    "pa_prefix_register": (_c_i32, [_c_p, _P_I32, _c_i32, _P_I32, _c_i32, _P_I32]),
    "pa_blocks_for_bytes": (_c_i64, [_c_i64, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_reshape_and_cache": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                      _c_i32, _c_i32, _c_p]),
    "pa_copy_blocks": (_c_i32, [_c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_p]),
    "pa_decode_workspace_bytes": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_decode_auto_partition": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_paged_attention_decode": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_f, _c_p, _c_i32,
                                           _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                           _c_p, _c_sz, _c_i32, _c_p]),
    "pa_paged_attention_decode_noalloc": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_f, _c_p,
                                                   _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                   _c_i32, _c_i32, _c_i32, _c_p]),
    "pa_shared_prefix_groups": (_c_i32, [_P_I32, _P_I32, _c_i32, _c_i32, _c_i32, _P_I32, _P_I32,
                                         _P_I32, _P_I32, _P_I32]),
    "pa_decode_shared_workspace_bytes": (_c_sz, [_c_i32] * 7),
    "pa_paged_attention_decode_shared": (_c_i32, [_c_p] * 8 + [_c_i32, _c_i32, _c_f, _c_p] +
                                         [_c_i32] * 7 + [_c_p, _c_sz, _c_i32, _c_p]),
    "pa_decode_step_shared": (_c_i32, [_c_p, _c_p, _c_p, _c_i32, _c_i32] + [_c_p] * 8 +
                              [_c_i32, _c_i32, _c_f, _c_p] + [_c_i32] * 7 +
                              [_c_p, _c_sz, _c_i32, _c_p]),
    "pa_paged_attention_decode_int8_shared": (_c_i32, [_c_p] * 10 + [_c_i32, _c_i32, _c_f, _c_p] +
                                              [_c_i32] * 7 + [_c_p, _c_sz, _c_i32, _c_p]),
    "pa_decode_step_int8_shared": (_c_i32, [_c_p] * 3 + [_c_i32] * 2 + [_c_p] * 10 +
                                   [_c_i32, _c_i32, _c_f, _c_p] + [_c_i32] * 7 +
                                   [_c_p, _c_sz, _c_i32, _c_p]),
    "pa_reshape_and_cache_int8": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32,
                                           _c_i32, _c_i32, _c_i32, _c_i32, _c_p]),
    "pa_paged_attention_decode_int8": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_f,
                                                _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                _c_i32, _c_i32, _c_p, _c_sz, _c_i32, _c_p]),
    "pa_paged_attention_prefill": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_f, _c_p,
                                            _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                            _c_i32, _c_p]),
    "pa_decode_step": (_c_i32, [_c_p, _c_p, _c_p, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_p,
                                _c_f, _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                _c_i32, _c_p, _c_sz, _c_i32, _c_p]),
    "pa_decode_step_int8": (_c_i32, [_c_p, _c_p, _c_p, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p,
                                     _c_p, _c_p, _c_p, _c_f, _c_p, _c_i32, _c_i32, _c_i32,
                                     _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_sz, _c_i32, _c_p]),
    "pa_timing_begin": (_c_i32, [_c_i32]),
    "pa_timing_end": (_c_i32, [ctypes.POINTER(ctypes.c_double), _P_I32]),
    "pa_timing_launches": (_c_i32, [_c_i32, ctypes.POINTER(ctypes.c_double), _c_i32, _P_I32]),
}

_STATUS = {0: "ok", -1: "invalid argument", -2: "out of blocks", -3: "bad block id",
           -4: "unsupported", -5: "device error", -6: "workspace too small",
           -7: "host memory allocation failed"}


class PAError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = int(status)
        super().__init__(f"{call}: {_STATUS.get(self.status, 'unknown status')} ({self.status})")


class OutOfBlocks(PAError):
    pass


def lib_path() -> str:
    return _LIB_PATH


def load():
    """The loaded library; raises if libpa.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m paged_kv_cache_06_amd._build`"
                " (hipcc, gfx950); there is no fallback path")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int, call: str) -> None:
    if status != 0:
        raise (OutOfBlocks if status == -2 else PAError)(status, call)


def status_string(status: int) -> str:
    return load().pa_status_string(status).decode()


# ---------------------------------------------------------------- host pool
def _i32p(a: np.ndarray):
    return a.ctypes.data_as(_P_I32)


class Pool:
    """Block pool of ``num_blocks`` ids (C++); see ``pa_pool_create``."""

    def __init__(self, num_blocks: int, free_order=None):
        lib = load()
        self._h = _c_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            if order.shape != (int(num_blocks),):
                raise ValueError("free_order must have num_blocks entries")
        _check(lib.pa_pool_create(int(num_blocks), None if order is None else _i32p(order),
                                  ctypes.byref(self._h)), "pa_pool_create")
        self.num_blocks = int(num_blocks)

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.pa_pool_destroy(self._h)
            self._h = None

    def alloc(self) -> int:
        b = _c_i32()
        _check(load().pa_alloc(self._h, ctypes.byref(b)), "pa_alloc")
        return b.value

    def incref(self, block: int) -> None:
        _check(load().pa_incref(self._h, int(block)), "pa_incref")

    def free(self, block: int) -> None:
        _check(load().pa_free(self._h, int(block)), "pa_free")

    def fork(self, table) -> None:
        t = np.ascontiguousarray(table, dtype=np.int32)
        _check(load().pa_fork(self._h, _i32p(t), t.size), "pa_fork")

    def free_table(self, table) -> None:
        t = np.ascontiguousarray(table, dtype=np.int32)
        _check(load().pa_free_table(self._h, _i32p(t), t.size), "pa_free_table")

    def append_slots(self, row: np.ndarray, nblocks: int, pos: int, n: int):
        """Slots of n tokens at pos.. of the sequence whose table is ``row``.

        ``row`` (int32, contiguous, capacity = len(row)) is updated in place.
        Returns (slots int64 [n], new nblocks, (src, dst) or None).
        """
        if row.dtype != np.int32 or not row.flags.c_contiguous:
            raise ValueError("row must be a contiguous int32 array")
        nb = _c_i32(int(nblocks))
        slots = np.empty(max(int(n), 1), dtype=np.int64)
        src, dst = _c_i32(), _c_i32()
        _check(load().pa_append_slots(self._h, _i32p(row), ctypes.byref(nb), row.size, int(pos),
                                      int(n), slots.ctypes.data_as(_P_I64), ctypes.byref(src),
                                      ctypes.byref(dst)), "pa_append_slots")
        cow = None if src.value < 0 else (src.value, dst.value)
        return slots[:int(n)], nb.value, cow

    def refcount(self, block: int) -> int:
        return int(load().pa_refcount(self._h, int(block)))

    def num_free(self) -> int:
        return int(load().pa_num_free(self._h))

    def stats(self) -> dict:
        st = _Stats()
        _check(load().pa_pool_stats(self._h, ctypes.byref(st)), "pa_pool_stats")
        return {"num_blocks": st.num_blocks, "free": st.num_free, "used": st.num_used,
                "shared": st.num_shared, "copies": st.copies, "cached": st.num_cached,
                "evictable": st.num_evictable, "prefix_hits": st.prefix_hits}

    def prefix_match(self, tokens, max_blocks: int | None = None) -> np.ndarray:
        """Cached blocks of the longest whole-block prefix of ``tokens`` (each
        gets one reference); int32 array in logical order."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        cap = t.size // BLOCK_SIZE if max_blocks is None else int(max_blocks)
        out = np.empty(max(cap, 1), dtype=np.int32)
        n = _c_i32()
        _check(load().pa_prefix_match(self._h, _i32p(t), t.size, _i32p(out), cap,
                                      ctypes.byref(n)), "pa_prefix_match")
        return out[:n.value]

    def prefix_register(self, table, tokens) -> int:
        """Enter the full blocks of a sequence (blocks ``table``, first tokens
        ``tokens``) in the prefix cache; returns how many were entered."""
        t = np.ascontiguousarray(table, dtype=np.int32)
        k = np.ascontiguousarray(tokens, dtype=np.int32)
        n = _c_i32()
        _check(load().pa_prefix_register(self._h, _i32p(t), t.size, _i32p(k), k.size,
                                         ctypes.byref(n)), "pa_prefix_register")
        return n.value


def swap_blocks(src: Pool, dst: Pool, blocks) -> np.ndarray:
    """Move ``blocks`` (held in ``src``) to ``dst`` (e.g. the device pool and a
    host pool): returns int64 [n, 2] (src block, dst block) pairs, the copies
    for :func:`transfer_blocks` and the new table entries."""
    b = np.ascontiguousarray(blocks, dtype=np.int32)
    pairs = np.empty((max(b.size, 1), 2), dtype=np.int64)
    _check(load().pa_swap_blocks(src._h, dst._h, _i32p(b), b.size,
                                 pairs.ctypes.data_as(_P_I64)), "pa_swap_blocks")
    return pairs[:b.size]


class BlockManager:
    """Per-sequence block tables on top of :class:`Pool` (host side of a step).

    Holds one int32 row of ``max_blocks`` entries per sequence; ``append``
    returns the new tokens' slots and any copy-on-write pair.
    """

    def __init__(self, pool: Pool, num_seqs: int, max_blocks: int, pad: int = 0):
        self.pool = pool
        self.rows = np.full((int(num_seqs), int(max_blocks)), int(pad), dtype=np.int32)
        self.nblocks = np.zeros(int(num_seqs), dtype=np.int32)
        self.lens = np.zeros(int(num_seqs), dtype=np.int64)

    def append(self, s: int, n: int):
        row = self.rows[s]
        slots, nb, cow = self.pool.append_slots(row, int(self.nblocks[s]), int(self.lens[s]), n)
        self.nblocks[s] = nb
        self.lens[s] += int(n)
        return slots, cow

    def match(self, s: int, tokens) -> int:
        """Start empty sequence ``s`` with the cached whole blocks of
        ``tokens``; returns the positions they cover."""
        if self.nblocks[s] != 0:
            raise ValueError("match target must be empty")
        got = self.pool.prefix_match(tokens, self.rows.shape[1])
        self.rows[s, :got.size] = got
        self.nblocks[s] = got.size
        self.lens[s] = got.size * BLOCK_SIZE
        return int(self.lens[s])

    def register(self, s: int, tokens) -> int:
        """Enter sequence ``s``'s full blocks, holding ``tokens``, in the cache."""
        return self.pool.prefix_register(self.rows[s, :int(self.nblocks[s])], tokens)

    def fork(self, dst: int, src: int) -> None:
        if self.nblocks[dst] != 0:
            raise ValueError("fork target must be empty")
        nb = int(self.nblocks[src])
        self.pool.fork(self.rows[src, :nb])
        self.rows[dst, :nb] = self.rows[src, :nb]
        self.nblocks[dst] = nb
        self.lens[dst] = self.lens[src]

    def release(self, s: int, pad: int = 0) -> None:
        nb = int(self.nblocks[s])
        self.pool.free_table(self.rows[s, :nb])
        self.rows[s, :] = pad
        self.nblocks[s] = 0
        self.lens[s] = 0

    def table(self, s: int) -> list:
        return self.rows[s, :int(self.nblocks[s])].tolist()


def blocks_for_bytes(nbytes: int, num_layers: int, num_kv_heads: int, head_dim: int,
                     elem_bytes: int) -> int:
    return int(load().pa_blocks_for_bytes(int(nbytes), int(num_layers), int(num_kv_heads),
                                          int(head_dim), int(elem_bytes)))


# ------------------------------------------------------------- device calls
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.int8: 3}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def new_kv_cache(num_blocks: int, num_kv_heads: int, head_dim: int, dtype, device="cuda",
                 fill: float | None = None):
    """(k_cache, v_cache) tensors in the library's layout (see include/pa.h)."""
    torch = _torch()
    x = 16 // torch.tensor([], dtype=dtype).element_size()
    _need(head_dim % x == 0, "head_dim must be a multiple of 16 bytes")
    kshape = (num_blocks, num_kv_heads, head_dim // x, BLOCK_SIZE, x)
    vshape = (num_blocks, num_kv_heads, head_dim, BLOCK_SIZE)
    if fill is None:
        return (torch.empty(kshape, dtype=dtype, device=device),
                torch.empty(vshape, dtype=dtype, device=device))
    return (torch.full(kshape, fill, dtype=dtype, device=device),
            torch.full(vshape, fill, dtype=dtype, device=device))


def new_kv_cache_int8(num_blocks: int, num_kv_heads: int, head_dim: int, device="cuda",
                      fill: int | None = None):
    """(k_cache, v_cache) int8 tensors of an INT8 cache: [NB, Hkv, D/64, 1024],
    one KiB slab of 64 dimensions x 16 tokens per row (layout in include/pa.h)."""
    torch = _torch()
    _need(head_dim % 64 == 0, "head_dim must be a multiple of 64")
    shape = (num_blocks, num_kv_heads, head_dim // 64, 1024)
    if fill is None:
        return (torch.empty(shape, dtype=torch.int8, device=device),
                torch.empty(shape, dtype=torch.int8, device=device))
    return (torch.full(shape, fill, dtype=torch.int8, device=device),
            torch.full(shape, fill, dtype=torch.int8, device=device))


def logical_view(k_cache, v_cache):
    """The caches as [num_blocks, Hkv, 16, head_dim] copies (for inspection)."""
    torch = _torch()
    if k_cache.dtype == torch.int8:
        nb, hkv, slabs, _ = k_cache.shape
        # K slab: [chunk of 16 dims][token][dim % 16]
        k = k_cache.reshape(nb, hkv, slabs, 4, 16, 16).permute(0, 1, 4, 2, 3, 5)
        # V slab: [token / 4][dim % 16][16-dim slice][token % 4]
        v = v_cache.reshape(nb, hkv, slabs, 4, 16, 4, 4).permute(0, 1, 3, 6, 2, 5, 4)
        return (k.reshape(nb, hkv, 16, slabs * 64).contiguous(),
                v.reshape(nb, hkv, 16, slabs * 64).contiguous())
    nb, hkv, dx, bs, x = k_cache.shape
    k = k_cache.permute(0, 1, 3, 2, 4).reshape(nb, hkv, bs, dx * x)
    v = v_cache.permute(0, 1, 3, 2)
    return k.contiguous(), v.contiguous()


def _cache_dims(k_cache, v_cache):
    torch = _torch()
    if k_cache.dtype == torch.int8:
        _need(k_cache.dim() == 4 and k_cache.shape[3] == 1024 and
              tuple(v_cache.shape) == tuple(k_cache.shape) and v_cache.dtype == torch.int8,
              "INT8 caches must both be int8 [NB, Hkv, D/64, 1024]")
        _need(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")
        nb, hkv, slabs, _ = k_cache.shape
        return nb, hkv, slabs * 64
    _need(k_cache.dim() == 5 and v_cache.dim() == 4, "caches must be [NB,Hkv,D/X,16,X] and "
          "[NB,Hkv,D,16]")
    nb, hkv, dx, bs, x = k_cache.shape
    d = dx * x
    _need(bs == BLOCK_SIZE and tuple(v_cache.shape) == (nb, hkv, d, BLOCK_SIZE),
          "k_cache / v_cache shapes disagree")
    _need(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")
    _need(k_cache.dtype == v_cache.dtype, "caches must share a dtype")
    return nb, hkv, d


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping) -> None:
    """Write key/value [T, Hkv, D] of new tokens into their slots (int64 [T])."""
    torch = _torch()
    nb, hkv, d = _cache_dims(k_cache, v_cache)
    t = key.shape[0]
    _need(tuple(key.shape) == (t, hkv, d) and tuple(value.shape) == (t, hkv, d),
          "key/value must be [T, Hkv, D]")
    _need(key.is_contiguous() and value.is_contiguous(), "key/value must be contiguous")
    _need(key.dtype == k_cache.dtype == value.dtype, "dtypes differ")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == t,
          "slot_mapping must be int64 [T]")
    _check(load().pa_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(slot_mapping.contiguous()), t, nb, hkv, d,
                                       _dtype_code(key), _stream(key)), "pa_reshape_and_cache")


def copy_blocks(k_cache, v_cache, block_pairs) -> None:
    """Copy whole blocks: block_pairs is int64 [n, 2] of (src, dst) on the device."""
    torch = _torch()
    nb, hkv, d = _cache_dims(k_cache, v_cache)
    _need(block_pairs.dtype == torch.int64 and block_pairs.dim() == 2 and
          block_pairs.shape[1] == 2, "block_pairs must be int64 [n, 2]")
    n = block_pairs.shape[0]
    _check(load().pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_pairs.contiguous()), n,
                                 nb, hkv, d, _dtype_code(k_cache), _stream(k_cache)),
           "pa_copy_blocks")


def _scales(scale, hkv, d, name):
    torch = _torch()
    _need(scale.dtype == torch.float32 and tuple(scale.shape) == (hkv, d) and
          scale.is_contiguous(), f"{name} must be contiguous float32 [Hkv, D]")
    return _ptr(scale)


def reshape_and_cache_int8(key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale) -> None:
    """Quantize key/value [T, Hkv, D] (fp32/fp16/bf16) with per-channel scales
    k_scale / v_scale (float32 [Hkv, D]) and write the codes into their slots."""
    torch = _torch()
    _need(k_cache.dtype == torch.int8, "INT8 caches expected")
    nb, hkv, d = _cache_dims(k_cache, v_cache)
    t = key.shape[0]
    _need(tuple(key.shape) == (t, hkv, d) and tuple(value.shape) == (t, hkv, d),
          "key/value must be [T, Hkv, D]")
    _need(key.is_contiguous() and value.is_contiguous(), "key/value must be contiguous")
    _need(key.dtype == value.dtype, "key/value dtypes differ")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == t,
          "slot_mapping must be int64 [T]")
    _check(load().pa_reshape_and_cache_int8(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping.contiguous()),
        _scales(k_scale, hkv, d, "k_scale"), _scales(v_scale, hkv, d, "v_scale"), t, nb, hkv, d,
        _dtype_code(key), _stream(key)), "pa_reshape_and_cache_int8")


def new_host_kv_cache(num_blocks: int, num_kv_heads: int, head_dim: int, dtype):
    """(k_cache, v_cache) in pinned host memory, laid out like the device caches
    (int8 dtype: the INT8 layout), for blocks moved out of the device pool."""
    torch = _torch()
    if dtype == torch.int8:
        shape = (num_blocks, num_kv_heads, head_dim // 64, 1024)
        return (torch.empty(shape, dtype=dtype, pin_memory=True),
                torch.empty(shape, dtype=dtype, pin_memory=True))
    x = 16 // torch.tensor([], dtype=dtype).element_size()
    kshape = (num_blocks, num_kv_heads, head_dim // x, BLOCK_SIZE, x)
    vshape = (num_blocks, num_kv_heads, head_dim, BLOCK_SIZE)
    return (torch.empty(kshape, dtype=dtype, pin_memory=True),
            torch.empty(vshape, dtype=dtype, pin_memory=True))


# Host tensors read by an enqueued transfer, kept alive (with an event
# recorded after the launch) until the stream has passed it: torch's pinned
# allocator would otherwise hand a freed pinned buffer to the next
# pin_memory() while the transfer still reads it.
_host_inflight: list = []


def release_finished_transfers() -> int:
    """Drop the references transfer_blocks keeps to host tensors whose copies
    the device has finished (each call of transfer_blocks does this too);
    returns how many copies still hold host tensors."""
    _host_inflight[:] = [(e, ts) for e, ts in _host_inflight if not e.query()]
    return len(_host_inflight)


def _keep_host_alive(tensors, stream) -> None:
    torch = _torch()
    release_finished_transfers()
    host = [t for t in tensors if not t.is_cuda]
    if host:
        ev = torch.cuda.Event()
        ev.record(stream)
        _host_inflight.append((ev, host))


def transfer_blocks(src_k, src_v, dst_k, dst_v, block_pairs) -> None:
    """Copy blocks between two caches of one shape (device or pinned host):
    block_pairs int64 [n, 2] of (src, dst), on the device or pinned.  The copy
    is enqueued on the current stream; host tensors among the arguments are
    kept alive until the stream has passed it."""
    torch = _torch()
    nbs, hkv, d = _cache_dims(src_k, src_v)
    nbd, hkv2, d2 = _cache_dims(dst_k, dst_v)
    _need((hkv, d) == (hkv2, d2) and src_k.dtype == dst_k.dtype, "caches differ in shape")
    for t in (src_k, src_v, dst_k, dst_v):
        _need(t.is_cuda or t.is_pinned(), "host caches must be pinned")
    _need(block_pairs.dtype == torch.int64 and block_pairs.dim() == 2 and
          block_pairs.shape[1] == 2 and block_pairs.is_contiguous() and
          (block_pairs.is_cuda or block_pairs.is_pinned()),
          "block_pairs must be contiguous int64 [n, 2], on the device or pinned")
    dev = next(t for t in (src_k, dst_k, block_pairs) if t.is_cuda) \
        if any(t.is_cuda for t in (src_k, dst_k, block_pairs)) else None
    cur = torch.cuda.current_stream(dev)
    stream = ctypes.c_void_p(cur.cuda_stream)
    _check(load().pa_transfer_blocks(_ptr(src_k), _ptr(src_v), nbs, _ptr(dst_k), _ptr(dst_v), nbd,
                                     _ptr(block_pairs), block_pairs.shape[0], hkv, d,
                                     _dtype_code(src_k), stream), "pa_transfer_blocks")
    _keep_host_alive((src_k, src_v, dst_k, dst_v, block_pairs), cur)


def decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
                           partition_size=PARTITION_AUTO) -> int:
    return int(load().pa_decode_workspace_bytes(int(num_seqs), int(num_q_heads), int(head_dim),
                                                int(max_context_len), int(partition_size)))


def decode_auto_partition(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                          dtype_code) -> int:
    return int(load().pa_decode_auto_partition(int(num_seqs), int(num_q_heads),
                                               int(num_kv_heads), int(head_dim),
                                               int(max_context_len), int(dtype_code)))


_workspaces = {}


def paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, *,
                           max_context_len: int | None = None,
                           partition_size: int = PARTITION_AUTO, workspace=None) -> None:
    """out[s, h] = softmax(scale * q[s, h] . K_s) V_s over the paged cache.

    q, out: [S, Hq, D]; block_tables int32 [S, MB]; context_lens int32 [S].
    ``max_context_len`` defaults to 16 * MB (an upper bound that needs no sync).
    ``workspace`` (uint8 device tensor) is allocated and kept per device when
    not given; calls sharing a workspace must not overlap.
    """
    torch = _torch()
    nb, hkv, d = _cache_dims(k_cache, v_cache)
    s, hq, dq = q.shape
    _need(dq == d and tuple(out.shape) == (s, hq, d), "q/out must be [S, Hq, D]")
    _need(q.is_contiguous() and out.is_contiguous(), "q/out must be contiguous")
    _need(q.dtype == out.dtype == k_cache.dtype, "dtypes differ")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == s and block_tables.is_contiguous(),
          "block_tables must be contiguous int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == s,
          "context_lens must be int32 [S]")
    mb = block_tables.shape[1]
    mcl = mb * BLOCK_SIZE if max_context_len is None else int(max_context_len)
    ws_ptr, ws_bytes = _workspace(q, s, hq, d, mcl, partition_size, workspace)
    _check(load().pa_paged_attention_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens.contiguous()),
        float(scale), _ptr(out), s, hq, hkv, d, mb, mcl, int(partition_size), ws_ptr, ws_bytes,
        _dtype_code(q), _stream(q)), "pa_paged_attention_decode")


def paged_attention_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                                   *, max_context_len: int | None = None,
                                   partition_size: int = PARTITION_AUTO) -> None:
    """paged_attention_decode with its workspace in the library's per-device
    scratch array (``pa_paged_attention_decode_noalloc``): no device memory is
    allocated by the call.  Calls that overlap on one device race."""
    torch = _torch()
    nb, hkv, d = _cache_dims(k_cache, v_cache)
    s, hq, dq = q.shape
    _need(dq == d and tuple(out.shape) == (s, hq, d), "q/out must be [S, Hq, D]")
    _need(q.is_contiguous() and out.is_contiguous(), "q/out must be contiguous")
    _need(q.dtype == out.dtype == k_cache.dtype, "dtypes differ")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == s and block_tables.is_contiguous(),
          "block_tables must be contiguous int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == s and
          context_lens.is_contiguous(), "context_lens must be contiguous int32 [S]")
    mb = block_tables.shape[1]
    mcl = mb * BLOCK_SIZE if max_context_len is None else int(max_context_len)
    _check(load().pa_paged_attention_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), _ptr(out), s, hq, hkv, d, mb, mcl, int(partition_size), _dtype_code(q),
        _stream(q)), "pa_paged_attention_decode_noalloc")


def decode_step(key, value, slot_mapping, q, k_cache, v_cache, block_tables, context_lens, scale,
                out, *, max_context_len: int | None = None, partition_size: int = PARTITION_AUTO,
                workspace=None) -> None:
    """reshape_and_cache(key, value, ..., slot_mapping) then paged_attention_decode,
    in fewer launches where the library can."""
    torch = _torch()
    nb, hkv, d = _cache_dims(k_cache, v_cache)
    t = key.shape[0]
    _need(tuple(key.shape) == (t, hkv, d) and tuple(value.shape) == (t, hkv, d),
          "key/value must be [T, Hkv, D]")
    _need(key.is_contiguous() and value.is_contiguous(), "key/value must be contiguous")
    _need(key.dtype == k_cache.dtype == value.dtype, "dtypes differ")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == t,
          "slot_mapping must be int64 [T]")
    s, hq, dq = q.shape
    _need(dq == d and tuple(out.shape) == (s, hq, d), "q/out must be [S, Hq, D]")
    _need(q.is_contiguous() and out.is_contiguous(), "q/out must be contiguous")
    _need(q.dtype == out.dtype == k_cache.dtype, "dtypes differ")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == s and block_tables.is_contiguous(),
          "block_tables must be contiguous int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == s,
          "context_lens must be int32 [S]")
    mb = block_tables.shape[1]
    mcl = mb * BLOCK_SIZE if max_context_len is None else int(max_context_len)
    ws_ptr, ws_bytes = _workspace(q, s, hq, d, mcl, partition_size, workspace)
    _check(load().pa_decode_step(
        _ptr(key), _ptr(value), _ptr(slot_mapping.contiguous()), t, nb, _ptr(q), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_tables), _ptr(context_lens.contiguous()), float(scale),
        _ptr(out), s, hq, hkv, d, mb, mcl, int(partition_size), ws_ptr, ws_bytes,
        _dtype_code(q), _stream(q)), "pa_decode_step")


def shared_prefix_groups(rows, nblocks, min_blocks: int = 1):
    """Groups of sequences whose tables begin with the same blocks
    (``pa_shared_prefix_groups``): rows int32 [S, MB] and nblocks [S] on the
    host.  Returns (prefix_seqs, prefix_start, prefix_blocks) int32 arrays."""
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    nb = np.ascontiguousarray(nblocks, dtype=np.int32)
    s, mb = rows.shape
    _need(nb.shape == (s,), "nblocks must have one entry per row")
    seqs = np.zeros(max(s, 1), np.int32)
    start = np.zeros(s // 2 + 1, np.int32)
    blocks = np.zeros(max(s // 2, 1), np.int32)
    ng, nm = _c_i32(), _c_i32()
    _check(load().pa_shared_prefix_groups(_i32p(rows), _i32p(nb), s, max(mb, 1), int(min_blocks),
                                          _i32p(seqs), _i32p(start), _i32p(blocks),
                                          ctypes.byref(ng), ctypes.byref(nm)),
           "pa_shared_prefix_groups")
    return seqs[:nm.value].copy(), start[:ng.value + 1].copy(), blocks[:ng.value].copy()


def decode_shared_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
                                  partition_size, num_groups, num_members) -> int:
    return int(load().pa_decode_shared_workspace_bytes(
        int(num_seqs), int(num_q_heads), int(head_dim), int(max_context_len),
        int(partition_size), int(num_groups), int(num_members)))


def _shared_args(prefix_seqs, prefix_start, prefix_blocks):
    torch = _torch()
    for t, name in ((prefix_seqs, "prefix_seqs"), (prefix_start, "prefix_start"),
                    (prefix_blocks, "prefix_blocks")):
        _need(t.dtype == torch.int32 and t.dim() == 1 and t.is_contiguous(),
              f"{name} must be a contiguous int32 vector")
    ng = prefix_blocks.numel()
    _need(prefix_start.numel() == ng + 1, "prefix_start must have num_groups + 1 entries")
    return ng, prefix_seqs.numel()


def paged_attention_decode_shared(q, k_cache, v_cache, block_tables, context_lens, prefix_seqs,
                                  prefix_start, prefix_blocks, scale, out, *,
                                  max_context_len: int | None = None,
                                  partition_size: int = PARTITION_AUTO, workspace=None) -> None:
    """paged_attention_decode reading each group's shared leading blocks once
    (``pa_paged_attention_decode_shared``); prefix_* are device int32 vectors
    as ``shared_prefix_groups`` gives them."""
    torch = _torch()
    nb, hkv, d = _cache_dims(k_cache, v_cache)
    s, hq, dq = q.shape
    _need(dq == d and tuple(out.shape) == (s, hq, d), "q/out must be [S, Hq, D]")
    _need(q.is_contiguous() and out.is_contiguous(), "q/out must be contiguous")
    _need(q.dtype == out.dtype == k_cache.dtype, "dtypes differ")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == s and block_tables.is_contiguous(),
          "block_tables must be contiguous int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == s and
          context_lens.is_contiguous(), "context_lens must be contiguous int32 [S]")
    ng, nm = _shared_args(prefix_seqs, prefix_start, prefix_blocks)
    mb = block_tables.shape[1]
    mcl = mb * BLOCK_SIZE if max_context_len is None else int(max_context_len)
    ws_ptr, ws_bytes = _workspace(q, s, hq, d, mcl, partition_size, workspace,
                                  decode_shared_workspace_bytes(s, hq, d, mcl, partition_size, ng,
                                                                nm))
    _check(load().pa_paged_attention_decode_shared(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(prefix_seqs), _ptr(prefix_start), _ptr(prefix_blocks), ng, nm, float(scale),
        _ptr(out), s, hq, hkv, d, mb, mcl, int(partition_size), ws_ptr, ws_bytes, _dtype_code(q),
        _stream(q)), "pa_paged_attention_decode_shared")


def decode_step_shared(key, value, slot_mapping, q, k_cache, v_cache, block_tables, context_lens,
                       prefix_seqs, prefix_start, prefix_blocks, scale, out, *,
                       max_context_len: int | None = None, partition_size: int = PARTITION_AUTO,
                       workspace=None) -> None:
    """decode_step with shared prefixes (``pa_decode_step_shared``)."""
    torch = _torch()
    nb, hkv, d = _cache_dims(k_cache, v_cache)
    t = key.shape[0]
    _need(tuple(key.shape) == (t, hkv, d) and tuple(value.shape) == (t, hkv, d),
          "key/value must be [T, Hkv, D]")
    _need(key.is_contiguous() and value.is_contiguous(), "key/value must be contiguous")
    _need(key.dtype == k_cache.dtype == value.dtype, "dtypes differ")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == t and
          slot_mapping.is_contiguous(), "slot_mapping must be contiguous int64 [T]")
    s, hq, dq = q.shape
    _need(dq == d and tuple(out.shape) == (s, hq, d), "q/out must be [S, Hq, D]")
    _need(q.is_contiguous() and out.is_contiguous(), "q/out must be contiguous")
    _need(q.dtype == out.dtype == k_cache.dtype, "dtypes differ")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == s and block_tables.is_contiguous(),
          "block_tables must be contiguous int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == s and
          context_lens.is_contiguous(), "context_lens must be contiguous int32 [S]")
    ng, nm = _shared_args(prefix_seqs, prefix_start, prefix_blocks)
    mb = block_tables.shape[1]
    mcl = mb * BLOCK_SIZE if max_context_len is None else int(max_context_len)
    ws_ptr, ws_bytes = _workspace(q, s, hq, d, mcl, partition_size, workspace,
                                  decode_shared_workspace_bytes(s, hq, d, mcl, partition_size, ng,
                                                                nm))
    _check(load().pa_decode_step_shared(
        _ptr(key), _ptr(value), _ptr(slot_mapping), t, nb, _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_tables), _ptr(context_lens), _ptr(prefix_seqs), _ptr(prefix_start),
        _ptr(prefix_blocks), ng, nm, float(scale), _ptr(out), s, hq, hkv, d, mb, mcl,
        int(partition_size), ws_ptr, ws_bytes, _dtype_code(q), _stream(q)),
        "pa_decode_step_shared")


def last_plan_partition() -> int:
    """The partition size the last decode through a workspace of this module
    planned with (word 2 of the plan's header in that workspace): the given
    or automatic one, or the automatic one doubled by the plan for an even
    batch.  0 if no decode has run."""
    torch = _torch()
    if not _workspaces:
        return 0
    ws = next(iter(_workspaces.values()))
    torch.cuda.synchronize(ws.device)
    return int(ws[:12].view(torch.int32)[2].item())


def _workspace(q, s, hq, d, mcl, partition_size, workspace, need=None):
    torch = _torch()
    if need is None:
        need = decode_workspace_bytes(s, hq, d, mcl, partition_size)
    if workspace is None and need > 0:
        key = (q.device, need)
        workspace = _workspaces.get(key)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            _workspaces.clear()
            _workspaces[key] = workspace
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return ws_ptr, ws_bytes


def decode_step_int8(key, value, slot_mapping, q, k_cache, v_cache, k_scale, v_scale,
                     block_tables, context_lens, scale, out, *, max_context_len: int | None = None,
                     partition_size: int = PARTITION_AUTO, workspace=None) -> None:
    """reshape_and_cache_int8 then paged_attention_decode_int8 in fewer launches."""
    torch = _torch()
    _need(k_cache.dtype == torch.int8, "INT8 caches expected")
    nb, hkv, d = _cache_dims(k_cache, v_cache)
    t = key.shape[0]
    _need(tuple(key.shape) == (t, hkv, d) and tuple(value.shape) == (t, hkv, d),
          "key/value must be [T, Hkv, D]")
    _need(key.is_contiguous() and value.is_contiguous(), "key/value must be contiguous")
    _need(key.dtype == value.dtype == q.dtype, "key/value/q dtypes differ")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == t,
          "slot_mapping must be int64 [T]")
    s, hq, dq = q.shape
    _need(dq == d and tuple(out.shape) == (s, hq, d), "q/out must be [S, Hq, D]")
    _need(q.is_contiguous() and out.is_contiguous() and q.dtype == out.dtype,
          "q/out must be contiguous, of one dtype")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == s and block_tables.is_contiguous(),
          "block_tables must be contiguous int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == s,
          "context_lens must be int32 [S]")
    mb = block_tables.shape[1]
    mcl = mb * BLOCK_SIZE if max_context_len is None else int(max_context_len)
    ws_ptr, ws_bytes = _workspace(q, s, hq, d, mcl, partition_size, workspace)
    _check(load().pa_decode_step_int8(
        _ptr(key), _ptr(value), _ptr(slot_mapping.contiguous()), t, nb, _ptr(q), _ptr(k_cache),
        _ptr(v_cache), _scales(k_scale, hkv, d, "k_scale"), _scales(v_scale, hkv, d, "v_scale"),
        _ptr(block_tables), _ptr(context_lens.contiguous()), float(scale), _ptr(out), s, hq, hkv,
        d, mb, mcl, int(partition_size), ws_ptr, ws_bytes, _dtype_code(q), _stream(q)),
        "pa_decode_step_int8")


def _int8_decode_args(q, k_cache, v_cache, block_tables, context_lens, out, max_context_len):
    torch = _torch()
    _need(k_cache.dtype == torch.int8, "INT8 caches expected")
    nb, hkv, d = _cache_dims(k_cache, v_cache)
    s, hq, dq = q.shape
    _need(dq == d and tuple(out.shape) == (s, hq, d), "q/out must be [S, Hq, D]")
    _need(q.is_contiguous() and out.is_contiguous(), "q/out must be contiguous")
    _need(q.dtype == out.dtype, "q/out dtypes differ")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == s and block_tables.is_contiguous(),
          "block_tables must be contiguous int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == s and
          context_lens.is_contiguous(), "context_lens must be contiguous int32 [S]")
    mb = block_tables.shape[1]
    mcl = mb * BLOCK_SIZE if max_context_len is None else int(max_context_len)
    return nb, hkv, d, s, hq, mb, mcl


def paged_attention_decode_int8_shared(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                       context_lens, prefix_seqs, prefix_start, prefix_blocks,
                                       scale, out, *, max_context_len: int | None = None,
                                       partition_size: int = PARTITION_AUTO,
                                       workspace=None) -> None:
    """paged_attention_decode_int8 reading each group's shared leading blocks
    once (``pa_paged_attention_decode_int8_shared``); prefix_* as for
    ``paged_attention_decode_shared``."""
    nb, hkv, d, s, hq, mb, mcl = _int8_decode_args(q, k_cache, v_cache, block_tables,
                                                   context_lens, out, max_context_len)
    ng, nm = _shared_args(prefix_seqs, prefix_start, prefix_blocks)
    ws_ptr, ws_bytes = _workspace(q, s, hq, d, mcl, partition_size, workspace,
                                  decode_shared_workspace_bytes(s, hq, d, mcl, partition_size, ng,
                                                                nm))
    _check(load().pa_paged_attention_decode_int8_shared(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _scales(k_scale, hkv, d, "k_scale"),
        _scales(v_scale, hkv, d, "v_scale"), _ptr(block_tables), _ptr(context_lens),
        _ptr(prefix_seqs), _ptr(prefix_start), _ptr(prefix_blocks), ng, nm, float(scale),
        _ptr(out), s, hq, hkv, d, mb, mcl, int(partition_size), ws_ptr, ws_bytes, _dtype_code(q),
        _stream(q)), "pa_paged_attention_decode_int8_shared")


def decode_step_int8_shared(key, value, slot_mapping, q, k_cache, v_cache, k_scale, v_scale,
                            block_tables, context_lens, prefix_seqs, prefix_start, prefix_blocks,
                            scale, out, *, max_context_len: int | None = None,
                            partition_size: int = PARTITION_AUTO, workspace=None) -> None:
    """decode_step_int8 with shared prefixes (``pa_decode_step_int8_shared``)."""
    torch = _torch()
    nb, hkv, d, s, hq, mb, mcl = _int8_decode_args(q, k_cache, v_cache, block_tables,
                                                   context_lens, out, max_context_len)
    t = key.shape[0]
    _need(tuple(key.shape) == (t, hkv, d) and tuple(value.shape) == (t, hkv, d),
          "key/value must be [T, Hkv, D]")
    _need(key.is_contiguous() and value.is_contiguous(), "key/value must be contiguous")
    _need(key.dtype == value.dtype == q.dtype, "key/value/q dtypes differ")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == t and
          slot_mapping.is_contiguous(), "slot_mapping must be contiguous int64 [T]")
    ng, nm = _shared_args(prefix_seqs, prefix_start, prefix_blocks)
    ws_ptr, ws_bytes = _workspace(q, s, hq, d, mcl, partition_size, workspace,
                                  decode_shared_workspace_bytes(s, hq, d, mcl, partition_size, ng,
                                                                nm))
    _check(load().pa_decode_step_int8_shared(
        _ptr(key), _ptr(value), _ptr(slot_mapping), t, nb, _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _scales(k_scale, hkv, d, "k_scale"), _scales(v_scale, hkv, d, "v_scale"),
        _ptr(block_tables), _ptr(context_lens), _ptr(prefix_seqs), _ptr(prefix_start),
        _ptr(prefix_blocks), ng, nm, float(scale), _ptr(out), s, hq, hkv, d, mb, mcl,
        int(partition_size), ws_ptr, ws_bytes, _dtype_code(q), _stream(q)),
        "pa_decode_step_int8_shared")


def paged_attention_decode_int8(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                context_lens, scale, out, *, max_context_len: int | None = None,
                                partition_size: int = PARTITION_AUTO, workspace=None) -> None:
    """paged_attention_decode over an INT8 cache whose values are code * scale
    (k_scale / v_scale float32 [Hkv, D]); q and out fp16 or bf16."""
    torch = _torch()
    _need(k_cache.dtype == torch.int8, "INT8 caches expected")
    nb, hkv, d = _cache_dims(k_cache, v_cache)
    s, hq, dq = q.shape
    _need(dq == d and tuple(out.shape) == (s, hq, d), "q/out must be [S, Hq, D]")
    _need(q.is_contiguous() and out.is_contiguous(), "q/out must be contiguous")
    _need(q.dtype == out.dtype, "q/out dtypes differ")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == s and block_tables.is_contiguous(),
          "block_tables must be contiguous int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and context_lens.numel() == s,
          "context_lens must be int32 [S]")
    mb = block_tables.shape[1]
    mcl = mb * BLOCK_SIZE if max_context_len is None else int(max_context_len)
    ws_ptr, ws_bytes = _workspace(q, s, hq, d, mcl, partition_size, workspace)
    _check(load().pa_paged_attention_decode_int8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _scales(k_scale, hkv, d, "k_scale"),
        _scales(v_scale, hkv, d, "v_scale"), _ptr(block_tables), _ptr(context_lens.contiguous()),
        float(scale), _ptr(out), s, hq, hkv, d, mb, mcl, int(partition_size), ws_ptr, ws_bytes,
        _dtype_code(q), _stream(q)), "pa_paged_attention_decode_int8")


def paged_attention_prefill(q, k_cache, v_cache, block_tables, query_start, context_lens, scale,
                            out, *, max_chunk_len: int) -> None:
    """Chunked prefill: the chunk queries q [T, Hq, D] (sequence s owns rows
    query_start[s] .. query_start[s+1]-1, the last positions of its
    context_lens[s]) attend causally over the paged cache; out [T, Hq, D]."""
    torch = _torch()
    nb, hkv, d = _cache_dims(k_cache, v_cache)
    t, hq, dq = q.shape
    _need(dq == d and tuple(out.shape) == (t, hq, d), "q/out must be [T, Hq, D]")
    _need(q.is_contiguous() and out.is_contiguous(), "q/out must be contiguous")
    _need(q.dtype == out.dtype == k_cache.dtype, "dtypes differ")
    s = context_lens.numel()
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and
          block_tables.shape[0] == s and block_tables.is_contiguous(),
          "block_tables must be contiguous int32 [S, MB]")
    _need(query_start.dtype == torch.int32 and query_start.numel() == s + 1 and
          query_start.is_contiguous(), "query_start must be contiguous int32 [S + 1]")
    _need(context_lens.dtype == torch.int32, "context_lens must be int32 [S]")
    _check(load().pa_paged_attention_prefill(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(query_start),
        _ptr(context_lens.contiguous()), float(scale), _ptr(out), s, hq, hkv, d,
        block_tables.shape[1], int(max_chunk_len), _dtype_code(q), _stream(q)),
        "pa_paged_attention_prefill")


# ------------------------------------------------------------------ timing
def timing_begin(capacity: int = 4096) -> None:
    _check(load().pa_timing_begin(int(capacity)), "pa_timing_begin")


def timing_end() -> dict:
    ms = (ctypes.c_double * len(KERNEL_KINDS))()
    n = (ctypes.c_int32 * len(KERNEL_KINDS))()
    _check(load().pa_timing_end(ms, n), "pa_timing_end")
    return {k: {"ms": ms[i], "launches": n[i]} for i, k in enumerate(KERNEL_KINDS)}


def timing_launches(kind: str) -> list:
    """Milliseconds of each launch of `kind` (a name of KERNEL_KINDS) that the
    last timing_end measured, in launch order."""
    i = KERNEL_KINDS.index(kind)
    n = ctypes.c_int32(0)
    _check(load().pa_timing_launches(i, None, 0, ctypes.byref(n)), "pa_timing_launches")
    ms = (ctypes.c_double * max(1, n.value))()
    _check(load().pa_timing_launches(i, ms, n.value, ctypes.byref(n)), "pa_timing_launches")
    return [ms[j] for j in range(n.value)]
