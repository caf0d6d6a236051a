"""Python binding of the host-side block pool in libpa.so (``include/pa_pool.h``).

Argument marshalling only: every decision (which block, when to grow, when to
copy, where each token's slot is) is taken by the C++ pool. Block tables are
Python lists of ints here and int32 arrays across the C boundary.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import PaError, load_library

_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_i64p = ctypes.POINTER(ctypes.c_int64)
_configured = False


def _lib() -> ctypes.CDLL:
    global _configured
    lib = load_library()
    if not _configured:
        c_int, c_i32, c_i64, c_p = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        lib.pa_pool_create.argtypes = [c_i32, c_i32, _c_i32p, ctypes.POINTER(c_p)]
        lib.pa_pool_create.restype = c_int
        lib.pa_pool_destroy.argtypes = [c_p]
        lib.pa_pool_destroy.restype = None
        lib.pa_pool_num_free.argtypes = [c_p]
        lib.pa_pool_num_free.restype = c_i32
        lib.pa_pool_ref_count.argtypes = [c_p, c_i32]
        lib.pa_pool_ref_count.restype = c_i32
        lib.pa_pool_blocks_for.argtypes = [c_p, c_i64]
        lib.pa_pool_blocks_for.restype = c_i64
        lib.pa_pool_allocate.argtypes = [c_p, c_i64, _c_i32p, c_i32, _c_i32p]
        lib.pa_pool_allocate.restype = c_int
        lib.pa_pool_append_slot.argtypes = [c_p, _c_i32p, _c_i32p, c_i32, c_i64, _c_i32p]
        lib.pa_pool_append_slot.restype = c_int
        lib.pa_pool_share.argtypes = [c_p, _c_i32p, c_i32]
        lib.pa_pool_share.restype = c_int
        lib.pa_pool_release.argtypes = [c_p, _c_i32p, c_i32]
        lib.pa_pool_release.restype = c_int
        lib.pa_pool_make_writable.argtypes = [c_p, _c_i32p, c_i32, c_i32, _c_i32p, _c_i32p]
        lib.pa_pool_make_writable.restype = c_int
        lib.pa_prepare_step.argtypes = [c_i32, _c_i32p, _c_i64p, _c_i64p, _c_i64p, c_i32, c_i32, _c_i64p,
                                        _c_i64p, _c_i32p, _c_i32p, c_i64, _c_i64p]
        lib.pa_prepare_step.restype = c_int
        _configured = True
    return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise PaError(status, where)


def _i32(values) -> ctypes.Array:
    values = list(values)
    return (ctypes.c_int32 * max(1, len(values)))(*values)


class BlockPool:
    """A pool of ``num_blocks`` KV blocks of ``block_size`` tokens (see pa_pool.h)."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self._lib = _lib()
        self.block_size = block_size
        handle = ctypes.c_void_p()
        order = None if free_order is None else _i32(int(b) for b in free_order)
        if free_order is not None and len(free_order) != num_blocks:
            raise ValueError("free_order must list every block once")
        _check(self._lib.pa_pool_create(num_blocks, block_size, order, ctypes.byref(handle)), "pa_pool_create")
        self._h = handle

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pa_pool_destroy(h)
            self._h = None

    def num_free(self) -> int:
        return int(self._lib.pa_pool_num_free(self._h))

    def ref_count(self, block: int) -> int:
        return int(self._lib.pa_pool_ref_count(self._h, block))

    def blocks_for(self, num_tokens: int) -> int:
        return int(self._lib.pa_pool_blocks_for(self._h, num_tokens))

    def can_allocate(self, num_tokens: int) -> bool:
        return self.blocks_for(num_tokens) <= self.num_free()

    def allocate(self, num_tokens: int) -> list[int]:
        cap = max(0, self.blocks_for(num_tokens))
        buf = (ctypes.c_int32 * max(1, cap))()
        n = ctypes.c_int32(0)
        _check(self._lib.pa_pool_allocate(self._h, num_tokens, buf, cap, ctypes.byref(n)), "pa_pool_allocate")
        return [int(buf[i]) for i in range(n.value)]

    def append_slot(self, table: list[int], cur_len: int):
        """Grow ``table`` in place to cover position ``cur_len``; the block
        taken, or None."""
        cap = max(len(table), cur_len // self.block_size + 1)
        buf = (ctypes.c_int32 * cap)(*table)
        n = ctypes.c_int32(len(table))
        taken = ctypes.c_int32(-1)
        _check(self._lib.pa_pool_append_slot(self._h, buf, ctypes.byref(n), cap, cur_len, ctypes.byref(taken)),
               "pa_pool_append_slot")
        table[:] = [int(buf[i]) for i in range(n.value)]
        return None if taken.value < 0 else int(taken.value)

    def share(self, blocks) -> None:
        blocks = list(blocks)
        _check(self._lib.pa_pool_share(self._h, _i32(blocks), len(blocks)), "pa_pool_share")

    def release(self, blocks) -> None:
        blocks = list(blocks)
        _check(self._lib.pa_pool_release(self._h, _i32(blocks), len(blocks)), "pa_pool_release")

    def make_writable(self, table: list[int], idx: int):
        """Copy-on-write for ``table[idx]`` (in place); (source, destination) or None."""
        buf = _i32(table)
        src, dst = ctypes.c_int32(-1), ctypes.c_int32(-1)
        _check(self._lib.pa_pool_make_writable(self._h, buf, len(table), idx, ctypes.byref(src),
                                               ctypes.byref(dst)), "pa_pool_make_writable")
        table[:] = [int(buf[i]) for i in range(len(table))]
        return None if src.value < 0 else (int(src.value), int(dst.value))


def prepare_step(tables, num_computed, num_new, block_size: int, max_blocks: int):
    """Step inputs from block tables (see pa_prepare_step): numpy arrays
    (slot_mapping int64 [T], positions int64 [T], block_tables int32
    [S, max_blocks], context_lens int32 [S])."""
    S = len(tables)
    flat = np.ascontiguousarray(np.concatenate([np.asarray(t, np.int32) for t in tables])
                                if S and sum(len(t) for t in tables) else np.zeros(1, np.int32))
    offs = np.zeros(S + 1, np.int64)
    offs[1:] = np.cumsum([len(t) for t in tables]) if S else []
    done = np.ascontiguousarray(np.asarray(num_computed, np.int64).reshape(S))
    new = np.ascontiguousarray(np.asarray(num_new, np.int64).reshape(S))
    T = int(new.sum()) if S else 0
    slots = np.zeros(max(1, T), np.int64)
    pos = np.zeros(max(1, T), np.int64)
    bt = np.zeros((max(1, S), max(1, max_blocks)), np.int32)
    lens = np.zeros(max(1, S), np.int32)
    n = ctypes.c_int64(0)
    ptr = lambda a, t: a.ctypes.data_as(t)  # noqa: E731
    _check(_lib().pa_prepare_step(S, ptr(flat, _c_i32p), ptr(offs, _c_i64p), ptr(done, _c_i64p),
                                  ptr(new, _c_i64p), block_size, max_blocks, ptr(slots, _c_i64p),
                                  ptr(pos, _c_i64p), ptr(bt, _c_i32p), ptr(lens, _c_i32p), T, ctypes.byref(n)),
           "pa_prepare_step")
    return slots[:T], pos[:T], bt[:S, :max_blocks], lens[:S]
