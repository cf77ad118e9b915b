"""Python handle on the library's host block manager (pa_bm_*)."""

from __future__ import annotations

import ctypes

import numpy as np

from ._lib import LIB
from .ops import NoFreeBlocks, PaError, check_status  # noqa: F401

_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)


class BlockManager:
    """Free list + reference counts + copy-on-write, implemented in C++ (libpa)."""

    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        order = None
        if free_order is not None:
            self._order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if self._order.shape != (num_blocks,):
                raise ValueError("free_order must list every block once")
            order = self._order.ctypes.data_as(_I32P)
        h = LIB.pa_bm_create(int(num_blocks), int(block_size), order)
        if not h:
            raise PaError("pa_bm_create: " + LIB.pa_last_error().decode(), 2)
        self._h = ctypes.c_void_p(h)
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            LIB.pa_bm_destroy(h)
            self._h = None

    # operations
    def add_seq(self, seq: int) -> None:
        check_status(LIB.pa_bm_add_seq(self._h, int(seq)), "pa_bm_add_seq")

    def append(self, seq: int, n: int) -> list:
        slots = np.empty(max(int(n), 1), dtype=np.int64)
        check_status(LIB.pa_bm_append(self._h, int(seq), int(n), slots.ctypes.data_as(_I64P)), "pa_bm_append")
        return slots[: int(n)].tolist()

    def append_batch(self, seqs) -> np.ndarray:
        ids = np.ascontiguousarray(np.asarray(list(seqs), dtype=np.int64))
        slots = np.empty(max(len(ids), 1), dtype=np.int64)
        check_status(LIB.pa_bm_append_batch(self._h, ids.ctypes.data_as(_I64P), len(ids),
                                            slots.ctypes.data_as(_I64P)), "pa_bm_append_batch")
        return slots[: len(ids)]

    def fork(self, parent: int, child: int) -> None:
        check_status(LIB.pa_bm_fork(self._h, int(parent), int(child)), "pa_bm_fork")

    def free_seq(self, seq: int) -> None:
        check_status(LIB.pa_bm_free_seq(self._h, int(seq)), "pa_bm_free_seq")

    def take_copies_array(self) -> np.ndarray:
        n = LIB.pa_bm_num_pending_copies(self._h)
        out = np.empty((max(n, 1), 2), dtype=np.int32)
        got = LIB.pa_bm_take_copies(self._h, out.ctypes.data_as(_I32P), n)
        if got < 0:
            raise PaError("pa_bm_take_copies: " + LIB.pa_last_error().decode(), 2)
        return out[:got]

    def take_copies(self) -> list:
        return [tuple(p) for p in self.take_copies_array().tolist()]

    # queries
    def table(self, seq: int) -> list:
        n = LIB.pa_bm_table(self._h, int(seq), None, 0)
        if n < 0:
            raise KeyError(seq)
        buf = np.empty(max(n, 1), dtype=np.int32)
        LIB.pa_bm_table(self._h, int(seq), buf.ctypes.data_as(_I32P), n)
        return buf[:n].tolist()

    def tables(self, seqs, max_blocks: int, pad: int = -1) -> np.ndarray:
        ids = np.ascontiguousarray(np.asarray(list(seqs), dtype=np.int64))
        out = np.empty((len(ids), max(int(max_blocks), 1)), dtype=np.int32)
        check_status(LIB.pa_bm_tables(self._h, ids.ctypes.data_as(_I64P), len(ids),
                                      out.ctypes.data_as(_I32P), int(max_blocks), int(pad)), "pa_bm_tables")
        return out[:, : int(max_blocks)]

    def num_tokens(self, seq: int) -> int:
        n = LIB.pa_bm_num_tokens(self._h, int(seq))
        if n < 0:
            raise KeyError(seq)
        return n

    def num_free(self) -> int:
        return int(LIB.pa_bm_num_free(self._h))

    def num_pending_copies(self) -> int:
        return int(LIB.pa_bm_num_pending_copies(self._h))

    def refcount(self, block: int) -> int:
        return int(LIB.pa_bm_refcount(self._h, int(block)))

    def replay(self, ops) -> None:
        for op in ops:
            if op[0] == "add":
                self.add_seq(op[1])
            elif op[0] == "append":
                self.append(op[1], op[2])
            elif op[0] == "fork":
                self.fork(op[1], op[2])
            elif op[0] == "free":
                self.free_seq(op[1])
            else:
                raise ValueError(op)
