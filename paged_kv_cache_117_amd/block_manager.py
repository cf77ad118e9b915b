"""Python handle on the library's host block manager (pa_bm_*)."""

from __future__ import annotations

import ctypes

import numpy as np

from ._lib import LIB
from .ops import NoFreeBlocks, PaError, check_status  # noqa: F401

_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)


class BlockManager:
    """Free list + reference counts + copy-on-write, swapping to a host pool
    and (``prefix_cache=True``) a chained-hash prefix cache, in C++ (libpa)."""

    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None, prefix_cache: bool = False):
        order = None
        if free_order is not None:
            self._order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if self._order.shape != (num_blocks,):
                raise ValueError("free_order must list every block once")
            order = self._order.ctypes.data_as(_I32P)
        create = LIB.pa_bm_create_cached if prefix_cache else LIB.pa_bm_create
        h = create(int(num_blocks), int(block_size), order)
        if not h:
            raise PaError("pa_bm_create: " + LIB.pa_last_error().decode(), 2)
        self.prefix_cache = bool(prefix_cache)
        self._h = ctypes.c_void_p(h)
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    # bound at class creation: at interpreter shutdown module globals (LIB)
    # may already be cleared when the last managers are collected
    _destroy = LIB.pa_bm_destroy

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._h = None
            try:
                type(self)._destroy(h)
            except Exception:  # the library itself is gone: nothing left to free
                pass

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

    # swapping
    def set_host_blocks(self, n: int) -> None:
        check_status(LIB.pa_bm_set_host_blocks(self._h, int(n)), "pa_bm_set_host_blocks")

    def _swap(self, fn, name, seqs) -> np.ndarray:
        ids = np.ascontiguousarray(np.asarray(list(seqs), dtype=np.int64))
        cap = sum(max(0, LIB.pa_bm_table(self._h, int(q), None, 0)) for q in ids)
        out = np.empty((max(cap, 1), 2), dtype=np.int32)
        n = ctypes.c_int(0)
        check_status(fn(self._h, ids.ctypes.data_as(_I64P), len(ids), out.ctypes.data_as(_I32P), cap,
                        ctypes.byref(n)), name)
        return out[: n.value]

    def swap_out(self, seqs) -> np.ndarray:
        """(device block, host block) pairs; the group's tables now name host blocks."""
        return self._swap(LIB.pa_bm_swap_out, "pa_bm_swap_out", seqs)

    def swap_in(self, seqs) -> np.ndarray:
        """(host block, device block) pairs; the group is back on the device."""
        return self._swap(LIB.pa_bm_swap_in, "pa_bm_swap_in", seqs)

    def is_swapped(self, seq: int) -> bool:
        r = LIB.pa_bm_is_swapped(self._h, int(seq))
        if r < 0:
            raise KeyError(seq)
        return bool(r)

    def num_host_free(self) -> int:
        return int(LIB.pa_bm_num_host_free(self._h))

    def host_refcount(self, block: int) -> int:
        return int(LIB.pa_bm_host_refcount(self._h, int(block)))

    # prefix cache
    def add_seq_cached(self, seq: int, tokens, extra: bytes = b"") -> int:
        """Start ``seq`` from its prompt; returns how many tokens the cache already holds."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        n = ctypes.c_int(0)
        check_status(LIB.pa_bm_add_seq_cached(self._h, int(seq), t.ctypes.data_as(_I32P), len(t), bytes(extra),
                                              len(extra), ctypes.byref(n)), "pa_bm_add_seq_cached")
        return n.value

    def append_tokens(self, seq: int, tokens) -> list:
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        slots = np.empty(max(len(t), 1), dtype=np.int64)
        check_status(LIB.pa_bm_append_tokens(self._h, int(seq), t.ctypes.data_as(_I32P), len(t),
                                             slots.ctypes.data_as(_I64P)), "pa_bm_append_tokens")
        return slots[: len(t)].tolist()

    def num_cached_blocks(self) -> int:
        return int(LIB.pa_bm_num_cached_blocks(self._h))

    def block_hash(self, seq: int, j: int) -> bytes:
        buf = ctypes.create_string_buffer(32)
        if LIB.pa_bm_block_hash(self._h, int(seq), int(j), buf) != 0:
            raise KeyError((seq, j))
        return buf.raw

    def cached_block(self, h: bytes) -> int:
        return int(LIB.pa_bm_cached_block(self._h, bytes(h)))

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
