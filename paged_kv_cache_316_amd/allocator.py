"""Python face of the library's C++ host block allocator (pa_alloc_*)."""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from ._lib import check, lib


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class BlockAllocator:
    """FIFO free list, reference counts, fork + copy-on-write, prefix hashing.

    Sequence ids are int64. Methods raise OutOfBlocks / AllocatorStateError
    (from the C status) and leave the allocator unchanged on failure.
    """

    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        self._h = ctypes.c_void_p()
        fo = None if free_order is None else _i32(free_order)
        if fo is not None and fo.shape != (num_blocks,):
            raise ValueError("free_order must have num_blocks entries")
        check(lib().pa_alloc_create(int(num_blocks), int(block_size),
                                    None if fo is None else fo.ctypes.data,
                                    ctypes.byref(self._h)))
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            lib().pa_alloc_destroy(h)
            self._h = None

    def allocate(self, seq: int, tokens: Sequence[int]) -> Tuple[int, np.ndarray]:
        t = _i32(tokens)
        slots = np.empty(len(t), dtype=np.int64)
        cached = ctypes.c_int32()
        check(lib().pa_alloc_allocate(self._h, int(seq), t.ctypes.data if len(t) else None,
                                      len(t), ctypes.byref(cached),
                                      slots.ctypes.data if len(t) else None))
        return cached.value, slots

    def append_slot(self, seq: int, token: int = 0) -> int:
        s = ctypes.c_int64()
        check(lib().pa_alloc_append_slot(self._h, int(seq), int(token), ctypes.byref(s)))
        return s.value

    def extend(self, seq: int, tokens: Sequence[int]) -> np.ndarray:
        t = _i32(tokens)
        slots = np.empty(len(t), dtype=np.int64)
        check(lib().pa_alloc_extend(self._h, int(seq), t.ctypes.data if len(t) else None, len(t),
                                    slots.ctypes.data if len(t) else None))
        return slots

    def fork(self, parent: int, child: int) -> None:
        check(lib().pa_alloc_fork(self._h, int(parent), int(child)))

    def free(self, seq: int) -> None:
        check(lib().pa_alloc_free(self._h, int(seq)))

    def take_copies(self) -> np.ndarray:
        n = ctypes.c_int32()
        buf = np.empty((16, 2), dtype=np.int32)
        st = lib().pa_alloc_take_copies(self._h, buf.ctypes.data, 16, ctypes.byref(n))
        if st != 0 and n.value > 16:
            buf = np.empty((n.value, 2), dtype=np.int32)
            st = lib().pa_alloc_take_copies(self._h, buf.ctypes.data, n.value, ctypes.byref(n))
        check(st)
        return buf[:n.value].copy()

    def seq_len(self, seq: int) -> int:
        n = ctypes.c_int32()
        check(lib().pa_alloc_seq_len(self._h, int(seq), ctypes.byref(n)))
        return n.value

    def block_table(self, seq: int) -> np.ndarray:
        n = ctypes.c_int32()
        cap = -(-self.seq_len(seq) // self.block_size)
        out = np.empty(max(cap, 1), dtype=np.int32)
        check(lib().pa_alloc_block_table(self._h, int(seq), out.ctypes.data, cap, ctypes.byref(n)))
        return out[:n.value].copy()

    def batch_tables(self, seq_ids: Sequence[int], max_blocks: Optional[int] = None
                     ) -> Tuple[np.ndarray, np.ndarray]:
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        if max_blocks is None:
            max_blocks = max([-(-self.seq_len(int(s)) // self.block_size) for s in ids] + [1])
        tables = np.empty((len(ids), max_blocks), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        check(lib().pa_alloc_batch_tables(self._h, ids.ctypes.data, len(ids), tables.ctypes.data,
                                          int(max_blocks), lens.ctypes.data))
        return tables, lens

    @property
    def num_free(self) -> int:
        return int(lib().pa_alloc_num_free(self._h))

    def ref_count(self, block: int) -> int:
        n = ctypes.c_int32()
        check(lib().pa_alloc_ref_count(self._h, int(block), ctypes.byref(n)))
        return n.value
