"""Host mirror of the physical KV block pool.

Layout of one pool: [num_blocks][num_kv_heads][block_size][head_dim], i.e.
head-major inside a block. The pages draw the pool as
[num_blocks, block_size, num_heads, head_dim] in their kernel outline ("LLM
inference engine internals", section 2.4); which of the two is used is a free
choice, and the library takes the head-major one so that one (block, head)
tile is contiguous. Everything below goes through ``_addr`` only.

Slot rule ("LLM inference engine internals", section 2.3, ``append_slot``):
slot = physical_block * block_size + offset, so block = slot // block_size
and offset = slot % block_size. A negative slot is padding and is skipped.
"""

from __future__ import annotations

from typing import Iterable, Sequence

import numpy as np


class PoolMirror:
    def __init__(self, num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                 np_dtype, fill_bits: int = 0):
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.block_size = block_size
        self.k = np.empty(shape, dtype=np_dtype)
        self.v = np.empty(shape, dtype=np_dtype)
        # fill with a bit pattern (e.g. a NaN) so unwritten slots are recognisable
        self.k.view(_uint_of(np_dtype))[...] = fill_bits
        self.v.view(_uint_of(np_dtype))[...] = fill_bits

    def _addr(self, slot: int):
        return slot // self.block_size, slot % self.block_size

    def write(self, slots: Sequence[int], k_rows: np.ndarray, v_rows: np.ndarray) -> None:
        """Store token i's K/V rows [Hkv, D] at slot[i]; negative slots are skipped."""
        slots = np.asarray(slots, dtype=np.int64)
        keep = slots >= 0
        blocks, offs = self._addr(slots[keep])
        self.k[blocks, :, offs, :] = np.asarray(k_rows)[keep]
        self.v[blocks, :, offs, :] = np.asarray(v_rows)[keep]

    def copy(self, pairs: Iterable[Sequence[int]]) -> None:
        """Copy-on-write: physical block dst becomes a copy of src, in the given order."""
        for src, dst in pairs:
            self.k[dst] = self.k[src]
            self.v[dst] = self.v[src]

    def gather(self, table: Sequence[int], length: int):
        """Logical K, V [length, Hkv, D] of a sequence through its block table."""
        t = np.arange(length, dtype=np.int64)
        blocks = np.asarray(table, dtype=np.int64)[t // self.block_size]
        offs = t % self.block_size
        return self.k[blocks, :, offs, :], self.v[blocks, :, offs, :]


def swap(dst: "PoolMirror", src: "PoolMirror", pairs: Iterable[Sequence[int]]) -> None:
    """Block swapping between two pools of one geometry (a device pool and its
    CPU swap space): block d of ``dst`` becomes a copy of block s of ``src``
    for each (s, d), all KV heads, K and V. Preemption by swapping moves a
    request's blocks out to CPU memory and back ("LLM inference engine
    internals", section 3.2; "Why PagedAttention multiplies LLM serving
    throughput", section "Scheduling and preemption"); the scheduler names the
    moves as blocks_to_swap_in / blocks_to_swap_out ("LLM inference engine
    internals", section 3.1)."""
    for s, d in pairs:
        dst.k[d] = src.k[s]
        dst.v[d] = src.v[s]


def _uint_of(np_dtype):
    return {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[np.dtype(np_dtype).itemsize]
