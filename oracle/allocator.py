"""Reference block manager (host only, plain Python).

Behaviour, with the passage each rule follows:

* Free list: a FIFO of physical block ids; blocks are taken from the front and
  returned to the back ("LLM inference engine internals", section 2.3, the
  ``free_blocks`` deque with ``popleft`` / ``append``). A seeded permutation of
  the pool may set its initial order.
* ``allocate(seq, tokens)``: ceil(n / B) blocks for an n-token prompt (same
  section, ``allocate``), except that leading full blocks whose content is
  already cached are shared instead (prefix caching below).
* ``append_slot(seq, token)``: if the last block has room, the slot is
  last_block * B + (n mod B); otherwise a new block is taken and the slot is
  new_block * B; an empty free list is an out-of-memory condition that leaves
  the state unchanged (same section, ``append_slot`` returning None).
* ``free(seq)``: the sequence's blocks are released in table order (same
  section, ``free``); with sharing, a release decrements the block's
  reference count and only a count of zero returns the block to the free list
  ("vLLM PagedAttention explained", section 4.2: pruned beams release the
  blocks they alone hold, shared ancestors stay).
* ``fork(parent, child)``: the child's table is a copy of the parent's and
  every block's reference count goes up by one ("vLLM PagedAttention
  explained", section 4.1: two samples map to the same physical blocks with
  ref count 2).
* Copy-on-write (same section): appending into a partially filled last block
  that other tables also hold (count > 1) first moves this sequence onto a new
  block: the pair (old, new) is queued for a device block copy, the old count
  drops by one and the new block starts at one. The page's example: blocks
  7, 1 shared at count 2; the first sample's append copies block 1 to block 3,
  after which block 1 and block 3 each have count 1.
* Prefix caching ("Why PagedAttention multiplies LLM serving throughput",
  section "Automatic prefix caching"; "vLLM PagedAttention explained", section
  7.1): each full block of a prompt gets a hash of (hash of the previous
  block, the block's token ids). While the leading blocks of a new prompt find
  a live block with the same hash and the same token ids, that block is shared
  (count + 1) and its K/V is not written again. A partial block is never
  shared this way. Our readings where the pages are silent: the hash is
  64-bit FNV-1a over the little-endian bytes of the previous hash (0 for the
  first block) followed by the int32 token ids; only full blocks laid down by
  ``allocate`` are registered; a block leaves the table when its count drops
  to zero; an existing entry is never overwritten.
* ``extend(seq, tokens)``: a prefill chunk appended to an existing sequence
  ("vLLM PagedAttention explained", section 7.2: chunks join the existing
  block table) — the same as one ``append_slot`` per token, but all or
  nothing when blocks run out.
"""

from __future__ import annotations

from collections import deque
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

_FNV_OFFSET = 0xCBF29CE484222325
_FNV_PRIME = 0x100000001B3
_M64 = (1 << 64) - 1


class OutOfBlocks(Exception):
    """No free block is left; the allocator state is unchanged."""


class AllocatorStateError(Exception):
    """Unknown or duplicate sequence id."""


def fnv1a64(data: bytes) -> int:
    """64-bit FNV-1a: for each byte, xor it in, then multiply by the FNV prime."""
    h = _FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * _FNV_PRIME) & _M64
    return h


def block_hash(prev: int, tokens: Sequence[int]) -> int:
    """FNV-1a 64 over prev (8 bytes LE) then each token (4 bytes LE, two's complement)."""
    data = int(prev).to_bytes(8, "little") + b"".join(
        int(t & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens)
    return fnv1a64(data)


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if block_size <= 0 or num_blocks <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.B = int(block_size)
        self.N = int(num_blocks)
        order = list(range(self.N)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(self.N)):
            raise ValueError("free_order must be a permutation of the pool")
        self.free: deque = deque(order)
        self.ref: List[int] = [0] * self.N
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.block_of_hash: Dict[int, int] = {}
        self.hash_of_block: Dict[int, int] = {}
        self.tokens_of_block: Dict[int, Tuple[int, ...]] = {}
        self.copies: List[Tuple[int, int]] = []

    # -- queries -----------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self.free)

    def block_table(self, seq: int) -> List[int]:
        self._need(seq)
        return list(self.tables[seq])

    def seq_len(self, seq: int) -> int:
        self._need(seq)
        return self.lens[seq]

    def take_copies(self) -> List[Tuple[int, int]]:
        c, self.copies = self.copies, []
        return c

    def _need(self, seq: int) -> None:
        if seq not in self.tables:
            raise AllocatorStateError(f"unknown sequence {seq}")

    # -- operations --------------------------------------------------------
    def allocate(self, seq: int, tokens: Sequence[int]) -> Tuple[int, List[int]]:
        """New sequence holding ``tokens``. Returns (cached_tokens, slots of all positions)."""
        if seq in self.tables:
            raise AllocatorStateError(f"sequence {seq} already exists")
        tokens = [int(t) for t in tokens]
        n, B = len(tokens), self.B
        nblk = -(-n // B)
        nfull = n // B
        hashes, prev = [], 0
        for j in range(nfull):
            prev = block_hash(prev, tokens[j * B:(j + 1) * B])
            hashes.append(prev)
        hits: List[int] = []
        for j in range(nfull):
            b = self.block_of_hash.get(hashes[j])
            if b is None or self.tokens_of_block[b] != tuple(tokens[j * B:(j + 1) * B]):
                break
            hits.append(b)
        if nblk - len(hits) > len(self.free):
            raise OutOfBlocks()
        table = []
        for b in hits:
            self.ref[b] += 1
            table.append(b)
        for j in range(len(hits), nblk):
            b = self.free.popleft()
            self.ref[b] = 1
            table.append(b)
            if j < nfull and hashes[j] not in self.block_of_hash:
                self.block_of_hash[hashes[j]] = b
                self.hash_of_block[b] = hashes[j]
                self.tokens_of_block[b] = tuple(tokens[j * B:(j + 1) * B])
        self.tables[seq] = table
        self.lens[seq] = n
        slots = [table[t // B] * B + t % B for t in range(n)]
        return len(hits) * B, slots

    def append_slot(self, seq: int, token: int = 0) -> int:
        self._need(seq)
        table, L, B = self.tables[seq], self.lens[seq], self.B
        if L % B:
            last = table[-1]
            if self.ref[last] > 1:  # shared partial block: copy on write
                if not self.free:
                    raise OutOfBlocks()
                new = self.free.popleft()
                self.ref[last] -= 1
                self.ref[new] = 1
                table[-1] = new
                self.copies.append((last, new))
                slot = new * B + L % B
            else:
                slot = last * B + L % B
        else:
            if not self.free:
                raise OutOfBlocks()
            new = self.free.popleft()
            self.ref[new] = 1
            table.append(new)
            slot = new * B
        self.lens[seq] = L + 1
        return slot

    def extend(self, seq: int, tokens: Sequence[int]) -> List[int]:
        self._need(seq)
        n, L, B = len(tokens), self.lens[seq], self.B
        need = -(-(L + n) // B) - (-(-L // B))
        if n and L % B and self.ref[self.tables[seq][-1]] > 1:
            need += 1
        if need > len(self.free):
            raise OutOfBlocks()
        return [self.append_slot(seq, t) for t in tokens]

    def fork(self, parent: int, child: int) -> None:
        self._need(parent)
        if child in self.tables:
            raise AllocatorStateError(f"sequence {child} already exists")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def free_seq(self, seq: int) -> None:
        self._need(seq)
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
                h = self.hash_of_block.pop(b, None)
                if h is not None:
                    del self.block_of_hash[h]
                    del self.tokens_of_block[b]
        del self.lens[seq]


def run_ops(alloc: BlockAllocator, ops) -> list:
    """Execute a workload's op script; return the device-side events in order.

    Events: ("phase", name), ("copy", [(src, dst), ...]) and
    ("write", slots[int64], rows[int64]). A copy always precedes the write of
    the token that caused it.
    """
    events = []
    for op in ops:
        kind = op[0]
        if kind == "phase":
            events.append(("phase", op[1]))
        elif kind == "alloc":
            _, seq, tokens, rows = op
            cached, slots = alloc.allocate(seq, tokens)
            if len(tokens) > cached:
                events.append(("write", np.asarray(slots[cached:], dtype=np.int64),
                               np.asarray(rows[cached:], dtype=np.int64)))
        elif kind in ("append", "extend"):
            _, seq, tok, rows = op
            if kind == "append":
                slots, rows = [alloc.append_slot(seq, tok)], [rows]
            else:
                slots = alloc.extend(seq, tok)
            copies = alloc.take_copies()
            if copies:
                events.append(("copy", copies))
            events.append(("write", np.asarray(slots, dtype=np.int64),
                           np.asarray(rows, dtype=np.int64)))
        elif kind == "fork":
            alloc.fork(op[1], op[2])
        elif kind == "free":
            alloc.free_seq(op[1])
        else:
            raise ValueError(f"unknown op {kind!r}")
    return events
