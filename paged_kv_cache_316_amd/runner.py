"""Host driver: turn a serving loop's allocator operations into device work.

``run_script`` feeds an op script (allocate / extend / append / fork / free,
with the K/V row id of every token it adds) to the C++ block allocator and
returns what the device must do, in order: block copies and slot writes.
Consecutive writes are merged into one batch; a copy flushes the pending
writes first, and the write of the token that caused a copy comes after it
(copy-on-write, "vLLM PagedAttention explained", section 4.1).

``apply_events`` then runs those events with the library's kernels
(pa_copy_blocks, pa_cache_write). K/V rows come from a device array
``rows_k`` / ``rows_v`` [R, Hkv, D] indexed by row id.
"""

from __future__ import annotations

from typing import List, Tuple

import numpy as np
import torch

from . import ops
from .allocator import BlockAllocator


def run_script(alloc: BlockAllocator, script) -> List[Tuple]:
    events: List[Tuple] = []
    pend_slots: List[np.ndarray] = []
    pend_rows: List[np.ndarray] = []

    def flush():
        if pend_slots:
            events.append(("write", np.concatenate(pend_slots), np.concatenate(pend_rows)))
            pend_slots.clear()
            pend_rows.clear()

    for op in script:
        kind = op[0]
        if kind == "phase":
            flush()
            events.append(("phase", op[1]))
        elif kind == "alloc":
            _, seq, tokens, rows = op
            cached, slots = alloc.allocate(seq, tokens)
            if len(tokens) > cached:
                pend_slots.append(slots[cached:])
                pend_rows.append(np.asarray(rows[cached:], dtype=np.int64))
        elif kind == "append" or kind == "extend":
            _, seq, tok, rows = op
            if kind == "append":
                slots = np.array([alloc.append_slot(seq, tok)], dtype=np.int64)
                rows = np.array([rows], dtype=np.int64)
            else:
                slots = alloc.extend(seq, tok)
                rows = np.asarray(rows, dtype=np.int64)
            copies = alloc.take_copies()
            if len(copies):
                flush()
                events.append(("copy", copies))
            pend_slots.append(slots)
            pend_rows.append(rows)
        elif kind == "fork":
            alloc.fork(op[1], op[2])
        elif kind == "free":
            alloc.free(op[1])
        else:
            raise ValueError(f"unknown op {kind!r}")
    flush()
    return events


def split_phases(events) -> dict:
    """{phase name: events}; events before the first marker are under "setup"."""
    out = {"setup": []}
    cur = "setup"
    for ev in events:
        if ev[0] == "phase":
            cur = ev[1]
            out.setdefault(cur, [])
        else:
            out[cur].append(ev)
    return out


class WriteBatch:
    """Device-resident inputs of one pa_cache_write call."""

    def __init__(self, slots: np.ndarray, rows: np.ndarray, rows_k: torch.Tensor,
                 rows_v: torch.Tensor):
        dev = rows_k.device
        idx = torch.from_numpy(np.ascontiguousarray(rows)).to(dev)
        self.slots = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).to(dev)
        self.k = rows_k.index_select(0, idx).contiguous()
        self.v = rows_v.index_select(0, idx).contiguous()

    def run(self, pool: ops.KVPool) -> None:
        ops.cache_write(pool, self.k, self.v, self.slots)


def apply_events(pool: ops.KVPool, events, rows_k: torch.Tensor, rows_v: torch.Tensor,
                 max_batch_tokens: int = 1 << 16) -> None:
    for ev in events:
        if ev[0] == "copy":
            ops.copy_blocks(pool, torch.from_numpy(np.ascontiguousarray(ev[1], dtype=np.int32))
                            .to(pool.k.device))
        elif ev[0] == "write":
            _, slots, rows = ev
            for a in range(0, len(slots), max_batch_tokens):
                WriteBatch(slots[a:a + max_batch_tokens], rows[a:a + max_batch_tokens],
                           rows_k, rows_v).run(pool)
