"""Expected results for a seeded workload, computed only from the oracle.

* ``pool_after(wl, phases)``: run the reference allocator over the workload's
  op script and apply its writes and copies to a host pool mirror that starts
  filled with a NaN bit pattern. Returns the mirror, the allocator and events.
* ``decode_out(wl, idx)``: fp64 attention of the decode queries over each
  sequence's logical K/V as the generator drew it (no block table involved).
* ``prefill_out(wl, which)``: fp64 causal attention of the prefill chunk rows.
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

from .allocator import BlockAllocator, run_ops
from .attention import decode_attention, prefill_attention
from .paging import PoolMirror

# quiet NaN patterns: an unwritten slot read by mistake poisons the result
NAN_BITS = {"f32": 0x7FC00001, "bf16": 0x7FC1}


def pool_after(wl, stop_before: Optional[str] = None):
    """Mirror of the pool after the op script (or up to phase ``stop_before``)."""
    alloc = BlockAllocator(wl.num_blocks, wl.block_size, wl.free_order)
    events = run_ops(alloc, wl.ops)
    np_dtype = np.float32 if wl.dtype == "f32" else np.uint16
    mirror = PoolMirror(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim,
                        np_dtype, NAN_BITS[wl.dtype])
    for ev in events:
        if ev[0] == "phase":
            if ev[1] == stop_before:
                break
        elif ev[0] == "copy":
            mirror.copy(ev[1])
        else:
            _, slots, rows = ev
            mirror.write(slots, wl.rows_k[rows], wl.rows_v[rows])
    return mirror, alloc, events


def _f64(wl, a):
    return wl.values(a).astype(np.float64)


def decode_out(wl, idx: Optional[Iterable[int]] = None) -> np.ndarray:
    """fp64 decode output for batch rows ``idx`` (default all): [len(idx), Hq, D]."""
    idx = list(range(len(wl.decode_seqs))) if idx is None else list(idx)
    ks, vs = [], []
    for i in idx:
        k, v = wl.logical_kv(wl.decode_seqs[i])
        ks.append(k.astype(np.float64))
        vs.append(v.astype(np.float64))
    return decode_attention(_f64(wl, wl.q[idx]), ks, vs, wl.scale)


def prefill_out(wl, which: Optional[Sequence[int]] = None,
                rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """fp64 prefill output for prefill sequences ``which`` (indices into
    ``wl.prefill_seqs``), restricted to chunk rows ``rows`` if given.
    Returns [len(which) * n_rows, Hq, D] in the chunk-major order of ``prefill_q``."""
    which = list(range(len(wl.prefill_seqs))) if which is None else list(which)
    C = wl.prefill_len
    rows = list(range(C)) if rows is None else list(rows)
    outs = []
    for j in which:
        seq = wl.prefill_seqs[j]
        k, v = wl.logical_kv(seq)
        start = int(wl.prefill_start[j])
        qj = _f64(wl, wl.prefill_q[j * C:(j + 1) * C])
        for i in rows:
            outs.append(prefill_attention(qj[i:i + 1], k[:start + i + 1], v[:start + i + 1],
                                          start + i, wl.scale)[0])
    return np.stack(outs) if outs else np.zeros((0, wl.num_q_heads, wl.head_dim))
