"""Expected results for a seeded workload, computed only from the oracle.

* ``pool_after(wl, phases)``: run the reference allocator over the workload's
  op script and apply its writes and copies to a host pool mirror that starts
  filled with a NaN bit pattern. Returns the mirror, the allocator and events.
* ``decode_out(wl, idx)``: fp64 attention of the decode queries over each
  sequence's logical K/V as the generator drew it (no block table involved);
  for an FP8 pool, the values its codes stand for (``fp8``).
* ``prefill_out(wl, which)``: fp64 causal attention of the prefill chunk rows.
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

from . import fp8
from .allocator import BlockAllocator, run_ops
from .attention import decode_attention, prefill_attention
from .paging import PoolMirror

# quiet NaN patterns: an unwritten slot read by mistake poisons the result
NAN_BITS = {"f32": 0x7FC00001, "bf16": 0x7FC1, "fp8_e4m3": 0x7F}
_MIRROR_DTYPE = {"f32": np.float32, "bf16": np.uint16, "fp8_e4m3": np.uint8}


_ALL_BF16 = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)  # every bf16 value


def _code_table(scale: float) -> np.ndarray:
    """fp8.quantize of every bf16 bit pattern: quantize acts on each value
    alone, so a bf16 array's codes are this table indexed by its bits."""
    return fp8.quantize(_ALL_BF16, scale)


def _quantize_bf16(wl, rows, scale):
    if rows.dtype == np.uint16:  # bf16 bits (all FP8 workloads draw bf16 rows)
        return _code_table(scale)[rows]
    return fp8.quantize(wl.values(rows), scale)


def stored_rows(wl, rows_k, rows_v):
    """What the pool holds for these K/V rows: the rows themselves, or their
    FP8 codes under the pool's scales."""
    if wl.pool_dtype != "fp8_e4m3":
        return rows_k, rows_v
    return _quantize_bf16(wl, rows_k, wl.k_scale), _quantize_bf16(wl, rows_v, wl.v_scale)


def logical_kv(wl, seq):
    """float64 K, V a sequence holds, as the pool represents them."""
    r = wl.hist[seq]
    if wl.pool_dtype != "fp8_e4m3":
        k, v = wl.logical_kv(seq)
        return k.astype(np.float64), v.astype(np.float64)
    ck, cv = stored_rows(wl, wl.rows_k[r], wl.rows_v[r])
    return (fp8.dequantize(np.arange(256), wl.k_scale)[ck],
            fp8.dequantize(np.arange(256), wl.v_scale)[cv])


def pool_after(wl, stop_before: Optional[str] = None):
    """Mirror of the pool after the op script (or up to phase ``stop_before``)."""
    alloc = BlockAllocator(wl.num_blocks, wl.block_size, wl.free_order)
    events = run_ops(alloc, wl.ops)
    mirror = PoolMirror(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim,
                        _MIRROR_DTYPE[wl.pool_dtype], NAN_BITS[wl.pool_dtype])
    for ev in events:
        if ev[0] == "phase":
            if ev[1] == stop_before:
                break
        elif ev[0] == "copy":
            mirror.copy(ev[1])
        else:
            _, slots, rows = ev
            mirror.write(slots, *stored_rows(wl, wl.rows_k[rows], wl.rows_v[rows]))
    return mirror, alloc, events


def _f64(wl, a):
    return wl.values(a).astype(np.float64)


def decode_out(wl, idx: Optional[Iterable[int]] = None) -> np.ndarray:
    """fp64 decode output for batch rows ``idx`` (default all): [len(idx), Hq, D]."""
    idx = list(range(len(wl.decode_seqs))) if idx is None else list(idx)
    ks, vs = [], []
    for i in idx:
        k, v = logical_kv(wl, wl.decode_seqs[i])
        ks.append(k)
        vs.append(v)
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
        k, v = logical_kv(wl, seq)
        start = int(wl.prefill_start[j])
        qj = _f64(wl, wl.prefill_q[j * C:(j + 1) * C])
        for i in rows:
            outs.append(prefill_attention(qj[i:i + 1], k[:start + i + 1], v[:start + i + 1],
                                          start + i, wl.scale)[0])
    return np.stack(outs) if outs else np.zeros((0, wl.num_q_heads, wl.head_dim))
