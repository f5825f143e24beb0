"""Containers and dtype helpers for the synthetic workloads (data only)."""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Any, Dict, List, Optional, Tuple

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even), as uint16 bits.

    Inputs are finite draws, so the NaN branch of a full converter is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One seeded workload.

    Storage convention: for dtype "f32" the arrays ``rows_k``, ``rows_v``,
    ``q`` and ``prefill_q`` hold float32 values; for "bf16" they hold the
    uint16 bit patterns of bfloat16 values. ``values(a)`` widens either to
    float32 exactly.

    ``rows_k[r]`` / ``rows_v[r]`` is the key/value of one written token,
    shape ``[num_kv_heads, head_dim]``. ``hist[seq]`` lists, in logical order,
    the row ids a sequence holds when the decode batch runs.

    ``ops`` is the script a serving loop issues to the block allocator:
      ("alloc",  seq, tokens[int32], rows[int64])   new sequence with a prompt
      ("extend", seq, tokens[int32], rows[int64])   append a chunk of tokens
      ("append", seq, token, row)                   append one token
      ("fork",   parent, child)                     child shares parent's blocks
      ("free",   seq)                               sequence finished / pruned
      ("phase",  name)                              start of "prefill" or "decode"
    Every token an op adds carries the row id of its key/value.
    """

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    free_order: np.ndarray
    rows_k: np.ndarray
    rows_v: np.ndarray
    q: np.ndarray
    decode_seqs: List[int]
    hist: Dict[int, np.ndarray]
    ops: List[Tuple[Any, ...]]
    prefill_seqs: List[int] = field(default_factory=list)
    prefill_start: Optional[np.ndarray] = None  # first chunk position per prefill seq
    prefill_len: int = 0
    prefill_q: Optional[np.ndarray] = None  # [len(prefill_seqs)*prefill_len, Hq, D]
    meta: Dict[str, Any] = field(default_factory=dict)
    # KV pool storage type when it differs from ``dtype``: "fp8_e4m3" stores
    # the K/V rows (drawn as ``dtype``) as 8-bit codes, one scale per pool
    kv_dtype: str = ""
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def pool_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def elt_bytes(self) -> int:
        """Bytes per stored K/V element in the pool."""
        return {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[self.pool_dtype]

    @property
    def seq_lens(self) -> np.ndarray:
        return np.array([len(self.hist[s]) for s in self.decode_seqs], dtype=np.int64)

    def values(self, a: np.ndarray) -> np.ndarray:
        """float32 view of stored values (exact for both dtypes)."""
        if self.dtype == "f32":
            return np.asarray(a, dtype=np.float32)
        return bf16_bits_to_f32(a)

    def logical_kv(self, seq: int) -> Tuple[np.ndarray, np.ndarray]:
        """The contiguous K and V (float32 values) a sequence holds at decode time."""
        r = self.hist[seq]
        return self.values(self.rows_k[r]), self.values(self.rows_v[r])
