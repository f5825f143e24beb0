"""Device entry points: argument marshalling from torch tensors to the C ABI.

torch supplies device memory and the current stream; every step of the
attention path runs in the library's HIP kernels.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

from ._lib import PA_BF16, PA_F32, PA_FP8_E4M3, PaPool, PagedKVError, check, lib

_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.float8_e4m3fn: PA_FP8_E4M3}


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


# Input checks: with PAGEDKV_CHECK=1 in the environment (or set_input_checks(True))
# every call first copies its index arrays (tables, lengths, slots, copy pairs,
# chunk offsets) to the host and has the library's pa_check_* functions verify
# them, raising on the first violation. A debug aid: it synchronizes the stream.
_CHECK_INPUTS = os.environ.get("PAGEDKV_CHECK", "") == "1"


def set_input_checks(on: bool) -> None:
    global _CHECK_INPUTS
    _CHECK_INPUTS = bool(on)


def _host(a, dtype) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def check_batch(pool: "KVPool", block_tables, seq_lens) -> None:
    """Tables and lengths index inside the pool (host check; raises PagedKVError)."""
    t, n = _host(block_tables, np.int32), _host(seq_lens, np.int32)
    if t.ndim != 2 or n.shape != (t.shape[0],):
        raise ValueError("block_tables must be [S, maxB] and seq_lens [S]")
    check(lib().pa_check_batch(ctypes.byref(pool.c), t.ctypes.data, t.shape[1], n.ctypes.data,
                               n.shape[0]))


def check_slots(pool: "KVPool", slot_mapping) -> None:
    """Slots inside the pool and distinct (host check)."""
    s = _host(slot_mapping, np.int64).reshape(-1)
    check(lib().pa_check_slots(ctypes.byref(pool.c), s.ctypes.data, s.shape[0]))


def check_copies(pool: "KVPool", src_dst) -> None:
    """Copy pairs inside the pool, no block both a source and a destination (host check)."""
    p = _host(src_dst, np.int32).reshape(-1, 2)
    check(lib().pa_check_copies(ctypes.byref(pool.c), p.ctypes.data, p.shape[0]))


def check_chunks(q_start_loc, seq_lens, num_decode: int, max_q_len: int, total_rows: int) -> None:
    """Chunk row offsets consistent with lengths, max_q_len and the rows of q (host check)."""
    loc, n = _host(q_start_loc, np.int32), _host(seq_lens, np.int32)
    if loc.shape != (n.shape[0] + 1,):
        raise ValueError("q_start_loc must have one entry more than seq_lens")
    check(lib().pa_check_chunks(loc.ctypes.data, n.ctypes.data, n.shape[0], int(num_decode),
                                int(max_q_len), int(total_rows)))


def check_shared_prefix(pool: "KVPool", block_tables, seq_lens, num_prefix_blocks: int) -> None:
    """check_batch plus: every row starts with row 0's first num_prefix_blocks blocks."""
    t, n = _host(block_tables, np.int32), _host(seq_lens, np.int32)
    if t.ndim != 2 or n.shape != (t.shape[0],):
        raise ValueError("block_tables must be [S, maxB] and seq_lens [S]")
    check(lib().pa_check_shared_prefix(ctypes.byref(pool.c), t.ctypes.data, t.shape[1],
                                       n.ctypes.data, n.shape[0], int(num_prefix_blocks)))


def check_grouped(pool: "KVPool", block_tables, seq_lens, prefix_lens, group_size: int) -> None:
    """check_batch plus the shared-prefix precondition of decode_grouped (host check)."""
    t, n = _host(block_tables, np.int32), _host(seq_lens, np.int32)
    p = _host(prefix_lens, np.int32)
    if t.ndim != 2 or n.shape != (t.shape[0],) or p.shape != n.shape:
        raise ValueError("block_tables must be [S, maxB], seq_lens and prefix_lens [S]")
    check(lib().pa_check_grouped(ctypes.byref(pool.c), t.ctypes.data, t.shape[1], n.ctypes.data,
                                 p.ctypes.data, n.shape[0], int(group_size)))


def group_prefix_lens(block_tables, seq_lens, group_size: int, block_size: int) -> np.ndarray:
    """Tokens each group of group_size consecutive rows shares (host computation on
    host copies of the tables): int32 [S], equal within a group."""
    t, n = _host(block_tables, np.int32), _host(seq_lens, np.int32)
    if t.ndim != 2 or n.shape != (t.shape[0],):
        raise ValueError("block_tables must be [S, maxB] and seq_lens [S]")
    out = np.zeros(n.shape[0], dtype=np.int32)
    check(lib().pa_group_prefix_lens(t.ctypes.data, t.shape[1], n.ctypes.data, n.shape[0],
                                     int(group_size), int(block_size), out.ctypes.data))
    return out


def _need(t: torch.Tensor, name: str, dtype=None, device=True) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


class KVPool:
    """One layer's K and V pools: [num_blocks, num_kv_heads, block_size, head_dim].

    float8_e4m3fn pools hold E4M3 codes; a code c of K stands for e4m3(c) * k_scale
    (V likewise). New K/V are written, and queries and outputs given, in bfloat16."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, k_scale: float = 1.0,
                 v_scale: float = 1.0, host: bool = False):
        if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 4:
            raise ValueError("k and v pools must be 4-D with equal shape and dtype")
        if k.dtype not in _DTYPES:
            raise ValueError(f"pool dtype {k.dtype} not supported")
        _need(k, "k_pool", device=not host)
        _need(v, "v_pool", device=not host)
        if host and not (k.is_pinned() and v.is_pinned()):
            raise ValueError("a host pool (swap space) must be pinned host memory")
        self.host = host
        self.k, self.v = k, v
        nb, h, b, d = k.shape
        self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim = nb, h, b, d
        self.dtype = k.dtype
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.c = PaPool(k.data_ptr(), v.data_ptr(), nb, h, b, d, _DTYPES[k.dtype],
                        self.k_scale, self.v_scale)

    @property
    def io_dtype(self) -> torch.dtype:
        """dtype of new K/V, queries and outputs: the pool's, bf16 for an FP8 pool."""
        return torch.bfloat16 if self.dtype == torch.float8_e4m3fn else self.dtype

    @classmethod
    def empty(cls, num_blocks, num_kv_heads, block_size, head_dim, dtype, device="cuda",
              k_scale: float = 1.0, v_scale: float = 1.0):
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        return cls(torch.empty(shape, dtype=dtype, device=device),
                   torch.empty(shape, dtype=dtype, device=device), k_scale, v_scale)

    @classmethod
    def empty_host(cls, num_blocks, num_kv_heads, block_size, head_dim, dtype,
                   k_scale: float = 1.0, v_scale: float = 1.0):
        """A CPU swap space: a pool in pinned host memory the device can address."""
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        return cls(torch.empty(shape, dtype=dtype, pin_memory=True),
                   torch.empty(shape, dtype=dtype, pin_memory=True), k_scale, v_scale, host=True)

    @property
    def kv_bytes_per_token(self) -> int:
        return 2 * self.num_kv_heads * self.head_dim * self.k.element_size()


def cache_write(pool: KVPool, k_new: torch.Tensor, v_new: torch.Tensor,
                slot_mapping: torch.Tensor) -> None:
    """Store k_new/v_new [T, Hkv, D] at slots (int64 [T]; negative = skip)."""
    T = slot_mapping.numel()
    _need(slot_mapping, "slot_mapping", torch.int64)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, pool.io_dtype)
        if tuple(t.shape) != (T, pool.num_kv_heads, pool.head_dim):
            raise ValueError(f"{n} must be [{T}, {pool.num_kv_heads}, {pool.head_dim}]")
    if _CHECK_INPUTS:
        check_slots(pool, slot_mapping)
    check(lib().pa_cache_write(ctypes.byref(pool.c), k_new.data_ptr(), v_new.data_ptr(),
                               slot_mapping.data_ptr(), T, _stream()))


def copy_blocks(pool: KVPool, src_dst: torch.Tensor) -> None:
    """pool[dst] = pool[src] for each row of int32 [n, 2] (device)."""
    _need(src_dst, "src_dst", torch.int32)
    n = src_dst.shape[0] if src_dst.numel() else 0
    if src_dst.numel() and tuple(src_dst.shape) != (n, 2):
        raise ValueError("src_dst must be [n, 2]")
    if _CHECK_INPUTS and n:
        check_copies(pool, src_dst)
    check(lib().pa_copy_blocks(ctypes.byref(pool.c), _ptr(src_dst), n, _stream()))


PA_SWAP_OUT, PA_SWAP_IN = 0, 1


def swap_blocks(device_pool: KVPool, host_pool: KVPool, pairs, direction: int) -> None:
    """Move whole blocks between the device pool and a pinned host pool.
    pairs: host int32 [n, 2] of (src, dst); PA_SWAP_OUT copies device -> host,
    PA_SWAP_IN host -> device. Asynchronous on the current stream."""
    import numpy as np
    if device_pool.host or not host_pool.host:
        raise ValueError("swap_blocks takes a device pool and a host pool")
    if isinstance(pairs, torch.Tensor):
        if pairs.is_cuda:
            raise ValueError("pairs must be host memory")
        pairs = pairs.numpy()
    arr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    check(lib().pa_swap_blocks(ctypes.byref(device_pool.c), ctypes.byref(host_pool.c),
                               arr.ctypes.data if arr.size else None, arr.shape[0], int(direction),
                               _stream()))


def swap_out(device_pool: KVPool, host_pool: KVPool, pairs) -> None:
    """host_pool[dst] = device_pool[src] for each (src, dst)."""
    swap_blocks(device_pool, host_pool, pairs, PA_SWAP_OUT)


def swap_in(device_pool: KVPool, host_pool: KVPool, pairs) -> None:
    """device_pool[dst] = host_pool[src] for each (src, dst)."""
    swap_blocks(device_pool, host_pool, pairs, PA_SWAP_IN)


def probe_stream_read(buf: torch.Tensor, sink: torch.Tensor, grid: int = 0) -> None:
    """Read all of `buf` once (measurement aid: the device's streaming-read rate)."""
    _need(buf, "buf")
    _need(sink, "sink", torch.int32)
    check(lib().pa_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), grid,
                                     _ptr(sink), _stream()))


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           workers: int = 0) -> int:
    return int(lib().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                               workers))


def attention_mixed_workspace_bytes(num_decode: int, num_prefill: int, num_q_heads: int,
                                    num_kv_heads: int, head_dim: int, max_q_len: int,
                                    workers: int = 0) -> int:
    return int(lib().pa_attention_mixed_workspace_bytes(num_decode, num_prefill, num_q_heads,
                                                        num_kv_heads, head_dim, max_q_len,
                                                        workers))


class DecodePlan:
    """Output and workspace for repeated decode calls of one shape."""

    def __init__(self, pool: KVPool, num_seqs: int, num_q_heads: int, workers: int = 0):
        self.pool = pool
        self.num_seqs, self.num_q_heads, self.workers = num_seqs, num_q_heads, workers
        self.out = torch.empty((num_seqs, num_q_heads, pool.head_dim), dtype=pool.io_dtype,
                               device=pool.k.device)
        nbytes = decode_workspace_bytes(num_seqs, num_q_heads, pool.num_kv_heads, pool.head_dim,
                                        workers)
        self.workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=pool.k.device)


def decode(q: torch.Tensor, pool: KVPool, block_tables: torch.Tensor, seq_lens: torch.Tensor,
           scale: float, workers: int = 0, plan: Optional[DecodePlan] = None,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Paged decode attention. q [S, Hq, D]; block_tables int32 [S, maxB]; seq_lens int32 [S]."""
    _need(q, "q", pool.io_dtype)
    _need(block_tables, "block_tables", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    S, Hq, D = q.shape
    if D != pool.head_dim or block_tables.dim() != 2 or block_tables.shape[0] != S \
            or seq_lens.shape != (S,):
        raise ValueError("shape mismatch between q, block_tables and seq_lens")
    if _CHECK_INPUTS:
        check_batch(pool, block_tables, seq_lens)
    if plan is None:
        plan = DecodePlan(pool, S, Hq, workers)
    elif (plan.num_seqs, plan.num_q_heads, plan.workers, plan.pool) != (S, Hq, workers, pool):
        raise ValueError("plan does not match this call")
    if out is None:
        out = plan.out
    _need(out, "out", pool.io_dtype)
    ws = plan.workspace
    check(lib().pa_decode(out.data_ptr(), q.data_ptr(), ctypes.byref(pool.c),
                          block_tables.data_ptr(), block_tables.shape[1], seq_lens.data_ptr(), S,
                          Hq, float(scale), int(workers), ws.data_ptr(), ws.numel(), _stream()))
    return out


def decode_noalloc(q: torch.Tensor, pool: KVPool, block_tables: torch.Tensor,
                   seq_lens: torch.Tensor, scale: float, out: torch.Tensor,
                   workers: int = 0) -> torch.Tensor:
    """pa_decode_noalloc: decode with the library's static scratch array instead of a
    workspace; `out` [S, Hq, D] is the caller's (nothing is allocated here)."""
    _need(q, "q", pool.io_dtype)
    _need(block_tables, "block_tables", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(out, "out", pool.io_dtype)
    S, Hq, D = q.shape
    if D != pool.head_dim or block_tables.dim() != 2 or block_tables.shape[0] != S \
            or seq_lens.shape != (S,) or out.shape != q.shape:
        raise ValueError("shape mismatch between q, out, block_tables and seq_lens")
    if _CHECK_INPUTS:
        check_batch(pool, block_tables, seq_lens)
    check(lib().pa_decode_noalloc(out.data_ptr(), q.data_ptr(), ctypes.byref(pool.c),
                                  block_tables.data_ptr(), block_tables.shape[1],
                                  seq_lens.data_ptr(), S, Hq, float(scale), int(workers),
                                  _stream()))
    return out


def decode_noalloc_scratch_bytes() -> int:
    return int(lib().pa_decode_noalloc_scratch_bytes())


def decode_grouped_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                   head_dim: int, workers: int = 0) -> int:
    return int(lib().pa_decode_grouped_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                       head_dim, workers))


def decode_grouped(q: torch.Tensor, pool: KVPool, block_tables: torch.Tensor,
                   seq_lens: torch.Tensor, prefix_lens: torch.Tensor, group_size: int,
                   scale: float, workers: int = 0, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode for groups of ``group_size`` consecutive sequences whose first
    ``prefix_lens[s]`` tokens are the same blocks; those are read once per group."""
    _need(q, "q", pool.io_dtype)
    _need(block_tables, "block_tables", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(prefix_lens, "prefix_lens", torch.int32)
    S, Hq, D = q.shape
    if D != pool.head_dim or block_tables.dim() != 2 or block_tables.shape[0] != S \
            or seq_lens.shape != (S,) or prefix_lens.shape != (S,):
        raise ValueError("shape mismatch between q, block_tables, seq_lens and prefix_lens")
    if _CHECK_INPUTS:
        check_grouped(pool, block_tables, seq_lens, prefix_lens, group_size)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", pool.io_dtype)
    if workspace is None:
        n = decode_grouped_workspace_bytes(S, Hq, pool.num_kv_heads, D, workers)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    check(lib().pa_decode_grouped(out.data_ptr(), q.data_ptr(), ctypes.byref(pool.c),
                                  block_tables.data_ptr(), block_tables.shape[1],
                                  seq_lens.data_ptr(), prefix_lens.data_ptr(), S, int(group_size),
                                  Hq, float(scale), int(workers), workspace.data_ptr(),
                                  workspace.numel(), _stream()))
    return out


def decode_shared_prefix_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                         head_dim: int, block_size: int, num_prefix_blocks: int,
                                         workers: int = 0) -> int:
    return int(lib().pa_decode_shared_prefix_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_prefix_blocks, workers))


def decode_shared_prefix(q: torch.Tensor, pool: KVPool, block_tables: torch.Tensor,
                         seq_lens: torch.Tensor, num_prefix_blocks: int, scale: float,
                         workers: int = 0, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention for a batch whose table rows all start with the same
    ``num_prefix_blocks`` full blocks; the shared blocks are read once."""
    _need(q, "q", pool.io_dtype)
    _need(block_tables, "block_tables", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    S, Hq, D = q.shape
    if D != pool.head_dim or block_tables.dim() != 2 or block_tables.shape[0] != S \
            or seq_lens.shape != (S,):
        raise ValueError("shape mismatch between q, block_tables and seq_lens")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", pool.io_dtype)
    if workspace is None:
        n = decode_shared_prefix_workspace_bytes(S, Hq, pool.num_kv_heads, D, pool.block_size,
                                                 num_prefix_blocks, workers)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    if _CHECK_INPUTS:
        check_shared_prefix(pool, block_tables, seq_lens, num_prefix_blocks)
    check(lib().pa_decode_shared_prefix(out.data_ptr(), q.data_ptr(), ctypes.byref(pool.c),
                                        block_tables.data_ptr(), block_tables.shape[1],
                                        seq_lens.data_ptr(), S, Hq, float(scale),
                                        int(num_prefix_blocks), int(workers),
                                        workspace.data_ptr(), workspace.numel(), _stream()))
    return out


def attention_mixed(q: torch.Tensor, q_start_loc: torch.Tensor, seq_lens: torch.Tensor,
                    pool: KVPool, block_tables: torch.Tensor, num_decode: int, max_q_len: int,
                    scale: float, workers: int = 0, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Attention for a batch of ``num_decode`` decode sequences (one row each,
    first) followed by chunked-prefill sequences. q [rows, Hq, D];
    q_start_loc int32 [S+1] with q_start_loc[i] = i for i <= num_decode."""
    _need(q, "q", pool.io_dtype)
    _need(q_start_loc, "q_start_loc", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(block_tables, "block_tables", torch.int32)
    S = seq_lens.shape[0]
    if q_start_loc.shape != (S + 1,) or block_tables.shape[0] != S or not 0 <= num_decode <= S:
        raise ValueError("shape mismatch between q_start_loc, seq_lens, block_tables, num_decode")
    if q.shape[2] != pool.head_dim:
        raise ValueError("q head_dim does not match the pool")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", pool.io_dtype)
    if workspace is None:
        n = attention_mixed_workspace_bytes(int(num_decode), S - int(num_decode), q.shape[1],
                                            pool.num_kv_heads, pool.head_dim, int(max_q_len),
                                            workers)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    if _CHECK_INPUTS:
        check_batch(pool, block_tables, seq_lens)
        check_chunks(q_start_loc, seq_lens, num_decode, max_q_len, q.shape[0])
    check(lib().pa_attention_mixed(out.data_ptr(), q.data_ptr(), q_start_loc.data_ptr(),
                                   seq_lens.data_ptr(), ctypes.byref(pool.c),
                                   block_tables.data_ptr(), block_tables.shape[1], int(num_decode),
                                   S - int(num_decode), q.shape[1], int(max_q_len), float(scale),
                                   int(workers), workspace.data_ptr(), workspace.numel(), _stream()))
    return out


def prefill_chunk(q: torch.Tensor, q_start_loc: torch.Tensor, seq_lens: torch.Tensor,
                  pool: KVPool, block_tables: torch.Tensor, max_q_len: int, scale: float,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal chunked-prefill attention. q [rows, Hq, D] bf16; q_start_loc int32 [S+1]."""
    _need(q, "q", pool.dtype)
    _need(q_start_loc, "q_start_loc", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(block_tables, "block_tables", torch.int32)
    S = seq_lens.shape[0]
    if q_start_loc.shape != (S + 1,) or block_tables.shape[0] != S:
        raise ValueError("shape mismatch between q_start_loc, seq_lens and block_tables")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", pool.dtype)
    if _CHECK_INPUTS:
        check_batch(pool, block_tables, seq_lens)
        check_chunks(q_start_loc, seq_lens, 0, max_q_len, q.shape[0])
    check(lib().pa_prefill_chunk(out.data_ptr(), q.data_ptr(), q_start_loc.data_ptr(),
                                 seq_lens.data_ptr(), ctypes.byref(pool.c),
                                 block_tables.data_ptr(), block_tables.shape[1], S, q.shape[1],
                                 int(max_q_len), float(scale), _stream()))
    return out


__all__ = ["KVPool", "DecodePlan", "attention_mixed", "cache_write", "check_batch", "check_chunks",
           "check_copies", "check_shared_prefix", "check_slots", "copy_blocks", "decode",
           "decode_noalloc", "decode_noalloc_scratch_bytes", "decode_grouped",
           "decode_grouped_workspace_bytes", "check_grouped", "group_prefix_lens",
           "set_input_checks",
           "decode_workspace_bytes", "decode_shared_prefix", "decode_shared_prefix_workspace_bytes",
           "prefill_chunk", "swap_blocks", "swap_in", "swap_out", "PA_SWAP_IN", "PA_SWAP_OUT",
           "PagedKVError"]
