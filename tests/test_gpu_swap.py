"""GPU parity of the block swap (pa_swap_blocks) against the oracle's swap:
bit-exact over the whole destination pool, in both directions, for each pool
dtype, across several launches (more than 256 pairs), and a decode after a
swap out / swap in round trip that lands the blocks at other ids."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_316_amd as pkv
import workloads
from oracle.paging import PoolMirror, swap

from gpu_util import Loaded, pool_bits

pytestmark = pytest.mark.gpu

BITS = {torch.float32: (np.uint32, torch.int32, 0x7FC00001),
        torch.bfloat16: (np.uint16, torch.int16, 0x7FC1),
        torch.float8_e4m3fn: (np.uint8, torch.uint8, 0x7F)}


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()


def _mirror(t_k, t_v):
    """Host mirror holding the pools' current bits."""
    k, v = pool_bits(t_k), pool_bits(t_v)
    m = PoolMirror(k.shape[0], k.shape[1], k.shape[2], k.shape[3], k.dtype)
    m.k[...] = k
    m.v[...] = v
    return m


def _random_pool(nb, H, B, D, dtype, seed, host=False):
    nbits, ibits, _ = BITS[dtype]
    g = torch.Generator().manual_seed(seed)
    shape = (nb, H, B, D)
    lo, hi = (0, 255) if ibits == torch.uint8 else (-(1 << 15), (1 << 15) - 1)
    if ibits == torch.int32:
        lo, hi = -(1 << 30), 1 << 30
    k = torch.randint(lo, hi, shape, generator=g, dtype=ibits).view(dtype)
    v = torch.randint(lo, hi, shape, generator=g, dtype=ibits).view(dtype)
    if host:
        pool = pkv.KVPool.empty_host(nb, H, B, D, dtype, 0.5, 0.25)
        pool.k.copy_(k)
        pool.v.copy_(v)
        return pool
    return pkv.KVPool(k.cuda(), v.cuda(), 0.5, 0.25)


def _pairs(rng, n, n_src, n_dst):
    return np.stack([rng.integers(0, n_src, n), rng.permutation(n_dst)[:n]], 1).astype(np.int32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float8_e4m3fn])
@pytest.mark.parametrize("n", [1, 7, 300, 520])
def test_swap_out_and_in_bit_exact(dtype, n):
    """Swap out n device blocks to a host pool, then swap in n host blocks to
    the device: both destination pools equal the oracle's, every byte."""
    H, B, D = 4, 16, 128
    nd, nh = 600, 700
    rng = np.random.default_rng(n)
    _note(f"swap {dtype} n={n}")
    dev = _random_pool(nd, H, B, D, dtype, seed=1)
    host = _random_pool(nh, H, B, D, dtype, seed=2, host=True)
    pairs = _pairs(rng, n, nd, nh)
    want_host = _mirror(host.k, host.v)
    swap(want_host, _mirror(dev.k, dev.v), pairs)
    pkv.swap_out(dev, host, pairs)
    torch.cuda.synchronize()
    got = _mirror(host.k, host.v)
    assert np.array_equal(got.k, want_host.k) and np.array_equal(got.v, want_host.v)
    # and back: n host blocks into device blocks
    in_pairs = _pairs(rng, n, nh, nd)
    want_dev = _mirror(dev.k, dev.v)
    swap(want_dev, got, in_pairs)
    pkv.swap_in(dev, host, in_pairs)
    torch.cuda.synchronize()
    got_dev = _mirror(dev.k, dev.v)
    assert np.array_equal(got_dev.k, want_dev.k) and np.array_equal(got_dev.v, want_dev.v)


def test_round_trip_then_decode_bitwise():
    """Preempt every sequence of a workload by swapping its blocks out, reuse
    the device blocks (overwritten with NaN), swap them back in at other ids and
    decode through the remapped tables: bitwise the output before the swap."""
    wl = workloads.make("llama13b", "small")
    g = Loaded(wl)
    base = g.decode()
    tables = g.tables.cpu().numpy()
    lens = g.lens.cpu().numpy()
    used = sorted({int(b) for i, L in enumerate(lens) for b in tables[i, :-(-int(L) // wl.block_size)]})
    host = pkv.KVPool.empty_host(len(used) + 3, wl.num_kv_heads, wl.block_size, wl.head_dim,
                                 torch.bfloat16)
    slot = {b: j + 2 for j, b in enumerate(used)}  # host ids, offset
    pkv.swap_out(g.pool, host, [(b, slot[b]) for b in used])
    torch.cuda.synchronize()
    g.pool.k.fill_(float("nan")); g.pool.v.fill_(float("nan"))
    rng = np.random.default_rng(3)
    new_id = dict(zip(used, rng.permutation(wl.num_blocks)[:len(used)].tolist()))
    pkv.swap_in(g.pool, host, [(slot[b], new_id[b]) for b in used])
    remap = np.vectorize(lambda b: new_id.get(int(b), 0))(tables).astype(np.int32)
    out = g.decode(tables=torch.from_numpy(remap).cuda())
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


def test_pageable_host_memory_is_refused():
    """A host pool in pageable memory is refused before any launch. The lookup
    the library relies on is checked first with HIP directly (a host call)."""
    arr = np.zeros((4, 2, 16, 128), dtype=np.uint16)
    hip = ctypes.CDLL("libamdhip64.so")

    class Attr(ctypes.Structure):
        _fields_ = [("type", ctypes.c_int), ("device", ctypes.c_int),
                    ("devicePointer", ctypes.c_void_p), ("hostPointer", ctypes.c_void_p),
                    ("isManaged", ctypes.c_int), ("allocationFlags", ctypes.c_uint)]
    a = Attr()
    e = hip.hipPointerGetAttributes(ctypes.byref(a), ctypes.c_void_p(arr.ctypes.data))
    hip.hipGetLastError()
    if e == 0 and a.type == 1 and a.devicePointer:
        pytest.skip("HIP reports this pageable buffer as mapped host memory")
    dev = pkv.KVPool.empty(4, 2, 16, 128, torch.bfloat16)
    from paged_kv_cache_316_amd._lib import PaPool, lib
    host_c = PaPool(arr.ctypes.data, arr.ctypes.data, 4, 2, 16, 128, 1, 1.0, 1.0)
    pairs = (ctypes.c_int32 * 2)(0, 1)
    L = lib()
    st = L.pa_swap_blocks(ctypes.byref(dev.c), ctypes.byref(host_c), pairs, 1, 0, None)
    assert st == -1 and b"host" in L.pa_last_error()
    with pytest.raises(ValueError):
        pkv.KVPool(torch.zeros(4, 2, 16, 128, dtype=torch.bfloat16),
                   torch.zeros(4, 2, 16, 128, dtype=torch.bfloat16), host=True)
