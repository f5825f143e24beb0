"""pa_decode_noalloc (decode with the library's static scratch array, for
callers that cannot allocate) against pa_decode, through the C ABI.

Both run the same kernels with the same worker count, so the outputs must be
bitwise equal; they are also held to the oracle's bar. Two calls in a row on
the shared array, the second with a smaller batch, must each match pa_decode
on the same input. A call needing more scratch than the array holds is
refused with nothing queued, and the next call still works."""

import numpy as np
import pytest
import torch

import paged_kv_cache_316_amd as pkv
import workloads
from oracle.expected import decode_out

from gpu_util import Loaded, assert_close, out_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("workers", [0, 7])
@pytest.mark.parametrize("name", ["llama70b", "llama13b", "llama13b_fp8", "tiny"])
def test_noalloc_matches_decode_twice_then_smaller(name, workers):
    wl = workloads.make(name, "small")
    print(f"noalloc: {name} small, workers={workers}", flush=True)
    g = Loaded(wl)
    S = len(wl.decode_seqs)
    want_full = decode_out(wl)
    # call 1: the whole batch; call 2: the same batch again; call 3: a smaller
    # batch (the second half of the sequences) on the array the earlier calls left
    for rows in (slice(0, S), slice(0, S), slice(S // 2, S)):
        q = g.q[rows].contiguous()
        tables = g.tables[rows].contiguous()
        lens = g.lens[rows].contiguous()
        ref = pkv.decode(q, g.pool, tables, lens, wl.scale, workers=workers).clone()
        out = torch.full_like(q, float("nan"))
        pkv.decode_noalloc(q, g.pool, tables, lens, wl.scale, out, workers=workers)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), f"{name}: differs from pa_decode"
        assert_close(wl, out_f64(out), want_full[rows], f"{name} noalloc rows {rows}")


def test_noalloc_refuses_oversized_calls_and_recovers():
    wl = workloads.make("llama70b", "small")
    g = Loaded(wl)
    S = len(wl.decode_seqs)
    cap = pkv.decode_noalloc_scratch_bytes()
    huge = 1
    while pkv.decode_workspace_bytes(S, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, huge) <= cap:
        huge *= 2
    out = torch.zeros_like(g.q)
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.decode_noalloc(g.q, g.pool, g.tables, g.lens, wl.scale, out, workers=huge)
    assert e.value.status == -5 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.float()) == 0  # nothing was queued
    pkv.decode_noalloc(g.q, g.pool, g.tables, g.lens, wl.scale, out)
    torch.cuda.synchronize()
    assert_close(wl, out_f64(out), decode_out(wl), "after a refused call")
