"""The library's calls under HIP graph capture: a decode step (cache write +
decode), the shared-prefix decode and a mixed prefill + decode step are
captured once and replayed several times, with eager work and synchronisation
between replays; every replay must give the eager result bit for bit. The
calls allocate nothing and record no memset, so they capture as they are; the
mixed and shared-prefix calls fork to and join from the library's second
stream inside the capture."""

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_316_amd as pkv
import workloads
from paged_kv_cache_316_amd.runner import WriteBatch

from gpu_util import Loaded, to_device

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()


def _replays(fn, out, n=4):
    """Eager result, then the captured call replayed n times with eager work
    (a decoy fill of `out`, a host sync) before each replay."""
    fn()
    torch.cuda.synchronize()
    want = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for i in range(n):
        out.fill_(float(i + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {i}"


def test_decode_step_in_a_graph():
    wl = workloads.make("llama13b", "small")
    g = Loaded(wl, upto_decode=True)
    dec = g.phases["decode"]
    w = [e for e in dec if e[0] == "write"]
    batch = WriteBatch(np.concatenate([e[1] for e in w]), np.concatenate([e[2] for e in w]),
                       g.rows_k, g.rows_v)
    plan = pkv.DecodePlan(g.pool, len(wl.decode_seqs), wl.num_q_heads)
    _note("graph: cache write + decode, llama13b small")

    def step():
        batch.run(g.pool)
        pkv.decode(g.q, g.pool, g.tables, g.lens, wl.scale, plan=plan)
    _replays(step, plan.out)


def test_shared_prefix_decode_in_a_graph():
    wl = workloads.make("prefix", "small")
    g = Loaded(wl)
    P = wl.meta["prefix_tokens"] // wl.block_size
    out = torch.empty_like(g.q)
    n = pkv.decode_shared_prefix_workspace_bytes(len(wl.decode_seqs), wl.num_q_heads,
                                                 wl.num_kv_heads, wl.head_dim, wl.block_size, P)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    _note("graph: shared-prefix decode, prefix small")
    _replays(lambda: pkv.decode_shared_prefix(g.q, g.pool, g.tables, g.lens, P, wl.scale,
                                              out=out, workspace=ws), out)


def test_mixed_step_in_a_graph():
    wl = workloads.make("llama70b", "small")
    g = Loaded(wl)
    C = wl.prefill_len
    pre = [wl.decode_seqs.index(x) for x in wl.prefill_seqs]
    dec = [i for i in range(len(wl.decode_seqs)) if i not in pre]
    nd = len(dec)
    order = torch.tensor(dec + pre, device="cuda")
    q = torch.cat([g.q[order[:nd]], to_device(wl, wl.prefill_q)]).contiguous()
    loc = torch.tensor(list(range(nd + 1)) + [nd + C * (j + 1) for j in range(len(pre))],
                       dtype=torch.int32, device="cuda")
    p_lens = torch.tensor([int(wl.prefill_start[j]) + C for j in range(len(pre))],
                          dtype=torch.int32, device="cuda")
    lens = torch.cat([g.lens[order[:nd]], p_lens]).contiguous()
    tables = g.tables[order].contiguous()
    out = torch.empty_like(q)
    ws = torch.empty(pkv.decode_workspace_bytes(nd, wl.num_q_heads, wl.num_kv_heads,
                                                wl.head_dim), dtype=torch.uint8, device="cuda")
    _note("graph: mixed step, llama70b small")
    _replays(lambda: pkv.attention_mixed(q, loc, lens, g.pool, tables, nd, C, wl.scale, out=out,
                                         workspace=ws), out)
