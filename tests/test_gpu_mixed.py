"""GPU parity of the mixed prefill + decode call (pa_attention_mixed) against
the fp64 oracle. The batch is one scheduler step of the Llama-2-70B-shaped
workload: the sequences that take a prefill chunk in this step contribute
their chunk rows, every other sequence its decode row. Bars as for decode and
prefill (bf16: rtol 2e-2 / atol 5e-3 per element)."""

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_316_amd as pkv
import workloads
from oracle.attention import prefill_attention
from oracle.expected import decode_out, prefill_out

from gpu_util import (Loaded, assert_close, full_decode_out, full_prefill_out, full_workload, out_f64,
                      to_device)

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()


def _step_batch(g, wl):
    """Decode sequences first (those without a chunk this step), then the chunks."""
    C = wl.prefill_len
    pre = [wl.decode_seqs.index(s) for s in wl.prefill_seqs]
    dec = [i for i in range(len(wl.decode_seqs)) if i not in pre]
    nd = len(dec)
    dec_t = torch.tensor(dec, device="cuda", dtype=torch.long)
    pre_t = torch.tensor(pre, device="cuda", dtype=torch.long)
    q = torch.cat([g.q[dec_t], to_device(wl, wl.prefill_q)]).contiguous()
    loc = torch.tensor(list(range(nd + 1)) + [nd + C * (j + 1) for j in range(len(pre))],
                       dtype=torch.int32, device="cuda")
    p_lens = torch.tensor([int(wl.prefill_start[j]) + C for j in range(len(pre))],
                          dtype=torch.int32, device="cuda")
    lens = torch.cat([g.lens[dec_t], p_lens]).contiguous()
    tables = torch.cat([g.tables[dec_t], g.tables[pre_t]]).contiguous()
    return dict(q=q, loc=loc, lens=lens, tables=tables, nd=nd, dec=dec, C=C)


def test_mixed_step_small():
    wl = workloads.make("llama70b", "small")
    g = Loaded(wl)
    b = _step_batch(g, wl)
    _note(f"mixed step: llama70b small, {b['nd']} decode rows + {len(wl.prefill_seqs)} chunks")
    out = pkv.attention_mixed(b["q"], b["loc"], b["lens"], g.pool, b["tables"], b["nd"], b["C"],
                              wl.scale)
    torch.cuda.synchronize()
    got = out_f64(out)
    nd = b["nd"]
    s1 = assert_close(wl, got[:nd], decode_out(wl, b["dec"]), "decode rows")
    s2 = assert_close(wl, got[nd:], prefill_out(wl), "prefill rows")
    _note(f"  decode {s1}  prefill {s2}")
    # the same kernels as the separate calls: bitwise the same rows, given the
    # decode the same number of work slices (beside chunks the mixed call
    # defaults to 2 per compute unit, the plain decode to 8)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    d = pkv.decode(b["q"][:nd].contiguous(), g.pool, b["tables"][:nd].contiguous(),
                   b["lens"][:nd].contiguous(), wl.scale, workers=2 * cus)
    p = pkv.prefill_chunk(b["q"][nd:].contiguous(), (b["loc"][nd:] - nd).contiguous(),
                          b["lens"][nd:].contiguous(), g.pool, b["tables"][nd:].contiguous(),
                          b["C"], wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(out[:nd].view(torch.int16), d.view(torch.int16))
    assert torch.equal(out[nd:].view(torch.int16), p.view(torch.int16))


@pytest.mark.slow
def test_mixed_step_full_every_row():
    """One step of the Llama-2-70B batch (248 decode rows, 8 chunks of 512):
    every decode row and every chunk row against the oracle."""
    wl = full_workload("llama70b")
    g = Loaded(wl)
    b = _step_batch(g, wl)
    nd, C = b["nd"], b["C"]
    _note(f"mixed step: llama70b full, {nd} decode rows + {len(wl.prefill_seqs)} chunks of {C}")
    out = out_f64(pkv.attention_mixed(b["q"], b["loc"], b["lens"], g.pool, b["tables"], nd, C,
                                      wl.scale))
    stats = assert_close(wl, out[:nd], full_decode_out("llama70b")[b["dec"]], "decode rows")
    _note(f"  decode rows: {stats}")
    stats = assert_close(wl, out[nd:], full_prefill_out("llama70b"), "prefill rows")
    _note(f"  prefill rows: {stats}")


def _ragged(Hq, Hkv, D, B, q_lens, L, seed, dtype=torch.bfloat16, n_decode=0):
    """n_decode single-row sequences then chunks of the given lengths; each
    sequence holds L[s] tokens in reverse block order."""
    rng = np.random.default_rng(seed)
    S = len(L)
    nbs = [-(-l // B) for l in L]
    nb = sum(nbs) + 2
    perm = rng.permutation(nb).astype(np.int32)
    maxb = max(nbs)
    tables = np.zeros((S, maxb), dtype=np.int32)
    ks, vs, slots = [], [], []
    nxt = 0
    for s in range(S):
        tables[s, :nbs[s]] = perm[nxt:nxt + nbs[s]][::-1]
        nxt += nbs[s]
        t = np.arange(L[s])
        slots.append(tables[s, t // B].astype(np.int64) * B + t % B)
        ks.append(rng.standard_normal((L[s], Hkv, D)).astype(np.float32))
        vs.append(rng.standard_normal((L[s], Hkv, D)).astype(np.float32))
    k = torch.from_numpy(np.concatenate(ks)).to(dtype)
    v = torch.from_numpy(np.concatenate(vs)).to(dtype)
    pool = pkv.KVPool.empty(nb, Hkv, B, D, dtype)
    pool.k.fill_(float("nan")); pool.v.fill_(float("nan"))
    pkv.cache_write(pool, k.cuda(), v.cuda(), torch.from_numpy(np.concatenate(slots)).cuda())
    rows = sum(q_lens)
    q = torch.from_numpy(rng.standard_normal((rows, Hq, D)).astype(np.float32)).to(dtype)
    loc = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    want = []
    kk = np.split(k.double().numpy(), np.cumsum(L)[:-1])
    vv = np.split(v.double().numpy(), np.cumsum(L)[:-1])
    qd = q.double().numpy()
    for s in range(S):
        for i in range(q_lens[s]):
            pos = L[s] - q_lens[s] + i
            want.append(prefill_attention(qd[loc[s] + i:loc[s] + i + 1], kk[s][:pos + 1],
                                          vv[s][:pos + 1], pos, 1 / np.sqrt(D))[0])
    dev = dict(q=q.cuda(), loc=torch.from_numpy(loc).cuda(), pool=pool,
               lens=torch.tensor(L, dtype=torch.int32, device="cuda"),
               tables=torch.from_numpy(tables).cuda())
    return dev, np.stack(want)


class _Bf16:
    dtype = "bf16"


@pytest.mark.parametrize("case", [
    # Hq, Hkv, D, B, decode lengths, (chunk rows, lengths)
    (8, 1, 128, 16, [1, 40, 700], [(1, 33), (17, 17), (100, 300)]),
    (16, 16, 64, 4, [5, 1000], [(64, 64), (3, 90)]),
    (6, 2, 128, 32, [], [(50, 50), (129, 260)]),              # chunks only
    (12, 4, 64, 8, [9, 19, 1, 333], []),                      # decode rows only
    # speculative-decoding verification: a few draft rows per sequence
    (16, 2, 128, 16, [70], [(4, 300), (5, 77), (2, 1000), (8, 8), (3, 513), (6, 6)]),
    (8, 8, 128, 16, [], [(2, 2), (7, 129), (4, 2048)]),
])
def test_mixed_ragged(case):
    Hq, Hkv, D, B, dl, chunks = case
    q_lens = [1] * len(dl) + [c[0] for c in chunks]
    L = list(dl) + [c[1] for c in chunks]
    _note(f"mixed ragged {case}")
    dev, want = _ragged(Hq, Hkv, D, B, q_lens, L, seed=sum(L))
    nd = len(dl)
    max_q = max([c[0] for c in chunks], default=0)
    out = pkv.attention_mixed(dev["q"], dev["loc"], dev["lens"], dev["pool"], dev["tables"], nd,
                              max_q, 1 / np.sqrt(D))
    torch.cuda.synchronize()
    assert_close(_Bf16, out_f64(out), want, f"{case}")
