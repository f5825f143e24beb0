"""GPU parity of pa_attention_mixed's multi-row path against the fp64 oracle:
batches whose chunks are short (max_q_len x query heads per KV head <= 32, a
bf16 pool) run as one multi-row decode over every sequence, decode rows
included; each (row, query head) column attends causally up to its own
row's position; units of more than 16 columns run on a pair of waves that
share each K/V tile, smaller ones on one wave. Cases: speculative-verification
shapes (a few draft rows per sequence) for groups of 8, 4, 2 and 1 query
heads, head_dim 64 and 128, both launch shapes, bf16 and FP8 pools,
blocks of 4 to 64 tokens, chunks without rows, decode rows mixed in, every
split of the work between wavefronts, and the Llama-2-70B-shaped workload
(small, and full size with every row compared).
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_316_amd as pkv
import workloads
from oracle import fp8
from oracle.attention import prefill_attention
from oracle.expected import logical_kv

from gpu_util import Loaded, assert_close, full_workload, out_f64
from test_gpu_mixed import _ragged

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


class _Bf16:
    dtype = "bf16"


def _run(case, workers=0, seed=None):
    Hq, Hkv, D, B, dl, chunks = case
    q_lens = [1] * len(dl) + [c[0] for c in chunks]
    L = list(dl) + [c[1] for c in chunks]
    max_q = max([c[0] for c in chunks], default=0)
    assert max_q * (Hq // Hkv) <= 32, "case must take the multi-row path"
    dev, want = _ragged(Hq, Hkv, D, B, q_lens, L, seed=sum(L) if seed is None else seed)
    nd = len(dl)
    out = torch.full_like(dev["q"], float("nan"))  # a row left unwritten shows up as NaN
    pkv.attention_mixed(dev["q"], dev["loc"], dev["lens"], dev["pool"], dev["tables"], nd, max_q,
                        1 / np.sqrt(D), workers, out=out)
    torch.cuda.synchronize()
    return assert_close(_Bf16, out_f64(out), want, f"{case} workers={workers}")


CASES = {
    # Hq, Hkv, D, B, decode lengths, (rows, length) of the short chunks
    "g8_k4": (64, 8, 128, 16, [5, 900], [(4, 300), (4, 4), (2, 1000), (3, 513), (1, 17), (0, 40)]),
    "g8_k4_only": (16, 2, 128, 16, [], [(4, 64), (4, 2048), (4, 5), (2, 2)]),
    "g4_k8": (32, 8, 128, 16, [33], [(8, 8), (8, 129), (5, 700), (7, 16)]),
    "g2_k16_b4": (8, 4, 128, 4, [1, 63], [(16, 200), (9, 16), (16, 33)]),
    "g1_k32_d64_b8": (16, 16, 64, 8, [2, 300], [(32, 32), (32, 1100), (17, 40), (1, 1)]),
    "g1_k32_d128": (4, 4, 128, 16, [], [(32, 640), (31, 31), (5, 6)]),
    "g8_b64": (16, 2, 128, 64, [70], [(4, 256), (3, 130), (4, 64)]),
    "g8_d64_b32": (16, 2, 64, 32, [1], [(4, 97), (2, 2)]),
    # at most 16 columns per unit: one wave per unit instead of a pair
    "g8_k2": (64, 8, 128, 16, [5, 900], [(2, 300), (2, 4), (1, 1000), (2, 513), (0, 40)]),
    "g4_k3_b8": (16, 4, 128, 8, [33], [(3, 129), (1, 700), (3, 16)]),
    "g1_k16_d64": (8, 8, 64, 16, [2], [(16, 64), (9, 300), (16, 16)]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_short_chunks(name):
    print(f"multi-row {name}: {_run(CASES[name])}", flush=True)


def _ragged_fp8(Hq, Hkv, D, B, q_lens, L, seed, ksc=2.0 ** -6, vsc=0.0123):
    """A batch like _ragged's over an FP8 pool: bf16 draws, quantized by the
    cache write; the oracle attends over the values the codes stand for.
    Sequence s holds L[s] tokens in reverse block order."""
    rng = np.random.default_rng(seed)
    nbs = [-(-l // B) for l in L]
    nb = sum(nbs) + 2
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.zeros((len(L), max(nbs)), dtype=np.int32)
    ks, vs, slots = [], [], []
    at = 0
    for s, n in enumerate(nbs):
        tables[s, :n] = perm[at:at + n][::-1]
        at += n
        t = np.arange(L[s])
        slots.append(tables[s, t // B].astype(np.int64) * B + t % B)
        ks.append(torch.from_numpy(rng.standard_normal((L[s], Hkv, D)).astype(np.float32)).bfloat16())
        vs.append(torch.from_numpy(rng.standard_normal((L[s], Hkv, D)).astype(np.float32)).bfloat16())
    pool = pkv.KVPool.empty(nb, Hkv, B, D, torch.float8_e4m3fn, k_scale=ksc, v_scale=vsc)
    pool.k.view(torch.uint8).fill_(0x7F); pool.v.view(torch.uint8).fill_(0x7F)  # NaN codes
    pkv.cache_write(pool, torch.cat(ks).cuda(), torch.cat(vs).cuda(),
                    torch.from_numpy(np.concatenate(slots)).cuda())
    q = torch.from_numpy(rng.standard_normal((sum(q_lens), Hq, D)).astype(np.float32)).bfloat16()
    loc = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    qd = q.double().numpy()
    want = []
    for s in range(len(L)):
        kk = fp8.dequantize(fp8.quantize(ks[s].float().numpy(), ksc), ksc)
        vv = fp8.dequantize(fp8.quantize(vs[s].float().numpy(), vsc), vsc)
        if q_lens[s]:
            want.append(prefill_attention(qd[loc[s]:loc[s + 1]], kk, vv, L[s] - q_lens[s],
                                          1 / np.sqrt(D)))
    dev = dict(q=q.cuda(), loc=torch.from_numpy(loc).cuda(), pool=pool,
               lens=torch.tensor(L, dtype=torch.int32, device="cuda"),
               tables=torch.from_numpy(tables).cuda())
    return dev, np.concatenate(want)


FP8_CASES = {
    # Hq, Hkv, D, B, decode lengths, (rows, length) of the short chunks
    "fp8_g8_k4": (64, 8, 128, 16, [5, 900], [(4, 300), (4, 4), (2, 1000), (3, 513), (1, 17), (0, 40)]),
    "fp8_g1_k32_b8": (4, 4, 128, 8, [], [(32, 640), (31, 31), (5, 6)]),
    "fp8_g8_k2": (16, 2, 128, 16, [33], [(2, 64), (2, 700), (1, 5)]),
    "fp8_g4_k4_d64": (16, 4, 64, 16, [1], [(4, 97), (2, 300), (4, 4)]),
}


@pytest.mark.parametrize("name", list(FP8_CASES))
@pytest.mark.parametrize("workers", [0, 7])
def test_short_chunks_fp8(name, workers):
    """Multi-row decode over FP8 codes (widened exactly to bf16 in LDS; k_scale
    folded into the softmax scale, v_scale into the output)."""
    Hq, Hkv, D, B, dl, chunks = FP8_CASES[name]
    q_lens = [1] * len(dl) + [c[0] for c in chunks]
    L = list(dl) + [c[1] for c in chunks]
    max_q = max(c[0] for c in chunks)
    dev, want = _ragged_fp8(Hq, Hkv, D, B, q_lens, L, seed=sum(L))
    out = torch.full_like(dev["q"], float("nan"))
    pkv.attention_mixed(dev["q"], dev["loc"], dev["lens"], dev["pool"], dev["tables"], len(dl),
                        max_q, 1 / np.sqrt(D), workers, out=out)
    torch.cuda.synchronize()
    print(f"multi-row {name} workers={workers}: "
          f"{assert_close(_Bf16, out_f64(out), want, name)}", flush=True)


def test_fp8_d64_beyond_16_columns_is_refused():
    """FP8 rows of 64 dims fill a tile with one wave-wide load, so a pair of
    waves cannot share it: more than 16 columns per unit is refused (on the
    host, before any launch) rather than sent to the bf16-only prefill kernel."""
    dev, _ = _ragged_fp8(8, 2, 64, 16, [8], [40], seed=3)
    with pytest.raises(pkv.PagedKVError, match="bf16"):
        pkv.attention_mixed(dev["q"], dev["loc"], dev["lens"], dev["pool"], dev["tables"], 0, 8,
                            0.125)


@pytest.mark.parametrize("workers", [1, 5, 64, 1000])
@pytest.mark.parametrize("name", ["g8_k4", "g8_k2"])
def test_worker_splits(name, workers):
    """Units split between work slices (pairs of waves for g8_k4, single
    waves for g8_k2) at any tile recombine to the same rows."""
    _run(CASES[name], workers=workers)


def _verify_llama70b(wl, k=4):
    """Every sequence of the Llama-2-70B-shaped batch verifies k draft tokens
    (its last k positions as causal rows), in the launch the bench times."""
    g = Loaded(wl)
    S = len(wl.decode_seqs)
    _note(f"llama70b {S} sequences x {k} rows")
    rng = np.random.default_rng(99)
    q = torch.from_numpy(rng.standard_normal((S * k, wl.num_q_heads, wl.head_dim))
                         .astype(np.float32)).to(torch.bfloat16)
    loc = torch.arange(0, S * k + 1, k, dtype=torch.int32, device="cuda")
    out = torch.full((S * k, wl.num_q_heads, wl.head_dim), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    pkv.attention_mixed(q.cuda(), loc, g.lens, g.pool, g.tables, 0, k, wl.scale, out=out)
    torch.cuda.synchronize()
    lens = g.lens.cpu().numpy()
    qd = q.double().numpy()
    want = []
    for i in range(S):
        K, V = logical_kv(wl, wl.decode_seqs[i])
        L = int(lens[i])
        want.append(prefill_attention(qd[i * k:(i + 1) * k], K[:L], V[:L], L - k, wl.scale))
    return assert_close(wl, out_f64(out), np.concatenate(want), "spec verify")


def _note(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name", ["llama70b", "llama70b_fp8"])
def test_llama70b_speculative_verification_small(name):
    _note(f"  {_verify_llama70b(workloads.make(name, 'small'))}")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["llama70b", "llama70b_fp8"])
def test_llama70b_speculative_verification_full_every_row(name):
    _note(f"  {_verify_llama70b(full_workload(name))}")
