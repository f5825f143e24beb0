"""GPU parity of pa_attention_mixed's multi-row path against the fp64 oracle:
batches whose chunks are short (max_q_len x query heads per KV head <= 32, a
bf16 pool) run as one multi-row decode over every sequence, decode rows
included; each (row, query head) column attends causally up to its own
row's position; units of more than 16 columns run on a pair of waves that
share each K/V tile, smaller ones on one wave. Cases: speculative-verification
shapes (a few draft rows per sequence) for groups of 8, 4, 2 and 1 query
heads, head_dim 64 and 128, both launch shapes,
blocks of 4 to 64 tokens, chunks without rows, decode rows mixed in, every
split of the work between wavefronts, and the Llama-2-70B-shaped workload
(small, and full size with every row compared).
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_316_amd as pkv
import workloads
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


def test_llama70b_speculative_verification_small():
    _note(f"  {_verify_llama70b(workloads.make('llama70b', 'small'))}")


@pytest.mark.slow
def test_llama70b_speculative_verification_full_every_row():
    _note(f"  {_verify_llama70b(full_workload('llama70b'))}")
