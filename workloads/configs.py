"""The seeded workloads.

Each workload is drawn from ``np.random.default_rng(seed)`` in a fixed order:
structure (lengths, tails, beam parent picks, prefill picks), then the
free-list permutation, then token ids, then K rows, V rows, decode queries and
prefill queries. Values are N(0, 1) float32, rounded once to the storage
dtype. The shapes follow the workloads the pages discuss (LLaMA-13B with 40
heads of 128, Llama-2-70B with 64 query / 8 KV heads of 128, block size 16,
the 4-token-block walk-through); no dataset, trace or weights are used.

Sizes: "full" is the workload as specified; "small" keeps every structural
feature (ragged lengths, partial last blocks, sharing, copies, GQA, prefill)
at sizes the fp64 oracle finishes in well under a second.
"""

from __future__ import annotations

import math
from typing import Callable, Dict, List

import numpy as np

from .data import Workload, f32_to_bf16_bits

VOCAB = 32000


class _Rows:
    """Hands out consecutive row ids; rows are drawn after the structure."""

    def __init__(self) -> None:
        self.n = 0

    def take(self, k: int) -> np.ndarray:
        r = np.arange(self.n, self.n + k, dtype=np.int64)
        self.n += k
        return r


def _draw_values(rng: np.random.Generator, shape, dtype: str, data_scale: float = 1.0):
    """N(0,1) float32 draws (times ``data_scale``) in C order, stored as ``dtype``.

    Drawn in fixed chunks through one reused buffer, so a multi-GB draw touches
    fresh memory only for its output.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    chunk = 1 << 22
    buf = np.empty(min(n, chunk), dtype=np.float32)
    ubuf = buf.view(np.uint32)
    tmp = np.empty_like(ubuf)
    for a in range(0, n, chunk):
        m = min(chunk, n - a)
        x = buf[:m]
        rng.standard_normal(out=x, dtype=np.float32)
        if data_scale != 1.0:
            x *= np.float32(data_scale)
        if dtype == "f32":
            out[a:a + m] = x
        else:  # round to nearest even bfloat16, as f32_to_bf16_bits does
            u, t = ubuf[:m], tmp[:m]
            np.right_shift(u, np.uint32(16), out=t)
            np.bitwise_and(t, np.uint32(1), out=t)
            np.add(t, np.uint32(0x7FFF), out=t)
            np.add(u, t, out=u)
            np.right_shift(u, np.uint32(16), out=u)
            out[a:a + m] = u
    return out.reshape(shape)


_STRUCTURE_ONLY = [False]


def _finish(rng, wl_kwargs, n_rows, n_q, n_prefill_q, dtype, Hkv, Hq, D, data_scale=1.0):
    if _STRUCTURE_ONLY[0]:  # values are drawn last, so skipping them changes nothing else
        z = np.zeros((0, Hkv, D), dtype=np.float32 if dtype == "f32" else np.uint16)
        return Workload(rows_k=z, rows_v=z, q=z, prefill_q=None, dtype=dtype,
                        num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D,
                        scale=1.0 / math.sqrt(D), **wl_kwargs)
    rows_k = _draw_values(rng, (n_rows, Hkv, D), dtype, data_scale)
    rows_v = _draw_values(rng, (n_rows, Hkv, D), dtype, data_scale)
    q = _draw_values(rng, (n_q, Hq, D), dtype)
    pq = _draw_values(rng, (n_prefill_q, Hq, D), dtype) if n_prefill_q else None
    return Workload(rows_k=rows_k, rows_v=rows_v, q=q, prefill_q=pq, dtype=dtype,
                    num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D,
                    scale=1.0 / math.sqrt(D), **wl_kwargs)


def _plain_decode(name, rng, lens, *, Hq, Hkv, D, B, dtype, pool=None,
                  data_scale=1.0, prefill_n=0, prefill_len=0):
    """S independent sequences: a prompt of L-1 tokens, then one decode token.

    With ``prefill_n`` > 0, that many seeded picks among sequences with
    L >= prefill_len + 1 instead hold L - 1 - prefill_len tokens at set-up and
    receive their last ``prefill_len`` positions before the decode token as one
    prefill chunk.
    """
    lens = np.asarray(lens, dtype=np.int64)
    S = len(lens)
    picks: List[int] = []
    if prefill_n:
        eligible = np.flatnonzero(lens >= prefill_len + 1)
        picks = sorted(int(x) for x in rng.choice(eligible, size=prefill_n, replace=False))
    need = int(sum(-(-int(L) // B) for L in lens))
    num_blocks = pool if pool is not None else int(math.ceil(1.1 * need))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    tokens = [rng.integers(0, VOCAB, size=int(L), dtype=np.int32) for L in lens]
    rows = _Rows()
    hist = {s: rows.take(int(lens[s])) for s in range(S)}
    ops = []
    starts = {}
    for s in range(S):
        L = int(lens[s])
        n0 = L - 1 - (prefill_len if s in picks else 0)
        ops.append(("alloc", s, tokens[s][:n0], hist[s][:n0]))
        starts[s] = n0
    if picks:
        ops.append(("phase", "prefill"))
        for s in picks:
            a = starts[s]
            ops.append(("extend", s, tokens[s][a:a + prefill_len], hist[s][a:a + prefill_len]))
    ops.append(("phase", "decode"))
    for s in range(S):
        L = int(lens[s])
        ops.append(("append", s, int(tokens[s][L - 1]), int(hist[s][L - 1])))
    kw = dict(name=name, block_size=B, num_blocks=num_blocks, free_order=free_order,
              decode_seqs=list(range(S)), hist=hist, ops=ops,
              prefill_seqs=picks, prefill_len=prefill_len,
              prefill_start=np.array([starts[s] for s in picks], dtype=np.int64) if picks else None,
              meta=dict(need_blocks=need))
    return _finish(rng, kw, rows.n, S, len(picks) * prefill_len, dtype, Hkv, Hq, D, data_scale)


def tiny(rng, size):
    """Two fp32 sequences of 7 and 11 tokens, 4 heads of 64, blocks of 4, 16-block pool.

    K and V are N(0,1) scaled by 1/sqrt(64) as data; the softmax scale 1/sqrt(64)
    is applied on top.
    """
    return _plain_decode("tiny", rng, [7, 11], Hq=4, Hkv=4, D=64, B=4, dtype="f32",
                         pool=16, data_scale=1.0 / 8.0)


def llama13b(rng, size):
    """LLaMA-13B-shaped decode layer: 40 MHA heads of 128, bf16, blocks of 16,
    lengths uniform on [1, 2048], pool 1.1x the need, random placement."""
    S, Lmax = (64, 2048) if size == "full" else (6, 300)
    lens = rng.integers(1, Lmax + 1, size=S)
    return _plain_decode("llama13b", rng, lens, Hq=40, Hkv=40, D=128, B=16, dtype="bf16")


def llama13b_fp8(rng, size):
    """The llama13b structure with an FP8 (E4M3) KV cache: queries and new K/V
    rows are bf16 as drawn, and the pool stores them as 8-bit codes with one
    scale per pool (2^-6, so N(0,1) values sit well inside the format's range)."""
    wl = llama13b(rng, size)
    wl.name = "llama13b_fp8"
    wl.kv_dtype = "fp8_e4m3"
    wl.k_scale = wl.v_scale = 2.0 ** -6
    return wl


def llama70b(rng, size):
    """Llama-2-70B-shaped GQA layer: 64 query / 8 KV heads of 128, bf16, blocks of 16,
    lengths log-uniform on [128, 8192]; 8 sequences also take a 512-row prefill chunk."""
    if size == "full":
        S, lo, hi, pn, pl = 256, 128, 8192, 8, 512
    else:
        S, lo, hi, pn, pl = 8, 16, 700, 2, 128
    lens = np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi + 1), size=S))).astype(np.int64)
    lens = np.clip(lens, lo, hi)
    if int((lens >= pl + 1).sum()) < pn:  # keep the prefill picks possible at small sizes
        lens[:pn] = np.maximum(lens[:pn], pl + 1)
    return _plain_decode("llama70b", rng, lens, Hq=64, Hkv=8, D=128, B=16, dtype="bf16",
                         prefill_n=pn, prefill_len=pl)


def llama70b_fp8(rng, size):
    """The llama70b structure with an FP8 (E4M3) KV cache, one scale per pool
    (2^-6): the GQA shape for attention over FP8 codes (decode, and short
    chunks such as speculative verification)."""
    wl = llama70b(rng, size)
    wl.name = "llama70b_fp8"
    wl.kv_dtype = "fp8_e4m3"
    wl.k_scale = wl.v_scale = 2.0 ** -6
    return wl


def _parallel_sampling(name, rng, size, prompt_full, prompt_small):
    """Parallel sampling: each prompt is forked into 3 samples that share its
    blocks (ref count 3) and then append divergent tails, one token per step."""
    G, P, tmax = (32, prompt_full, 256) if size == "full" else (2, prompt_small, 20)
    B, H, D, n = 16, 40, 128, 3
    tails = rng.integers(1, tmax + 1, size=(G, n))
    full = P // B
    need = sum(full + sum(-(-(P + int(t)) // B) - full for t in tails[g]) for g in range(G))
    num_blocks = int(math.ceil(1.1 * need))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    ptok = rng.integers(0, VOCAB, size=(G, P), dtype=np.int32)
    ttok = rng.integers(0, VOCAB, size=(G, n, tmax), dtype=np.int32)
    rows = _Rows()
    prow = [rows.take(P) for _ in range(G)]
    trow = [[rows.take(int(tails[g, i])) for i in range(n)] for g in range(G)]
    ops, hist = [], {}
    for g in range(G):
        ops.append(("alloc", n * g, ptok[g], prow[g]))
        for i in range(1, n):
            ops.append(("fork", n * g, n * g + i))
    for t in range(tmax - 1):
        for g in range(G):
            for i in range(n):
                if t < tails[g, i] - 1:
                    ops.append(("append", n * g + i, int(ttok[g, i, t]), int(trow[g][i][t])))
    ops.append(("phase", "decode"))
    for g in range(G):
        for i in range(n):
            t = int(tails[g, i]) - 1
            ops.append(("append", n * g + i, int(ttok[g, i, t]), int(trow[g][i][t])))
            hist[n * g + i] = np.concatenate([prow[g], trow[g][i]])
    kw = dict(name=name, block_size=B, num_blocks=num_blocks, free_order=free_order,
              decode_seqs=list(range(n * G)), hist=hist, ops=ops,
              meta=dict(need_blocks=need, samples=n, groups=G, prompt=P))
    return _finish(rng, kw, rows.n, n * G, 0, "bf16", H, H, D)


def cow(rng, size):
    """Copy-on-write parallel sampling on 512-token prompts (block aligned)."""
    return _parallel_sampling("cow", rng, size, 512, 48)


def cow504(rng, size):
    """As ``cow`` with 504-token prompts, so each prompt's last block is half
    full and is copied when a sample first appends into it while shared."""
    return _parallel_sampling("cow504", rng, size, 504, 40)


def beam(rng, size):
    """Beam search, width 4: each step every new beam picks a parent uniformly
    with replacement, forks from it and appends a token; old beams are freed."""
    G, P, tmax = (32, 512, 256) if size == "full" else (2, 40, 12)
    W, B, H, D = 4, 16, 40, 128
    T = rng.integers(1, tmax + 1, size=G)
    picks = [rng.integers(0, W, size=(int(T[g]), W)) for g in range(G)]
    bound = sum(-(-P // B) + W * (-(-int(T[g]) // B) + 1) for g in range(G))
    num_blocks = int(math.ceil(1.1 * bound))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    ptok = rng.integers(0, VOCAB, size=(G, P), dtype=np.int32)
    stok = [rng.integers(0, VOCAB, size=(int(T[g]), W), dtype=np.int32) for g in range(G)]
    rows = _Rows()
    prow = [rows.take(P) for _ in range(G)]
    srow = [rows.take(int(T[g]) * W).reshape(int(T[g]), W) for g in range(G)]
    ops = []
    hist: Dict[int, np.ndarray] = {}
    next_id = [0]

    def fresh():
        next_id[0] += 1
        return next_id[0] - 1

    live = []
    for g in range(G):
        ids = [fresh() for _ in range(W)]
        ops.append(("alloc", ids[0], ptok[g], prow[g]))
        hist[ids[0]] = list(prow[g])
        for i in range(1, W):
            ops.append(("fork", ids[0], ids[i]))
            hist[ids[i]] = list(hist[ids[0]])
        live.append(ids)

    def step(g, t):
        new = [fresh() for _ in range(W)]
        for j in range(W):
            par = live[g][int(picks[g][t, j])]
            ops.append(("fork", par, new[j]))
            hist[new[j]] = list(hist[par])
        for old in live[g]:
            ops.append(("free", old))
            del hist[old]
        for j in range(W):
            ops.append(("append", new[j], int(stok[g][t, j]), int(srow[g][t, j])))
            hist[new[j]].append(int(srow[g][t, j]))
        live[g] = new

    for t in range(tmax - 1):
        for g in range(G):
            if t < T[g] - 1:
                step(g, t)
    ops.append(("phase", "decode"))
    for g in range(G):
        step(g, int(T[g]) - 1)
    seqs = [s for g in range(G) for s in live[g]]
    hist = {s: np.asarray(hist[s], dtype=np.int64) for s in seqs}
    kw = dict(name="beam", block_size=B, num_blocks=num_blocks, free_order=free_order,
              decode_seqs=seqs, hist=hist, ops=ops,
              meta=dict(bound_blocks=bound, width=W, groups=G, prompt=P))
    return _finish(rng, kw, rows.n, len(seqs), 0, "bf16", H, H, D)


def prefix(rng, size):
    """Prefix-cached batch: every request starts with the same system prompt
    (same token ids, so the same K/V) followed by a unique tail; the tail's last
    token is the decode token."""
    S, Pn, tlo, thi = (256, 1024, 16, 512) if size == "full" else (8, 64, 16, 60)
    B, H, D = 16, 40, 128
    tails = rng.integers(tlo, thi + 1, size=S)
    need = -(-Pn // B) + int(sum(-(-int(t) // B) for t in tails))
    num_blocks = int(math.ceil(1.1 * need))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    ptok = rng.integers(0, VOCAB, size=Pn, dtype=np.int32)
    ttok = [rng.integers(0, VOCAB, size=int(t), dtype=np.int32) for t in tails]
    rows = _Rows()
    prow = rows.take(Pn)
    trow = [rows.take(int(t)) for t in tails]
    ops, hist = [], {}
    for s in range(S):
        ops.append(("alloc", s, np.concatenate([ptok, ttok[s][:-1]]),
                    np.concatenate([prow, trow[s][:-1]])))
        hist[s] = np.concatenate([prow, trow[s]])
    ops.append(("phase", "decode"))
    for s in range(S):
        ops.append(("append", s, int(ttok[s][-1]), int(trow[s][-1])))
    kw = dict(name="prefix", block_size=B, num_blocks=num_blocks, free_order=free_order,
              decode_seqs=list(range(S)), hist=hist, ops=ops,
              meta=dict(need_blocks=need, prefix_tokens=Pn))
    return _finish(rng, kw, rows.n, S, 0, "bf16", H, H, D)


# name -> (seed, builder). Seeds: one per workload, fixed.
CONFIGS: Dict[str, tuple] = {
    "tiny": (1, tiny),
    "llama13b": (2, llama13b),
    "cow": (3, cow),
    "cow504": (31, cow504),
    "beam": (32, beam),
    "prefix": (4, prefix),
    "llama70b": (5, llama70b),
    "llama13b_fp8": (21, llama13b_fp8),
    "llama70b_fp8": (51, llama70b_fp8),
}


def config_names() -> List[str]:
    return list(CONFIGS)


def make(name: str, size: str = "full", seed: int | None = None,
         values: bool = True) -> Workload:
    """Draw workload ``name`` ("full" or "small"); the seed defaults to the
    workload's own and is offset for the small size so the two differ.
    ``values=False`` skips the K/V/q draws (empty arrays): structure only."""
    if size not in ("full", "small"):
        raise ValueError(f"size must be 'full' or 'small', not {size!r}")
    base, fn = CONFIGS[name]
    if seed is None:
        seed = base if size == "full" else 1000 + base
    rng = np.random.default_rng(seed)
    _STRUCTURE_ONLY[0] = not values
    try:
        wl = fn(rng, size)
    finally:
        _STRUCTURE_ONLY[0] = False
    wl.meta["seed"] = seed
    wl.meta["size"] = size
    return wl
