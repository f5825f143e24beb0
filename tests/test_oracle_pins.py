"""Pins of the fp64 oracle's attention against facts outside itself (CPU only).

Each pin is a function of the attention routines under test, so the same
battery also runs against deliberately broken copies of the oracle
(``test_planted_mistakes_are_caught``): every plausible mistake must trip at
least one pin.
"""

import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import workloads
from oracle import brute
from oracle.attention import decode_attention, prefill_attention
from oracle.paging import PoolMirror

RNG = np.random.default_rng(20240601)


def _rand_case(rng, S=3, Hq=4, Hkv=2, D=8, Lmax=12):
    lens = rng.integers(1, Lmax + 1, size=S)
    q = rng.standard_normal((S, Hq, D))
    ks = [rng.standard_normal((int(L), Hkv, D)) for L in lens]
    vs = [rng.standard_normal((int(L), Hkv, D)) for L in lens]
    return q, ks, vs


# ---------------------------------------------------------------- pins ----
def pin_brute_force(dec, pre):
    """Pure-Python loops (math.exp / math.fsum) agree to 1e-12 on tiny inputs."""
    rng = np.random.default_rng(7)
    for Hq, Hkv in ((4, 4), (4, 2), (6, 1)):
        q, ks, vs = _rand_case(rng, S=3, Hq=Hq, Hkv=Hkv, D=5, Lmax=9)
        scale = 1 / math.sqrt(5)
        got = dec(q, ks, vs, scale)
        want = np.array(brute.decode(q.tolist(), [k.tolist() for k in ks],
                                     [v.tolist() for v in vs], scale))
        if not np.allclose(got, want, rtol=0, atol=1e-12):
            return False
    return True


def _sdpa(q, k, v, scale, mask=None):
    """torch SDPA in float64 on CPU: q [Hq, Lq, D], k/v [Hkv, Lk, D] expanded per head."""
    G = q.shape[0] // k.shape[0]
    k = k.repeat_interleave(G, dim=0).contiguous()
    v = v.repeat_interleave(G, dim=0).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)


def pin_sdpa_decode(dec, pre):
    """Identity block table with one block covering the sequence = contiguous
    attention: torch's scaled_dot_product_attention (float64, CPU) agrees."""
    rng = np.random.default_rng(11)
    for Hq, Hkv, D in ((8, 8, 16), (8, 2, 16), (4, 1, 32)):
        q, ks, vs = _rand_case(rng, S=4, Hq=Hq, Hkv=Hkv, D=D, Lmax=40)
        scale = 1 / math.sqrt(D)
        got = dec(q, ks, vs, scale)
        for s in range(len(ks)):
            want = _sdpa(torch.from_numpy(q[s][:, None, :]),
                         torch.from_numpy(ks[s].transpose(1, 0, 2)),
                         torch.from_numpy(vs[s].transpose(1, 0, 2)), scale)[:, 0, :].numpy()
            if not np.allclose(got[s], want, rtol=0, atol=1e-12):
                return False
    return True


def pin_sdpa_prefill(dec, pre):
    """Causal chunk: with the chunk covering the whole sequence this is SDPA with
    is_causal; with earlier cached tokens it is SDPA with the matching mask."""
    rng = np.random.default_rng(13)
    Hq, Hkv, D = 4, 2, 16
    scale = 1 / math.sqrt(D)
    for L, C in ((10, 10), (23, 7), (16, 1)):
        K = rng.standard_normal((L, Hkv, D))
        V = rng.standard_normal((L, Hkv, D))
        qr = rng.standard_normal((C, Hq, D))
        start = L - C
        got = pre(qr, K, V, start, scale)
        tq = torch.from_numpy(qr.transpose(1, 0, 2))
        tk = torch.from_numpy(K.transpose(1, 0, 2))
        tv = torch.from_numpy(V.transpose(1, 0, 2))
        if C == L:
            G = Hq // Hkv
            want = torch.nn.functional.scaled_dot_product_attention(
                tq, tk.repeat_interleave(G, 0), tv.repeat_interleave(G, 0),
                is_causal=True, scale=scale)
        else:
            mask = torch.arange(L)[None, :] <= (start + torch.arange(C))[:, None]
            want = _sdpa(tq, tk, tv, scale, mask)
        if not np.allclose(got, want.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12):
            return False
    return True


def pin_zero_keys_mean(dec, pre):
    """All-zero keys: every logit is 0, the softmax is uniform, the output is mean(V)."""
    rng = np.random.default_rng(17)
    q = rng.standard_normal((2, 4, 8))
    ks = [np.zeros((L, 2, 8)) for L in (5, 13)]
    vs = [rng.standard_normal((L, 2, 8)) for L in (5, 13)]
    got = dec(q, ks, vs, 0.3)
    for s in range(2):
        want = np.repeat(vs[s].mean(axis=0), 2, axis=0)  # head h reads KV head h // 2
        if not np.allclose(got[s], want, rtol=0, atol=1e-14):
            return False
    return True


def pin_single_token(dec, pre):
    """One cached token: its weight is exactly 1, the output is V[0] bit for bit."""
    rng = np.random.default_rng(19)
    q = rng.standard_normal((3, 4, 8))
    ks = [rng.standard_normal((1, 4, 8)) for _ in range(3)]
    vs = [rng.standard_normal((1, 4, 8)) for _ in range(3)]
    got = dec(q, ks, vs, 0.5)
    return all(np.array_equal(got[s], vs[s][0]) for s in range(3))


def pin_known_weights(dec, pre):
    """Two keys with logits 0 and ln 3 (scale 1): weights are exactly 1/4 and 3/4."""
    q = np.zeros((1, 1, 2)); q[0, 0, 0] = 1.0
    K = np.array([[[0.0, 5.0]], [[math.log(3.0), -2.0]]])
    V = np.array([[[4.0, 0.0]], [[0.0, 8.0]]])
    got = dec(q, [K], [V], 1.0)[0, 0]
    return np.allclose(got, [1.0, 6.0], rtol=0, atol=1e-14)


def pin_prefill_rows_are_decodes(dec, pre):
    """Chunk row i equals a decode over the first start+i+1 tokens."""
    rng = np.random.default_rng(23)
    L, C, Hq, Hkv, D = 19, 6, 4, 2, 8
    K = rng.standard_normal((L, Hkv, D)); V = rng.standard_normal((L, Hkv, D))
    qr = rng.standard_normal((C, Hq, D))
    start = L - C
    got = pre(qr, K, V, start, 0.4)
    for i in range(C):
        want = dec(qr[i][None], [K[:start + i + 1]], [V[:start + i + 1]], 0.4)[0]
        if not np.allclose(got[i], want, rtol=0, atol=1e-13):
            return False
    return True


PINS = [pin_brute_force, pin_sdpa_decode, pin_sdpa_prefill, pin_zero_keys_mean,
        pin_single_token, pin_known_weights, pin_prefill_rows_are_decodes]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin):
    assert pin(decode_attention, prefill_attention)


# ------------------------------------------------------ planted mistakes ----
def _mut_decode(kind):
    def dec(q, ks, vs, scale):
        q = np.asarray(q, dtype=np.float64)
        S, Hq, D = q.shape
        out = np.zeros((S, Hq, D))
        for s in range(S):
            K = np.asarray(ks[s], dtype=np.float64); V = np.asarray(vs[s], dtype=np.float64)
            Hkv = K.shape[1]; G = Hq // Hkv
            for h in range(Hq):
                g = (h % Hkv) if kind == "gqa_modulo" else h // G
                k, v = K[:, g, :], V[:, g, :]
                if kind == "drop_last":
                    k, v = k[:-1] if len(k) > 1 else k, v[:-1] if len(v) > 1 else v
                if kind == "v_is_k":
                    v = k
                sc = 1.0 if kind == "no_scale" else scale
                if kind == "scale_sqrt":
                    sc = math.sqrt(scale)
                z = sc * (k @ q[s, h])
                e = np.exp(z - z.max())
                p = e if kind == "no_norm" else e / e.sum()
                if kind == "reverse_v":
                    v = v[::-1]
                out[s, h] = p @ v
        return out
    return dec


def _mut_prefill(kind):
    def pre(q_rows, K, V, start, scale):
        q_rows = np.asarray(q_rows, dtype=np.float64)
        C, Hq, D = q_rows.shape
        Hkv = K.shape[1]; G = Hq // Hkv
        out = np.zeros((C, Hq, D))
        for i in range(C):
            n = start + i + (0 if kind == "causal_off_by_one" else 1)
            if kind == "no_causal":
                n = K.shape[0]
            if kind == "chunk_relative":
                n = i + 1
            n = max(n, 1)
            for h in range(Hq):
                g = h // G
                z = scale * (K[:n, g, :] @ q_rows[i, h])
                e = np.exp(z - z.max())
                out[i, h] = (e / e.sum()) @ V[:n, g, :]
        return out
    return pre


DECODE_MUTANTS = ["gqa_modulo", "drop_last", "v_is_k", "no_scale", "scale_sqrt",
                  "no_norm", "reverse_v"]
PREFILL_MUTANTS = ["causal_off_by_one", "no_causal", "chunk_relative"]


@pytest.mark.parametrize("kind", DECODE_MUTANTS)
def test_planted_decode_mistake_is_caught(kind):
    bad = _mut_decode(kind)
    failed = [p.__name__ for p in PINS if not p(bad, prefill_attention)]
    assert failed, f"no pin catches decode mutant {kind}"


@pytest.mark.parametrize("kind", PREFILL_MUTANTS)
def test_planted_prefill_mistake_is_caught(kind):
    bad = _mut_prefill(kind)
    failed = [p.__name__ for p in PINS if not p(decode_attention, bad)]
    assert failed, f"no pin catches prefill mutant {kind}"


# -------------------------------------------------- randomized brute force ----
@settings(max_examples=40, deadline=None)
@given(S=st.integers(1, 3), Hkv=st.integers(1, 3), G=st.sampled_from([1, 2, 4]),
       D=st.integers(1, 8), Lmax=st.integers(1, 20), seed=st.integers(0, 2**31 - 1))
def test_brute_force_random(S, Hkv, G, D, Lmax, seed):
    rng = np.random.default_rng(seed)
    q, ks, vs = _rand_case(rng, S=S, Hq=Hkv * G, Hkv=Hkv, D=D, Lmax=Lmax)
    scale = 1 / math.sqrt(D)
    got = decode_attention(q, ks, vs, scale)
    want = np.array(brute.decode(q.tolist(), [k.tolist() for k in ks],
                                 [v.tolist() for v in vs], scale))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_tiny_workload_brute_force():
    """The 2-sequence fp32 workload, end to end through the brute-force loops."""
    wl = workloads.make("tiny")
    ks, vs = [], []
    for s in wl.decode_seqs:
        k, v = wl.logical_kv(s)
        ks.append(k.astype(np.float64)); vs.append(v.astype(np.float64))
    q = wl.values(wl.q).astype(np.float64)
    got = decode_attention(q, ks, vs, wl.scale)
    want = np.array(brute.decode(q.tolist(), [k.tolist() for k in ks],
                                 [v.tolist() for v in vs], wl.scale))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ------------------------------------------------------------ invariances ----
def _paged_attention_via_mirror(q, ks, vs, scale, B, placement):
    """Write each sequence's K/V into a mirror pool at blocks chosen by
    ``placement`` (a list of physical ids consumed in order), read it back
    through the block tables, and attend."""
    S, Hq, D = q.shape
    Hkv = ks[0].shape[1]
    nb = sum(-(-len(k) // B) for k in ks)
    pool = PoolMirror(len(placement), Hkv, B, D, np.float64)
    it = iter(placement)
    tables = []
    for s in range(S):
        table = [next(it) for _ in range(-(-len(ks[s]) // B))]
        tables.append(table)
        slots = [table[t // B] * B + t % B for t in range(len(ks[s]))]
        pool.write(slots, ks[s], vs[s])
    assert nb <= len(placement)
    gk, gv = zip(*[pool.gather(tables[s], len(ks[s])) for s in range(S)])
    return decode_attention(q, gk, gv, scale)


def test_placement_invariance():
    """Any permutation of physical block placement gives a bitwise-identical output."""
    rng = np.random.default_rng(29)
    q, ks, vs = _rand_case(rng, S=4, Hq=4, Hkv=2, D=8, Lmax=30)
    base = _paged_attention_via_mirror(q, ks, vs, 0.35, 4, list(range(64)))
    for _ in range(5):
        perm = list(rng.permutation(64))
        assert np.array_equal(base, _paged_attention_via_mirror(q, ks, vs, 0.35, 4, perm))
    assert np.array_equal(base, decode_attention(q, ks, vs, 0.35))


def test_cow_shared_equals_copied():
    """Sequences that share prompt blocks (ref count > 1) read the same K/V, and
    give the same output, as when every shared block is physically duplicated."""
    rng = np.random.default_rng(31)
    B, Hkv, D = 4, 2, 8
    prompt_k = rng.standard_normal((10, Hkv, D)); prompt_v = rng.standard_normal((10, Hkv, D))
    tails = [(rng.standard_normal((n, Hkv, D)), rng.standard_normal((n, Hkv, D))) for n in (1, 3, 6)]
    q = rng.standard_normal((3, 4, D))
    # shared: blocks 0..2 hold the prompt (last one partial, copied on divergence)
    shared = PoolMirror(32, Hkv, B, D, np.float64)
    shared.write(list(range(10)), prompt_k, prompt_v)
    tables, nxt = [], 3
    for i, (tk, tv) in enumerate(tails):
        table = [0, 1, 2]
        if i < 2:  # first two samples copy the partial block 2
            shared.copy([(2, nxt)]); table[2] = nxt; nxt += 1
        for j in range(len(tk)):
            pos = 10 + j
            if pos // B >= len(table):
                table.append(nxt); nxt += 1
            shared.write([table[pos // B] * B + pos % B], tk[j:j + 1], tv[j:j + 1])
        tables.append(table)
    got_shared = decode_attention(q, *zip(*[shared.gather(tables[i], 10 + len(tails[i][0]))
                                              for i in range(3)]), 0.3)
    ks = [np.concatenate([prompt_k, tk]) for tk, _ in tails]
    vs = [np.concatenate([prompt_v, tv]) for _, tv in tails]
    got_copied = _paged_attention_via_mirror(q, ks, vs, 0.3, B, list(range(40)))
    assert np.array_equal(got_shared, got_copied)


def test_kv_bytes_per_token_llama13b():
    """The page's ~800 KB of KV per token for LLaMA-13B: 2 (K,V) x 40 layers x
    40 heads x 128 dims x 2 bytes."""
    per_token = 2 * 40 * 40 * 128 * 2
    assert per_token == 819200
    assert abs(per_token / 1024 - 800) < 1e-9
    assert abs(2048 * per_token / 2**30 - 1.5625) < 1e-9  # "about 1.6 GB" at 2048 tokens
