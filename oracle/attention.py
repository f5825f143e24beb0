"""Plain fp64 softmax attention over logical (contiguous) K/V.

Decode ("vLLM PagedAttention explained", section 3.3, step 2): the new token's
query attends to every cached token of its own sequence, the new token
included. Softmax and the weighted sum of V, which the kernel outline on "LLM
inference engine internals" (section 2.4) leaves as a comment, are written
here as their textbook definitions with the usual 1/sqrt(D) scale passed in.

Grouped heads (not on the pages): query head h reads KV head h // G with
G = Hq / Hkv, contiguous groups.

Chunked prefill ("vLLM PagedAttention explained", section 7.2): a chunk of C
prompt positions starting at absolute position a0 attends causally, row i to
keys 0 .. a0 + i.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np


def _attend(qv: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one query vector q [D], K/V [L, D]; float64."""
    if K.shape[0] == 0:  # empty context: defined as zeros
        return np.zeros(V.shape[1], dtype=np.float64)
    z = scale * (K @ qv)
    z = z - z.max()
    e = np.exp(z)
    p = e / e.sum()
    return p @ V


def decode_attention(q: np.ndarray, ks: Sequence[np.ndarray], vs: Sequence[np.ndarray],
                     scale: float) -> np.ndarray:
    """q [S, Hq, D]; ks[s], vs[s] [L_s, Hkv, D] (any float dtype) -> [S, Hq, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    S, Hq, D = q.shape
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        K = np.asarray(ks[s], dtype=np.float64)
        V = np.asarray(vs[s], dtype=np.float64)
        Hkv = K.shape[1]
        if Hq % Hkv:
            raise ValueError("query heads must be a multiple of KV heads")
        G = Hq // Hkv
        for h in range(Hq):
            g = h // G
            out[s, h] = _attend(q[s, h], K[:, g, :], V[:, g, :], scale)
    return out


def prefill_attention(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, start: int,
                      scale: float) -> np.ndarray:
    """Causal attention of C chunk rows (absolute positions start .. start+C-1).

    q_rows [C, Hq, D]; K, V [>= start+C, Hkv, D] logical keys/values of the
    sequence. Row i sees keys 0 .. start + i. Returns [C, Hq, D] float64.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    C, Hq, D = q_rows.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((C, Hq, D), dtype=np.float64)
    for i in range(C):
        n = start + i + 1
        for h in range(Hq):
            g = h // G
            out[i, h] = _attend(q_rows[i, h], K[:n, g, :], V[:n, g, :], scale)
    return out
