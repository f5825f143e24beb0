"""Attention in pure-Python loops (math.exp, math.fsum): tiny inputs only.

Written independently of ``attention.py`` from the definition of softmax
attention, so the two pin each other on small cases.
"""

from __future__ import annotations

import math


def attend(q, K, V, scale):
    """q: list[D]; K, V: list[L] of list[D]. Returns list[D]."""
    L = len(K)
    D = len(V[0]) if L else len(q)
    if L == 0:
        return [0.0] * D
    logits = [scale * math.fsum(q[d] * K[t][d] for d in range(len(q))) for t in range(L)]
    mx = max(logits)
    w = [math.exp(x - mx) for x in logits]
    tot = math.fsum(w)
    return [math.fsum(w[t] * V[t][d] for t in range(L)) / tot for d in range(D)]


def decode(q, ks, vs, scale):
    """q[s][h][d]; ks[s][t][g][d]; vs likewise. GQA: head h reads KV head h // G."""
    out = []
    for s in range(len(q)):
        Hq = len(q[s])
        Hkv = len(ks[s][0]) if ks[s] else Hq
        G = Hq // Hkv
        row = []
        for h in range(Hq):
            g = h // G
            K = [ks[s][t][g] for t in range(len(ks[s]))]
            V = [vs[s][t][g] for t in range(len(vs[s]))]
            row.append(attend(q[s][h], K, V, scale))
        out.append(row)
    return out
