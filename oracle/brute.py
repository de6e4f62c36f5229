"""Scalar brute force of the prefill path, for tiny inputs (test infrastructure).

Independent of ``oracle.reference``: pure Python floats, ``math`` functions and
explicit loops, one (query, head) at a time. It exists to pin the vectorised
oracle: both must agree to ~1e-12 on tiny shapes.

Definitions followed: RoPE bands theta_k = base^(-2k/d) ("Llama 3.1
Architecture: Dense Scaling to 405B and 128K Context", "1. High Base
Frequency"), adjacent channel pairs rotated by position * theta_k (RoFormer);
query head h uses KV head h // (Hq/Hkv); causal plus same-document visibility
("The Llama 3 Herd of Models", "A Deliberately Standard Dense Transformer");
scaled dot-product softmax.
"""

from __future__ import annotations

import math


def _rotate(vec, pos, base):
    d = len(vec)
    out = [0.0] * d
    for k in range(d // 2):
        ang = pos * (base ** (-(2.0 * k) / d))
        c, s = math.cos(ang), math.sin(ang)
        a, b = vec[2 * k], vec[2 * k + 1]
        out[2 * k] = a * c - b * s
        out[2 * k + 1] = a * s + b * c
    return out


def _doc_of(cu_docs, t):
    d = 0
    while not (cu_docs[d] <= t < cu_docs[d + 1]):
        d += 1
    return d


def brute_rope_attention(q, k, v, cu_docs=None, base=500000.0, positions=None, scale=None):
    """q [B][S][Hq][D], k/v [B][S][Hkv][D] as nested lists of floats.

    Returns (O [B][S][Hq][D], LSE [B][Hq][S]) as nested lists.
    """
    B, S, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0][0])
    g = Hq // Hkv
    if cu_docs is None:
        cu_docs = [0, S]
    cu_docs = [int(c) for c in cu_docs]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = [[[[0.0] * D for _ in range(Hq)] for _ in range(S)] for _ in range(B)]
    LSE = [[[0.0] * S for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        pos = [t if positions is None else int(positions[b][t]) for t in range(S)]
        for i in range(S):
            di = _doc_of(cu_docs, i)
            for h in range(Hq):
                kvh = h // g
                qi = _rotate([float(x) for x in q[b][i][h]], pos[i], base)
                keys, scores = [], []
                for j in range(S):
                    if j > i or _doc_of(cu_docs, j) != di:
                        continue
                    kj = _rotate([float(x) for x in k[b][j][kvh]], pos[j], base)
                    scores.append(math.fsum(qi[d] * kj[d] for d in range(D)) * scale)
                    keys.append(j)
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = math.fsum(w)
                for d in range(D):
                    O[b][i][h][d] = math.fsum(w[n] * float(v[b][keys[n]][kvh][d])
                                              for n in range(len(keys))) / tot
                LSE[b][h][i] = mx + math.log(tot)
    return O, LSE
