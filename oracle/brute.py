"""Loop-level twins of the oracle for tiny inputs (pure Python; test infrastructure).

They restate the same definitions element by element so that the vectorised oracle in
``method.py`` can be checked against something that does not share its library calls.
"""
from __future__ import annotations

import math


def score_loops(q, w, k):
    """S[s] = sum_h w[h] * max(0, sum_d q[h][d] * k[s][d]) with explicit loops."""
    H, D = len(q), len(q[0])
    out = []
    for s in range(len(k)):
        tot = 0.0
        for h in range(H):
            dot = 0.0
            for d in range(D):
                dot += float(q[h][d]) * float(k[s][d])
            tot += float(w[h]) * (dot if dot > 0.0 else 0.0)
        out.append(tot)
    return out


def topk_by_rank(S, K):
    """Selected iff rank(s) < min(K, n), rank(s) = #{s' : S[s'] > S[s] or (S[s'] == S[s] and
    s' < s)}; returned ascending and padded with -1 to length K."""
    n = len(S)
    k = min(K, n)
    sel = []
    for s in range(n):
        rank = 0
        for s2 in range(n):
            if S[s2] > S[s] or (S[s2] == S[s] and s2 < s):
                rank += 1
        if rank < k:
            sel.append(s)
    return sel + [-1] * (K - len(sel))


def attention_loops(q, rows, scale, D_v):
    """Dense attention of one token over ``rows`` with explicit loops (two-pass softmax)."""
    H = len(q)
    o = [[0.0] * D_v for _ in range(H)]
    lse = [0.0] * H
    for h in range(H):
        z = []
        for r in rows:
            acc = 0.0
            for d in range(len(r)):
                acc += float(q[h][d]) * float(r[d])
            z.append(scale * acc)
        m = max(z)
        den = sum(math.exp(v - m) for v in z)
        for s, r in enumerate(rows):
            p = math.exp(z[s] - m) / den
            for d in range(D_v):
                o[h][d] += p * float(r[d])
        lse[h] = m + math.log(den)
    return o, lse
