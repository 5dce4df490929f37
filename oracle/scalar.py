"""Pure-Python scalar attention for tiny inputs (test infrastructure).

An independent second implementation used to pin ``oracle.attention``: nested
loops, ``math.exp``/``math.log`` and ``math.fsum`` only, no numpy arithmetic.  It
follows the same definition (scaled dot products, masked keys excluded, softmax,
weighted sum of V rows; LSE = log of the sum of exp of the visible scaled scores)
but shares no code with ``oracle.attention``.
"""
from __future__ import annotations

import math


def _vis(i, j, Nq, Nk, causal, left, right):
    off = Nk - Nq
    if causal and j > i + off:
        return False
    if left >= 0 and j < i + off - left:
        return False
    if right >= 0 and j > i + off + right:
        return False
    return 0 <= j < Nk


def attention_scalar(q, k, v, scale, causal=False, left=-1, right=-1):
    """q: nested lists [B][Hq][Nq][D]; k, v: [B][Hkv][Nk][D].  Returns (O, LSE) lists."""
    B, Hq = len(q), len(q[0])
    Nq, D = len(q[0][0]), len(q[0][0][0])
    Hkv, Nk = len(k[0]), len(k[0][0])
    g = Hq // Hkv
    O = [[[[0.0] * D for _ in range(Nq)] for _ in range(Hq)] for _ in range(B)]
    L = [[[-math.inf] * Nq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for i in range(Nq):
                scores = []
                for j in range(Nk):
                    if _vis(i, j, Nq, Nk, causal, left, right):
                        dot = math.fsum(q[b][h][i][d] * k[b][kh][j][d] for d in range(D))
                        scores.append((j, scale * dot))
                if not scores:
                    continue
                mx = max(s for _, s in scores)
                w = [(j, math.exp(s - mx)) for j, s in scores]
                z = math.fsum(x for _, x in w)
                L[b][h][i] = mx + math.log(z)
                for d in range(D):
                    O[b][h][i][d] = math.fsum(x * v[b][kh][j][d] for j, x in w) / z
    return O, L


def logsumexp_scalar(values):
    """log(sum(exp(x))) of a list of finite floats by the shifted definition."""
    mx = max(values)
    return mx + math.log(math.fsum(math.exp(x - mx) for x in values))
