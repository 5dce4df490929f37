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


def attention_scalar_ext(q, k, v, scale, causal=False, left=-1, right=-1, softcap=0.0,
                         alibi_slopes=None, bias=None, block_mask=None, block_q=1, block_k=1):
    """The scalar definition with score modifiers, for tiny inputs: per (query, key) the
    score is scale * dot, then softcap * tanh(score / softcap) when softcap > 0, then minus
    slope_h * |i + off - j| when ALiBi slopes are given, then plus bias[b][h][j]; keys
    outside the causal / window rule or in a block with block_mask[b][h][i // block_q]
    [j // block_k] false are left out.  Nested lists in and out, as attention_scalar."""
    B, Hq = len(q), len(q[0])
    Nq, D = len(q[0][0]), len(q[0][0][0])
    Hkv, Nk = len(k[0]), len(k[0][0])
    g = Hq // Hkv
    off = Nk - Nq
    O = [[[[0.0] * D for _ in range(Nq)] for _ in range(Hq)] for _ in range(B)]
    L = [[[-math.inf] * Nq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for i in range(Nq):
                scores = []
                for j in range(Nk):
                    if not _vis(i, j, Nq, Nk, causal, left, right):
                        continue
                    if block_mask is not None and not block_mask[b][h][i // block_q][j // block_k]:
                        continue
                    x = scale * math.fsum(q[b][h][i][d] * k[b][kh][j][d] for d in range(D))
                    if softcap > 0:
                        x = softcap * math.tanh(x / softcap)
                    if alibi_slopes is not None:
                        x -= alibi_slopes[h] * abs(i + off - j)
                    if bias is not None:
                        x += bias[b][h][j]
                    scores.append((j, x))
                if not scores:
                    continue
                mx = max(x for _, x in scores)
                w = [(j, math.exp(x - mx)) for j, x in scores]
                z = math.fsum(x for _, x in w)
                L[b][h][i] = mx + math.log(z)
                for d in range(D):
                    O[b][h][i][d] = math.fsum(x * v[b][kh][j][d] for j, x in w) / z
    return O, L
