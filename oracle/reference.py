"""Float64 reference for exact attention (test infrastructure; see ``oracle/__init__``).

Notation follows the pages: Q ``[B, Hq, Nq, D]``, K/V ``[B, Hkv, Nk, D]``, grouped
query heads ``g = Hq / Hkv`` with query head ``h`` reading KV head ``h // g``
(mlx-bun forward shader, head mapping; mlx-mfa "Native GQA").

Readings taken where the pages leave a point open (each is listed in the design doc):

* Window ``(left, right)``, ``-1`` = unbounded (mlx-mfa "Sliding window" feature):
  key ``j`` is visible to query ``i`` iff ``i+off-left <= j <= i+off+right``,
  both ends inclusive.
* Causal alignment is bottom-right: ``off = Nk - Nq``; key ``j`` is visible under
  the causal mask iff ``j <= i + off``.  For ``Nq == Nk`` this is the mlx-bun
  shader's ``kpos > q_row`` rule.
* A row with no visible key returns ``O = 0`` and ``LSE = -inf``.
* The LSE is the natural log of the sum of ``exp`` of the *scaled* scores.
"""
from __future__ import annotations

import math

import numpy as np

_BF16 = "bf16"
_F16 = "f16"


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of fp16 / bf16 storage given as uint16 bit patterns."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("expected uint16 bit patterns")
    if dtype == _F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == _BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def window_bounds(i, Nq: int, Nk: int, causal: bool, left: int, right: int):
    """Inclusive visible key range ``[lo, hi]`` of query row(s) ``i`` (may be empty)."""
    i = np.asarray(i, dtype=np.int64)
    off = Nk - Nq
    lo = np.zeros_like(i)
    if left >= 0:
        lo = np.maximum(lo, i + off - left)
    hi = np.full_like(i, Nk - 1)
    if causal:
        hi = np.minimum(hi, i + off)
    if right >= 0:
        hi = np.minimum(hi, i + off + right)
    return lo, hi


def visible(i, j, Nq: int, Nk: int, causal: bool, left: int, right: int):
    """Boolean visibility of key ``j`` to query ``i`` (broadcasting)."""
    i, j = np.broadcast_arrays(np.asarray(i, dtype=np.int64), np.asarray(j, dtype=np.int64))
    off = Nk - Nq
    ok = (j >= 0) & (j < Nk)
    if causal:
        ok = ok & (j <= i + off)
    if left >= 0:
        ok = ok & (j >= i + off - left)
    if right >= 0:
        ok = ok & (j <= i + off + right)
    return ok


def _rows_attention(qr, kk, vv, scale, vis):
    """Definition of attention for a block of rows.

    qr ``[r, D]``, kk/vv ``[Nk, D]``, vis ``[r, Nk]`` bool.  Returns O ``[r, D]``,
    LSE ``[r]``, P ``[r, Nk]``.
    """
    s = scale * (qr @ kk.T)
    s = np.where(vis, s, -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.exp(s - m[:, None])          # exp(-inf) = 0 at masked positions
    z = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(any_vis[:, None], e / np.where(any_vis, z, 1.0)[:, None], 0.0)
        lse = np.where(any_vis, m + np.log(np.where(any_vis, z, 1.0)), -np.inf)
    o = p @ vv
    return o, lse, p


def attention(q, k, v, scale: float, causal: bool = False, left: int = -1,
              right: int = -1, rows=None, row_block: int = 512):
    """O = softmax(scale·QKᵀ + mask)·V and LSE, in float64.

    q ``[B, Hq, Nq, D]``, k/v ``[B, Hkv, Nk, D]`` (float64 or anything numpy widens
    exactly).  ``rows`` optionally restricts the computation to a list of
    ``(b, h, i)`` triples; then the result is ``(O [n, D], LSE [n])`` in that order.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    cols = np.arange(Nk)
    if rows is not None:
        rows = list(rows)
        O = np.zeros((len(rows), D))
        L = np.zeros(len(rows))
        for n, (b, h, i) in enumerate(rows):
            kv = h // g
            vis = visible(np.array([[i]]), cols[None, :], Nq, Nk, causal, left, right)
            o, lse, _ = _rows_attention(q[b, h, i][None, :], k[b, kv], v[b, kv], scale, vis)
            O[n] = o[0]
            L[n] = lse[0]
        return O, L
    O = np.zeros((B, Hq, Nq, D))
    L = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            for r0 in range(0, Nq, row_block):
                r1 = min(Nq, r0 + row_block)
                ii = np.arange(r0, r1)
                vis = visible(ii[:, None], cols[None, :], Nq, Nk, causal, left, right)
                o, lse, _ = _rows_attention(q[b, h, r0:r1], k[b, kv], v[b, kv], scale, vis)
                O[b, h, r0:r1] = o
                L[b, h, r0:r1] = lse
    return O, L


def attention_backward(q, k, v, dout, scale: float, causal: bool = False, left: int = -1,
                       right: int = -1):
    """Gradients of ``attention``'s O with respect to Q, K, V, float64 (mlx-bun
    flash-attention.ts backward: the D-vector, dK/dV and dQ passes).

    With P the attention probabilities of the forward (masked keys have P = 0) and
    ``dO = dout``:
    ``dV = P^T dO``, ``dP = dO V^T``, ``D_i = sum_d dO_id O_id`` (= sum_j P_ij dP_ij),
    ``dS = P * (dP - D)``, ``dQ = scale * dS K``, ``dK = scale * dS^T Q``.
    With grouped query heads, dK and dV of a KV head sum the contributions of its ``g``
    query heads.  Rows with no visible key contribute nothing.  Returns ``(dQ, dK, dV)``
    shaped like ``q``, ``k``, ``v``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    ii = np.arange(Nq)[:, None]
    jj = np.arange(Nk)[None, :]
    vis = visible(ii, jj, Nq, Nk, causal, left, right)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            _, _, p = _rows_attention(q[b, h], k[b, kv], v[b, kv], scale, vis)
            o = p @ v[b, kv]
            dp = dout[b, h] @ v[b, kv].T
            dvec = (dout[b, h] * o).sum(axis=1)
            ds = p * (dp - dvec[:, None])
            dq[b, h] = scale * (ds @ k[b, kv])
            dk[b, kv] += scale * (ds.T @ q[b, h])
            dv[b, kv] += p.T @ dout[b, h]
    return dq, dk, dv


def attention_ext(q, k, v, scale: float, causal: bool = False, left: int = -1, right: int = -1,
                  softcap: float = 0.0, alibi_slopes=None, bias=None, block_mask=None,
                  block_q: int = 0, block_k: int = 0, rows=None):
    """Attention with score modifiers and a block-sparse mask, float64 (mlx-mfa 2.5.2
    feature list: "Softcap", "ALiBi", "Block-sparse attention"; mlx-mfa 2.61.0 "Native
    attn_bias" additive bias).

    q ``[B, Hq, Nq, D]``, k/v ``[B, Hkv, Nk, D]``.  The score of query ``i`` and key ``j``
    (``off = Nk - Nq``) is built in this order:

    * ``s = scale * q_i . k_j``;
    * softcap ``c > 0``: ``s = c * tanh(s / c)``;
    * ALiBi (``alibi_slopes[h]``, one per query head): ``s -= slope_h * |i + off - j|``;
    * additive bias (``bias`` of shape ``[B, Hq, Nk]``, a per-key bias broadcast over
      the queries): ``s += bias[b, h, j]``;

    then the causal / window visibility of ``attention`` and the block mask
    (``block_mask[b, h, i // block_q, j // block_k]`` true = computed) both remove keys,
    and the softmax runs over the remaining ones.  A row left with no key gives
    ``O = 0``, ``LSE = -inf``.  Returns ``(O, LSE)`` like ``attention``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    off = Nk - Nq
    cols = np.arange(Nk)

    def row_block(b, h, ii):
        kv = h // g
        s = scale * (q[b, h, ii] @ k[b, kv].T)
        if softcap > 0:
            s = softcap * np.tanh(s / softcap)
        if alibi_slopes is not None:
            s = s - float(alibi_slopes[h]) * np.abs(ii[:, None] + off - cols[None, :])
        if bias is not None:
            s = s + np.asarray(bias, dtype=np.float64)[b, h][None, :]
        vis = visible(ii[:, None], cols[None, :], Nq, Nk, causal, left, right)
        if block_mask is not None:
            bm = np.asarray(block_mask).astype(bool)[b, h]
            vis = vis & bm[ii[:, None] // block_q, cols[None, :] // block_k]
        s = np.where(vis, s, -np.inf)
        any_vis = vis.any(axis=1)
        m = np.where(any_vis, s.max(axis=1, initial=-np.inf), 0.0)
        e = np.exp(s - m[:, None])
        z = e.sum(axis=1)
        with np.errstate(invalid="ignore", divide="ignore"):
            p = np.where(any_vis[:, None], e / np.where(any_vis, z, 1.0)[:, None], 0.0)
            lse = np.where(any_vis, m + np.log(np.where(any_vis, z, 1.0)), -np.inf)
        return p @ v[b, kv], lse

    if rows is not None:
        rows = list(rows)
        O = np.zeros((len(rows), D))
        L = np.zeros(len(rows))
        for n, (b, h, i) in enumerate(rows):
            o, lse = row_block(b, h, np.array([i]))
            O[n], L[n] = o[0], lse[0]
        return O, L
    O = np.zeros((B, Hq, Nq, D))
    L = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            for r0 in range(0, Nq, 512):
                ii = np.arange(r0, min(Nq, r0 + 512))
                O[b, h, ii], L[b, h, ii] = row_block(b, h, ii)
    return O, L


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float,
                     causal: bool = False, left: int = -1, right: int = -1, rows=None):
    """Packed variable-length attention, float64 (mlx-mfa "Variable-length" feature:
    sequences packed back to back and delimited by ``cu_seqlens``).

    q ``[total_q, Hq, D]``, k/v ``[total_k, Hkv, D]``; sequence ``b`` owns query tokens
    ``cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1`` and keys ``cu_seqlens_k[b] ..
    cu_seqlens_k[b+1]-1``.  Each sequence is attended on its own, exactly as ``attention``
    would on ``[1, H, L, D]`` slices, so the causal / window alignment is bottom-right per
    sequence: ``off_b = Lk_b - Lq_b``.  (The mlx-mfa 2.5.2 page reports a correction of the
    varlen causal output for ``N_q < N_k`` without naming the convention; bottom-right is
    the reading under which a block of new queries after ``Lk_b - Lq_b`` cached keys sees
    them all, as chunked prefill needs.)  A sequence with queries but no keys gives
    ``O = 0`` and ``LSE = -inf`` on its rows.

    Returns O ``[total_q, Hq, D]`` and LSE ``[Hq, total_q]``; query tokens outside every
    sequence keep ``O = 0``, ``LSE = -inf``.  ``rows`` optionally restricts the work to a
    list of ``(token, head)`` pairs and then returns ``(O [n, D], LSE [n])``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    if len(cq) != len(ck) or len(cq) < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")
    if any(b < a for a, b in zip(cq[:-1], cq[1:])) or any(b < a for a, b in zip(ck[:-1], ck[1:])):
        raise ValueError("cu_seqlens must be non-decreasing")
    if cq[0] < 0 or ck[0] < 0 or cq[-1] > q.shape[0] or ck[-1] > k.shape[0]:
        raise ValueError("cu_seqlens out of range")
    total_q, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")

    def seq_views(b):
        qs = q[cq[b]:cq[b + 1]].transpose(1, 0, 2)[None]    # [1, Hq, Lq, D]
        ks = k[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]    # [1, Hkv, Lk, D]
        vs = v[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
        return qs, ks, vs

    if rows is not None:
        rows = list(rows)
        O = np.zeros((len(rows), D))
        L = np.full(len(rows), -np.inf)
        for n, (t, h) in enumerate(rows):
            b = next((s for s in range(len(cq) - 1) if cq[s] <= t < cq[s + 1]), None)
            if b is None or ck[b + 1] == ck[b]:
                continue
            qs, ks, vs = seq_views(b)
            o, lse = attention(qs, ks, vs, scale, causal, left, right, rows=[(0, h, t - cq[b])])
            O[n], L[n] = o[0], lse[0]
        return O, L
    O = np.zeros((total_q, Hq, D))
    L = np.full((Hq, total_q), -np.inf)
    for b in range(len(cq) - 1):
        if cq[b + 1] == cq[b] or ck[b + 1] == ck[b]:
            continue
        qs, ks, vs = seq_views(b)
        o, lse = attention(qs, ks, vs, scale, causal, left, right)
        O[cq[b]:cq[b + 1]] = o[0].transpose(1, 0, 2)
        L[:, cq[b]:cq[b + 1]] = lse[0]
    return O, L


def attention_varlen_paged(q, k_pages, v_pages, block_table, seq_lens_k, cu_seqlens_q,
                           scale: float, page_size: int, causal: bool = False, left: int = -1,
                           right: int = -1, rows=None):
    """Packed queries over a paged KV cache, float64 (mlx-mfa 2.5.2 capability
    table, packed variable-length queries over paged keys; MXFlashAttn paged-cache addressing).

    q ``[total_q, Hq, D]`` with sequence ``b`` owning query tokens ``cu_seqlens_q[b] ..
    cu_seqlens_q[b+1]-1``; its ``Lk_b = seq_lens_k[b]`` keys are gathered from the
    ``[P, page_size, Hkv, D]`` pools through ``block_table`` (``gather_paged``).  The result
    is ``attention_varlen`` over the gathered keys: each sequence on its own, bottom-right
    aligned.  Returns O ``[total_q, Hq, D]`` and LSE ``[Hq, total_q]`` (or the sampled rows).
    """
    q = np.asarray(q, dtype=np.float64)
    Hkv, D = k_pages.shape[2], k_pages.shape[3]
    B = len(seq_lens_k)
    ks, vs = [], []
    for b in range(B):
        n = int(seq_lens_k[b])
        ks.append(gather_paged(k_pages, block_table, b, n, page_size))
        vs.append(gather_paged(v_pages, block_table, b, n, page_size))
    k = np.concatenate(ks) if ks else np.zeros((0, Hkv, D))
    v = np.concatenate(vs) if vs else np.zeros((0, Hkv, D))
    cu_k = np.concatenate([[0], np.cumsum([int(x) for x in seq_lens_k])])
    return attention_varlen(q, k, v, cu_seqlens_q, cu_k, scale, causal, left, right, rows)


def attention_probs(q, k, scale: float, causal=False, left=-1, right=-1):
    """The probability matrix P ``[B, Hq, Nq, Nk]`` (small sizes only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    P = np.zeros((B, Hq, Nq, Nk))
    ii = np.arange(Nq)[:, None]
    jj = np.arange(Nk)[None, :]
    vis = visible(ii, jj, Nq, Nk, causal, left, right)
    for b in range(B):
        for h in range(Hq):
            _, _, p = _rows_attention(q[b, h], k[b, h // g], np.zeros((Nk, 1)), scale, vis)
            P[b, h] = p
    return P


def gather_paged(pages: np.ndarray, block_table: np.ndarray, b: int, L: int,
                 page_size: int) -> np.ndarray:
    """The first ``L`` tokens of sequence ``b`` from a ``[P, page_size, Hkv, D]`` pool.

    Token ``t`` sits at page ``block_table[b, t // page_size]``, slot
    ``t % page_size`` (the paged-cache addressing of the MXFlashAttn decode page).
    """
    out = np.empty((L,) + pages.shape[2:], dtype=pages.dtype)
    for t in range(L):
        page = int(block_table[b, t // page_size])
        if page < 0 or page >= pages.shape[0]:
            raise IndexError(f"block_table[{b}, {t // page_size}] = {page} out of range")
        out[t] = pages[page, t % page_size]
    return out


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale: float,
                 page_size: int):
    """Single-token decode over a paged KV cache, float64.

    q ``[B, Hq, D]``; pools ``[P, page_size, Hkv, D]`` (float64 values); every cached
    token of sequence ``b`` (``seq_lens[b]`` of them) is visible.  Returns O
    ``[B, Hq, D]`` and LSE ``[B, Hq]``.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_pages.shape[2]
    g = Hq // Hkv
    O = np.zeros((B, Hq, D))
    L = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        if n <= 0:
            continue
        kb = gather_paged(k_pages, block_table, b, n, page_size)  # [n, Hkv, D]
        vb = gather_paged(v_pages, block_table, b, n, page_size)
        for h in range(Hq):
            kv = h // g
            vis = np.ones((1, n), dtype=bool)
            o, lse, _ = _rows_attention(q[b, h][None, :], kb[:, kv], vb[:, kv], scale, vis)
            O[b, h] = o[0]
            L[b, h] = lse[0]
    return O, L


def decode_paged_multi(q, k_pages, v_pages, block_table, seq_lens, scale: float,
                       page_size: int):
    """Decode of ``Nq`` new tokens per sequence over a paged KV cache, float64 (mlx-mfa
    "Flash Decode" feature, which covers up to four new tokens; MTPLX verify attention).

    q ``[B, Nq, Hq, D]``; the ``seq_lens[b]`` cached tokens include the new ones, which are
    the last ``Nq`` positions, so new token ``n`` sees the keys at positions
    ``<= seq_lens[b] - Nq + n`` (bottom-right causal).  Returns O ``[B, Nq, Hq, D]`` and
    LSE ``[B, Nq, Hq]``.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Nq, Hq, D = q.shape
    O = np.zeros((B, Nq, Hq, D))
    L = np.full((B, Nq, Hq), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        if n <= 0:
            continue
        kb = gather_paged(k_pages, block_table, b, n, page_size).transpose(1, 0, 2)[None]
        vb = gather_paged(v_pages, block_table, b, n, page_size).transpose(1, 0, 2)[None]
        o, lse = attention(q[b].transpose(1, 0, 2)[None], kb, vb, scale, causal=True)
        O[b] = o[0].transpose(1, 0, 2)
        L[b] = lse[0].T
    return O, L


def lse_merge(parts):
    """Combine partial results over a partition of the keys.

    ``parts`` is a list of ``(O_s, LSE_s)`` where ``O_s`` is the normalised output of
    attention restricted to key subset ``s`` and ``LSE_s`` its log-sum-exp (``-inf``
    for an empty subset).  With ``M = max_s LSE_s`` and ``w_s = exp(LSE_s - M)``,
    the full result is ``O = sum_s w_s O_s / sum_s w_s`` and
    ``LSE = M + log(sum_s w_s)``.
    """
    lses = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])
    outs = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])
    M = lses.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Ms), 0.0)
    W = w.sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        O = (w[..., None] * outs).sum(axis=0) / np.where(W > 0, W, 1.0)[..., None]
        lse = np.where(W > 0, Ms + np.log(np.where(W > 0, W, 1.0)), -np.inf)
    return np.where((W > 0)[..., None], O, 0.0), lse


def visited_tiles(Nq: int, Nk: int, BM: int, BN: int, causal: bool, left: int,
                  right: int):
    """For each query tile, the sorted key-tile indices with >= 1 visible pair.

    Brute force over every ``(i, j)`` with ``i < Nq`` and ``j < Nk``.
    """
    n_qt = math.ceil(Nq / BM)
    n_kt = math.ceil(Nk / BN)
    out = []
    ii = np.arange(Nq)[:, None]
    jj = np.arange(Nk)[None, :]
    vis = visible(ii, jj, Nq, Nk, causal, left, right)
    for qt in range(n_qt):
        blk = vis[qt * BM: min(Nq, (qt + 1) * BM)]
        cols = blk.any(axis=0)
        tiles = [kt for kt in range(n_kt) if cols[kt * BN: min(Nk, (kt + 1) * BN)].any()]
        out.append(tiles)
    return out
