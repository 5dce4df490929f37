"""Pins for the CPU oracle: closed forms, invariants, an independent scalar
implementation and PyTorch's float64 attention routine.  CPU only.

Each ``pin_*`` function raises AssertionError on a mismatch; the tests call them on
the real oracle, and ``test_planted_mistakes`` plants plausible mistakes into the
oracle (on the CPU) to show that some pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest

import attn_inputs as A
import oracle
import oracle.reference as OA
from oracle.scalar import attention_scalar, attention_scalar_ext, logsumexp_scalar

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _fsum_dot(a, b):
    return math.fsum(float(x) * float(y) for x, y in zip(a, b))


# ----------------------------------------------------------------------------- pins

def pin_golden():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q, k, v = (np.array(c[n], dtype=np.float64) for n in ("q", "k", "v"))
        O, L = oracle.attention(q, k, v, c["scale"], c["causal"], c["left"], c["right"])
        np.testing.assert_allclose(O, np.array(c["O"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(L, np.array(c["LSE"]), rtol=0, atol=1e-14)


def pin_single_key():
    # Nk = 1: O = V[0] and LSE = scale * q.k0 (closed form), for every query row
    q, k, v = _rand((2, 4, 3, 8), 1), _rand((2, 2, 1, 8), 2), _rand((2, 2, 1, 8), 3)
    scale = 0.37
    O, L = oracle.attention(q, k, v, scale, causal=False)
    for b in range(2):
        for h in range(4):
            for i in range(3):
                assert np.allclose(O[b, h, i], v[b, h // 2, 0], atol=1e-13)
                assert abs(L[b, h, i] - scale * _fsum_dot(q[b, h, i], k[b, h // 2, 0])) < 1e-12


def pin_identical_keys():
    # all keys equal: every visible key has the same score s, so O is the plain mean of
    # the visible V rows and LSE = s + log(n_visible).  With causal + window (left=3),
    # row i sees keys max(0, i-3) .. i (inclusive reading): n = min(i, 3) + 1.
    Nq = Nk = 10
    q = _rand((1, 1, Nq, 4), 4)
    k = np.broadcast_to(_rand((1, 1, 1, 4), 5), (1, 1, Nk, 4)).copy()
    v = _rand((1, 1, Nk, 4), 6)
    scale = 0.5
    O, L = oracle.attention(q, k, v, scale, causal=True, left=3, right=0)
    for i in range(Nq):
        lo = max(0, i - 3)
        n = i - lo + 1
        s = scale * _fsum_dot(q[0, 0, i], k[0, 0, 0])
        mean = [math.fsum(v[0, 0, j, d] for j in range(lo, i + 1)) / n for d in range(4)]
        assert np.allclose(O[0, 0, i], mean, atol=1e-13), i
        assert abs(L[0, 0, i] - (s + math.log(n))) < 1e-12, i


def pin_causal_row0():
    q, k, v = _rand((1, 2, 6, 8), 7), _rand((1, 2, 6, 8), 8), _rand((1, 2, 6, 8), 9)
    O, L = oracle.attention(q, k, v, 0.3, causal=True)
    for h in range(2):
        assert np.allclose(O[0, h, 0], v[0, h, 0], atol=1e-14)
        assert abs(L[0, h, 0] - 0.3 * _fsum_dot(q[0, h, 0], k[0, h, 0])) < 1e-12


def pin_probs_sum_to_one():
    q, k = _rand((1, 2, 7, 5), 10), _rand((1, 1, 9, 5), 11)
    for causal, left, right in [(False, -1, -1), (True, -1, -1), (True, 2, 0), (False, 1, 1)]:
        P = oracle.attention_probs(q, k, 0.7, causal, left, right)
        s = P.sum(axis=-1)
        assert np.all(np.abs(s - 1.0) < 1e-12)
        assert np.all(P >= 0)


def pin_lse_bruteforce():
    # LSE against a pure-Python log-sum-exp of the visible scaled scores
    q, k, v = _rand((1, 2, 5, 6), 12), _rand((1, 2, 8, 6), 13), _rand((1, 2, 8, 6), 14)
    scale = 0.8
    _, L = oracle.attention(q, k, v, scale, causal=True)
    off = 8 - 5
    for h in range(2):
        for i in range(5):
            vals = [scale * _fsum_dot(q[0, h, i], k[0, h, j]) for j in range(i + off + 1)]
            assert abs(L[0, h, i] - logsumexp_scalar(vals)) < 1e-12


def pin_scalar_oracle():
    # independent pure-Python implementation on tiny inputs, GQA, Nq != Nk, all masks
    q, k, v = _rand((2, 4, 5, 3), 15), _rand((2, 2, 7, 3), 16), _rand((2, 2, 7, 3), 17)
    for causal, left, right in [(False, -1, -1), (True, -1, -1), (True, 2, 0), (False, 1, 2),
                                (True, 0, 0), (False, -1, 1)]:
        O, L = oracle.attention(q, k, v, 0.9, causal, left, right)
        Os, Ls = attention_scalar(q.tolist(), k.tolist(), v.tolist(), 0.9, causal, left, right)
        np.testing.assert_allclose(O, np.array(Os), atol=1e-13, rtol=0)
        np.testing.assert_array_equal(np.isinf(L), np.isinf(np.array(Ls)))
        fin = np.isfinite(L)
        np.testing.assert_allclose(L[fin], np.array(Ls)[fin], atol=1e-13, rtol=0)


def pin_wide_window_is_full():
    q, k, v = _rand((1, 2, 9, 4), 18), _rand((1, 2, 9, 4), 19), _rand((1, 2, 9, 4), 20)
    for causal in (False, True):
        O0, L0 = oracle.attention(q, k, v, 0.5, causal)
        O1, L1 = oracle.attention(q, k, v, 0.5, causal, left=9, right=9)
        O2, L2 = oracle.attention(q, k, v, 0.5, causal, left=100, right=-1)
        for O, L in ((O1, L1), (O2, L2)):
            np.testing.assert_array_equal(O, O0)
            np.testing.assert_array_equal(L, L0)


def pin_zero_window_is_identity():
    # (left=0, right=0): each row sees only key i+off -> O_i = V_{i+off}
    q, k, v = _rand((1, 1, 4, 5), 21), _rand((1, 1, 6, 5), 22), _rand((1, 1, 6, 5), 23)
    O, L = oracle.attention(q, k, v, 1.1, causal=False, left=0, right=0)
    for i in range(4):
        assert np.allclose(O[0, 0, i], v[0, 0, i + 2], atol=1e-14)
        assert abs(L[0, 0, i] - 1.1 * _fsum_dot(q[0, 0, i], k[0, 0, i + 2])) < 1e-12


def pin_gqa_is_repeated_mha():
    q, k, v = _rand((2, 6, 5, 4), 24), _rand((2, 2, 7, 4), 25), _rand((2, 2, 7, 4), 26)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)  # head h reads kv h // 3
    for causal in (False, True):
        O0, L0 = oracle.attention(q, k, v, 0.6, causal)
        O1, L1 = oracle.attention(q, kr, vr, 0.6, causal)
        np.testing.assert_array_equal(O0, O1)
        np.testing.assert_array_equal(L0, L1)


def pin_affine_v():
    q, k, v = _rand((1, 2, 6, 4), 27), _rand((1, 2, 6, 4), 28), _rand((1, 2, 6, 4), 29)
    c = np.array([0.5, -1.0, 2.0, 3.0])
    O0, L0 = oracle.attention(q, k, v, 0.4, True)
    O1, L1 = oracle.attention(q, k, 2.5 * v + c, 0.4, True)
    np.testing.assert_allclose(O1, 2.5 * O0 + c, atol=1e-12)
    np.testing.assert_array_equal(L0, L1)


def pin_torch_sdpa():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    q, k, v = _rand((2, 3, 33, 16), 30), _rand((2, 3, 33, 16), 31), _rand((2, 3, 33, 16), 32)
    for causal in (False, True):
        O, _ = oracle.attention(q, k, v, 0.25, causal)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                             torch.from_numpy(v), is_causal=causal, scale=0.25)
        np.testing.assert_allclose(O, ref.numpy(), atol=1e-12, rtol=0)


def pin_fully_masked_rows():
    # causal with Nq > Nk: rows i < Nq - Nk see nothing -> O = 0, LSE = -inf
    q, k, v = _rand((1, 1, 6, 3), 33), _rand((1, 1, 2, 3), 34), _rand((1, 1, 2, 3), 35)
    O, L = oracle.attention(q, k, v, 1.0, causal=True)
    assert np.all(O[0, 0, :4] == 0.0) and np.all(np.isneginf(L[0, 0, :4]))
    assert np.allclose(O[0, 0, 4], v[0, 0, 0]) and np.all(np.isfinite(L[0, 0, 4:]))


def pin_lse_merge_identity():
    # merging attention over any partition of the keys equals the one-shot result
    q, k, v = _rand((1, 2, 3, 5), 36), _rand((1, 2, 20, 5), 37), _rand((1, 2, 20, 5), 38)
    O, L = oracle.attention(q, k, v, 0.7)
    for cuts in ([0, 7, 20], [0, 1, 2, 3, 20], [0, 20], [0, 5, 5, 12, 20]):
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            if a == b:
                parts.append((np.zeros_like(O), np.full_like(L, -np.inf)))  # empty split
            else:
                parts.append(oracle.attention(q, k[:, :, a:b], v[:, :, a:b], 0.7))
        Om, Lm = oracle.lse_merge(parts)
        np.testing.assert_allclose(Om, O, atol=1e-12, rtol=0)
        np.testing.assert_allclose(Lm, L, atol=1e-12, rtol=0)


def pin_decode_paged():
    # paged decode equals (i) attention on the contiguous tokens and (ii) the last row
    # of causal prefill over the same tokens; and is invariant to the page permutation
    p = A.paged_inputs(3, 4, 2, 8, "f16", 40, len_lo=1, len_hi=50, extra_pages=3)
    kp, vp, q = (oracle.widen(x, "f16") for x in (p.k_pages, p.v_pages, p.q))
    O, L = oracle.decode_paged(q, kp, vp, p.block_table, p.seq_lens, 0.3, p.page_size)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    # rebuild the contiguous tokens from the generator's own draw order
    rng = np.random.default_rng(40)
    rng.integers(1, 50, endpoint=True, size=3)
    total_pages = p.pages_used + 3
    rng.permutation(total_pages)
    A._normal_bits(rng, (3, 4, 8), "f16")
    tot = int(p.seq_lens.sum())
    kt = oracle.widen(A._normal_bits(rng, (tot, 2, 8), "f16"), "f16")
    vt = oracle.widen(A._normal_bits(rng, (tot, 2, 8), "f16"), "f16")
    t0 = 0
    for b in range(3):
        n = int(p.seq_lens[b])
        kk = kt[t0:t0 + n].transpose(1, 0, 2)[None]
        vv = vt[t0:t0 + n].transpose(1, 0, 2)[None]
        t0 += n
        O1, L1 = oracle.attention(q[b][None, :, None, :], kk, vv, 0.3)
        np.testing.assert_allclose(O[b], O1[0, :, 0], atol=1e-13)
        np.testing.assert_allclose(L[b], L1[0, :, 0], atol=1e-13)
        # decode(L) == last row of causal prefill whose last query is q
        qq = np.concatenate([_rand((1, 4, n - 1, 8), 41 + b), q[b][None, :, None, :]], axis=2)
        O2, L2 = oracle.attention(qq, kk, vv, 0.3, causal=True)
        np.testing.assert_allclose(O[b], O2[0, :, -1], atol=1e-13)
        np.testing.assert_allclose(L[b], L2[0, :, -1], atol=1e-13)
    # a different physical placement of the same pages gives the same result
    perm = np.random.default_rng(7).permutation(kp.shape[0])
    inv = np.argsort(perm)
    bt2 = np.where(p.block_table >= 0, inv[np.maximum(p.block_table, 0)], -1)
    O3, L3 = oracle.decode_paged(q, kp[perm], vp[perm], bt2, p.seq_lens, 0.3, p.page_size)
    np.testing.assert_array_equal(O3, O)
    np.testing.assert_array_equal(L3, L)


def pin_visited_tiles():
    # closed-form tile counts: causal Nq=Nk=N with BM=2*BN visits 2(qt+1) tiles per
    # q-tile; a window of left=W, right=0 visits at most ceil((BM + W) / BN) + 1.
    t = oracle.visited_tiles(512, 512, 128, 64, True, -1, -1)
    assert [len(x) for x in t] == [2, 4, 6, 8]
    assert t[1] == [0, 1, 2, 3]
    t = oracle.visited_tiles(100, 100, 32, 16, False, -1, -1)
    assert all(x == list(range(7)) for x in t)
    t = oracle.visited_tiles(1024, 1024, 128, 64, True, 128, 0)
    assert t[0] == [0, 1] and t[3] == [4, 5, 6, 7]
    for qt, tiles in enumerate(t):
        q0, q1 = 128 * qt, 128 * qt + 127
        lo, hi = max(0, q0 - 128), q1
        assert tiles == list(range(lo // 64, hi // 64 + 1)), (qt, tiles)
    # bottom-right alignment: Nq=1, Nk=1000 causal visits every key tile
    assert oracle.visited_tiles(1, 1000, 128, 64, True, -1, -1) == [list(range(16))]
    # Nq > Nk causal: the first query tile is entirely masked
    assert oracle.visited_tiles(256, 64, 128, 64, True, -1, -1)[0] == []


def pin_window_workload_pairs():
    # the sliding-window workload (N=8192, causal, left=512, right=0): the inclusive reading gives
    # min(i, 512) + 1 visible keys per row.
    N, W = 8192, 512
    i = np.arange(N)
    lo, hi = oracle.window_bounds(i, N, N, True, W, 0)
    n = hi - lo + 1
    assert np.array_equal(n, np.minimum(i, W) + 1)
    assert int(n.sum()) == 4_071_168


def _sdpa_with_lse(torch, q, k, v, scale, mask):
    """torch's float64 attention plus a torch logsumexp of the masked scores.

    q ``[Lq, Hq, D]``, k/v ``[Lk, Hkv, D]`` numpy; mask ``[Lq, Lk]`` bool tensor (True =
    visible).  Grouped heads go through SDPA's own ``enable_gqa`` head mapping.
    """
    F = torch.nn.functional
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                       enable_gqa=True)
    kk = tk.repeat_interleave(q.shape[1] // k.shape[1], dim=1)
    sc = (tq @ kk.transpose(-1, -2)) * scale
    lse = torch.logsumexp(sc.masked_fill(~mask, float("-inf")), dim=-1)
    return o[0].permute(1, 0, 2).numpy(), lse[0].numpy()


def pin_varlen_block_diagonal():
    # equal query / key lengths: packed attention is one attention over the concatenated
    # tokens with a block-diagonal mask (lower-triangular blocks when causal), built by
    # torch.block_diag / torch.tril and evaluated by torch's float64 SDPA
    torch = pytest.importorskip("torch")
    lens = [5, 1, 12, 7]
    T = sum(lens)
    q, k, v = _rand((T, 4, 8), 50), _rand((T, 2, 8), 51), _rand((T, 2, 8), 52)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    for causal in (False, True):
        O, L = oracle.attention_varlen(q, k, v, cu, cu, 0.4, causal)
        blocks = [torch.ones(n, n, dtype=torch.bool) for n in lens]
        if causal:
            blocks = [torch.tril(b) for b in blocks]
        Or, Lr = _sdpa_with_lse(torch, q, k, v, 0.4, torch.block_diag(*blocks))
        np.testing.assert_allclose(O, Or, atol=1e-12, rtol=0)
        np.testing.assert_allclose(L, Lr, atol=1e-12, rtol=0)


def pin_varlen_lower_right():
    # chunked-prefill packing (Lq_b <= Lk_b): each sequence equals torch's float64 SDPA
    # under its bottom-right causal bias (torch.nn.attention.bias.causal_lower_right)
    torch = pytest.importorskip("torch")
    from torch.nn.attention.bias import causal_lower_right
    lq, lk = [3, 1, 9, 4], [10, 6, 9, 30]
    q = _rand((sum(lq), 4, 8), 53)
    k, v = _rand((sum(lk), 1, 8), 54), _rand((sum(lk), 1, 8), 55)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    O, L = oracle.attention_varlen(q, k, v, cq, ck, 0.3, causal=True)
    for b in range(4):
        mask = causal_lower_right(lq[b], lk[b])._materialize()
        Or, Lr = _sdpa_with_lse(torch, q[cq[b]:cq[b + 1]], k[ck[b]:ck[b + 1]], v[ck[b]:ck[b + 1]],
                                0.3, mask)
        np.testing.assert_allclose(O[cq[b]:cq[b + 1]], Or, atol=1e-12, rtol=0)
        np.testing.assert_allclose(L[:, cq[b]:cq[b + 1]], Lr, atol=1e-12, rtol=0)


def pin_varlen_window_scalar():
    # sliding windows with Lq_b != Lk_b agree, sequence by sequence, with the independent
    # pure-Python implementation (which takes off = Nk - Nq itself)
    lq, lk = [4, 6, 2], [7, 6, 9]
    q = _rand((sum(lq), 2, 3), 56)
    k, v = _rand((sum(lk), 2, 3), 57), _rand((sum(lk), 2, 3), 58)
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    for causal, left, right in ((False, 2, 1), (True, 3, -1), (False, -1, 0), (True, 0, 0)):
        O, L = oracle.attention_varlen(q, k, v, cq, ck, 0.9, causal, left, right)
        for b in range(3):
            qs = q[cq[b]:cq[b + 1]].transpose(1, 0, 2)[None].tolist()
            ks = k[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None].tolist()
            vs = v[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None].tolist()
            Os, Ls = attention_scalar(qs, ks, vs, 0.9, causal, left, right)
            np.testing.assert_allclose(O[cq[b]:cq[b + 1]], np.array(Os[0]).transpose(1, 0, 2),
                                       atol=1e-13, rtol=0)
            np.testing.assert_allclose(L[:, cq[b]:cq[b + 1]], np.array(Ls[0]), atol=1e-13, rtol=0)


def pin_varlen_empty_and_isolated():
    # a sequence with no queries, one with queries but no keys (O = 0, LSE = -inf) and
    # padding tokens after the last sequence; rows of one sequence do not depend on the
    # tokens of any other
    lq, lk = [3, 0, 4, 2], [5, 2, 0, 6]
    q = _rand((sum(lq) + 2, 2, 4), 59)
    k, v = _rand((sum(lk) + 3, 1, 4), 60), _rand((sum(lk) + 3, 1, 4), 61)
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    O, L = oracle.attention_varlen(q, k, v, cq, ck, 0.5, causal=True)
    assert np.all(O[3:7] == 0.0) and np.all(np.isneginf(L[:, 3:7]))     # no keys
    assert np.all(O[9:] == 0.0) and np.all(np.isneginf(L[:, 9:]))       # padding
    assert np.all(np.isfinite(L[:, :3])) and np.all(np.isfinite(L[:, 7:9]))
    # sequence 3 (Lq 2, Lk 6): the last query sees all 6 keys, the first 5 of them
    np.testing.assert_allclose(O[8, 0], _ORIG_ATT(q[8:9].transpose(1, 0, 2)[None], k[7:13, :, :].transpose(1, 0, 2)[None],
                                                  v[7:13].transpose(1, 0, 2)[None], 0.5)[0][0, 0, 0], atol=1e-13)
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[:5] += 1.0
    v2[:5] *= -3.0
    q2[:3] += 2.0
    O2, L2 = oracle.attention_varlen(q2, k2, v2, cq, ck, 0.5, causal=True)
    np.testing.assert_array_equal(O2[3:], O[3:])
    np.testing.assert_array_equal(L2[:, 3:], L[:, 3:])
    # the row-sampling form returns the same rows (up to the BLAS summation order)
    rows = [(0, 1), (2, 0), (4, 1), (8, 0), (9, 1)]
    Or, Lr = oracle.attention_varlen(q, k, v, cq, ck, 0.5, causal=True, rows=rows)
    for n, (t, h) in enumerate(rows):
        np.testing.assert_allclose(Or[n], O[t, h], atol=1e-14, rtol=0)
        assert Lr[n] == L[h, t] or abs(Lr[n] - L[h, t]) <= 1e-14


def _paged_varlen_tokens(seed, Hq, Hkv, D, lq, ctx, extra_pages):
    """The contiguous Q, K, V tokens of a paged_varlen_inputs draw, redrawn in its order."""
    lq, ctx = np.asarray(lq), np.asarray(ctx)
    lk = lq + ctx
    rng = np.random.default_rng(seed)
    rng.permutation(int(sum(-(-int(L) // 16) for L in lk)) + extra_pages)
    q = oracle.widen(A._normal_bits(rng, (int(lq.sum()), Hq, D), "bf16"), "bf16")
    k = oracle.widen(A._normal_bits(rng, (int(lk.sum()), Hkv, D), "bf16"), "bf16")
    v = oracle.widen(A._normal_bits(rng, (int(lk.sum()), Hkv, D), "bf16"), "bf16")
    return q, k, v, lk


def pin_varlen_paged():
    # chunked prefill over pages: each sequence equals torch's float64 SDPA under its
    # bottom-right causal bias on the contiguous tokens (all ctx + new keys); a one-token
    # chunk equals paged decode; moving the pages in the pool changes nothing
    torch = pytest.importorskip("torch")
    from torch.nn.attention.bias import causal_lower_right
    lq, ctx = [5, 1, 17, 3], [40, 9, 0, 64]
    p = A.paged_varlen_inputs(4, 2, 8, "bf16", 70, seqlens_q=lq, ctx_lens=ctx, extra_pages=2)
    kp, vp, q = (oracle.widen(x, "bf16") for x in (p.k_pages, p.v_pages, p.q))
    O, L = oracle.attention_varlen_paged(q, kp, vp, p.block_table, p.seq_lens_k, p.cu_seqlens_q,
                                         0.35, 16, causal=True)
    qt, kt, vt, lk = _paged_varlen_tokens(70, 4, 2, 8, lq, ctx, 2)
    np.testing.assert_array_equal(qt, q)
    cq = p.cu_seqlens_q
    ck = np.concatenate([[0], np.cumsum(lk)])
    for b in range(4):
        mask = causal_lower_right(lq[b], int(lk[b]))._materialize()
        Or, Lr = _sdpa_with_lse(torch, q[cq[b]:cq[b + 1]], kt[ck[b]:ck[b + 1]], vt[ck[b]:ck[b + 1]],
                                0.35, mask)
        np.testing.assert_allclose(O[cq[b]:cq[b + 1]], Or, atol=1e-12, rtol=0)
        np.testing.assert_allclose(L[:, cq[b]:cq[b + 1]], Lr, atol=1e-12, rtol=0)
    # sequence 1 has a one-token chunk: it is paged decode of that token
    Od, Ld = oracle.decode_paged(q[cq[1]:cq[2]], kp, vp, p.block_table[1:2], p.seq_lens_k[1:2],
                                 0.35, 16)
    np.testing.assert_allclose(O[cq[1]], Od[0], atol=1e-13, rtol=0)
    np.testing.assert_allclose(L[:, cq[1]], Ld[0], atol=1e-13, rtol=0)
    perm = np.random.default_rng(3).permutation(kp.shape[0])
    inv = np.argsort(perm)
    bt2 = np.where(p.block_table >= 0, inv[np.maximum(p.block_table, 0)], -1)
    O3, L3 = oracle.attention_varlen_paged(q, kp[perm], vp[perm], bt2, p.seq_lens_k, cq, 0.35, 16,
                                           causal=True)
    np.testing.assert_array_equal(O3, O)
    np.testing.assert_array_equal(L3, L)


def pin_decode_multi():
    # Nq new tokens over the paged cache: one token equals paged decode; every sequence
    # equals torch's float64 SDPA with the bottom-right causal bias on its gathered keys
    torch = pytest.importorskip("torch")
    from torch.nn.attention.bias import causal_lower_right
    p = A.paged_multi_inputs(3, 3, 4, 2, 8, "f16", 80, len_lo=3, len_hi=60, extra_pages=2)
    q, kp, vp = (oracle.widen(x, "f16") for x in (p.q, p.k_pages, p.v_pages))
    O, L = oracle.decode_paged_multi(q, kp, vp, p.block_table, p.seq_lens, 0.4, 16)
    for b in range(3):
        n = int(p.seq_lens[b])
        kb = oracle.gather_paged(kp, p.block_table, b, n, 16)
        vb = oracle.gather_paged(vp, p.block_table, b, n, 16)
        Or, Lr = _sdpa_with_lse(torch, q[b], kb, vb, 0.4, causal_lower_right(3, n)._materialize())
        np.testing.assert_allclose(O[b], Or, atol=1e-12, rtol=0)
        np.testing.assert_allclose(L[b], Lr.T, atol=1e-12, rtol=0)
    O1, L1 = oracle.decode_paged_multi(q[:, 2:], kp, vp, p.block_table, p.seq_lens, 0.4, 16)
    Od, Ld = oracle.decode_paged(q[:, 2], kp, vp, p.block_table, p.seq_lens, 0.4, 16)
    np.testing.assert_allclose(O1[:, 0], Od, atol=1e-13, rtol=0)
    np.testing.assert_allclose(L1[:, 0], Ld, atol=1e-13, rtol=0)


def pin_ext_scalar():
    # softcap, ALiBi, key bias and a block mask together, against the independent scalar
    # implementation on tiny inputs (Nq != Nk, GQA)
    q, k, v = _rand((1, 4, 5, 3), 90, 2.0), _rand((1, 2, 7, 3), 91, 2.0), _rand((1, 2, 7, 3), 92)
    slopes = [0.5, 0.25, 0.125, 0.0625]
    bias = _rand((1, 4, 7), 93)
    bm = (np.random.default_rng(94).random((1, 4, 3, 4)) > 0.3)
    for causal, left, right, sc in ((True, -1, -1, 3.0), (False, 2, 1, 0.0), (False, -1, -1, 1.5)):
        O, L = oracle.attention_ext(q, k, v, 0.7, causal, left, right, softcap=sc,
                                    alibi_slopes=slopes, bias=bias, block_mask=bm, block_q=2,
                                    block_k=2)
        Os, Ls = attention_scalar_ext(q.tolist(), k.tolist(), v.tolist(), 0.7, causal, left, right,
                                      sc, slopes, bias.tolist(), bm.tolist(), 2, 2)
        np.testing.assert_allclose(O, np.array(Os), atol=1e-13, rtol=0)
        np.testing.assert_allclose(L, np.array(Ls), atol=1e-13, rtol=0)


def pin_ext_bias_torch():
    # the per-key bias is torch's float attn_mask broadcast over the query rows (float64
    # SDPA); with ALiBi under the causal mask, -slope * (i + off - j) differs from the key
    # bias slope * j only by a per-row constant, which the softmax removes and the LSE keeps
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    q, k, v = _rand((2, 3, 9, 8), 95), _rand((2, 3, 12, 8), 96), _rand((2, 3, 12, 8), 97)
    bias = _rand((2, 3, 12), 98)
    O, L = oracle.attention_ext(q, k, v, 0.3, bias=bias)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=torch.from_numpy(bias)[:, :, None, :], scale=0.3)
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-12, rtol=0)
    slopes = np.array([0.3, 0.1, 0.02])
    Oa, La = oracle.attention_ext(q, k, v, 0.3, causal=True, alibi_slopes=slopes)
    kb = np.broadcast_to(slopes[None, :, None] * np.arange(12)[None, None, :], (2, 3, 12))
    Ob, Lb = oracle.attention_ext(q, k, v, 0.3, causal=True, bias=kb)
    np.testing.assert_allclose(Oa, Ob, atol=1e-12, rtol=0)
    i = np.arange(9)
    np.testing.assert_allclose(La, Lb - slopes[None, :, None] * (i + 3)[None, None, :], atol=1e-12,
                               rtol=0)


def pin_ext_limits_and_blocks():
    # softcap -> infinity and zero slopes give plain attention; an all-true block mask
    # changes nothing; a block mask equals torch's float64 SDPA with the block mask
    # expanded element-wise (np.kron) as a boolean attn_mask
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    q, k, v = _rand((1, 2, 10, 4), 99), _rand((1, 2, 10, 4), 100), _rand((1, 2, 10, 4), 101)
    O0, L0 = oracle.attention(q, k, v, 0.5, True)
    O1, L1 = oracle.attention_ext(q, k, v, 0.5, True, softcap=1e9, alibi_slopes=[0.0, 0.0],
                                  block_mask=np.ones((1, 2, 5, 4), bool), block_q=2, block_k=3)
    np.testing.assert_allclose(O1, O0, atol=1e-12, rtol=0)
    np.testing.assert_allclose(L1, L0, atol=1e-12, rtol=0)
    for shape, bq, bk in (((1, 2, 5, 4), 2, 3), ((1, 2, 5, 5), 2, 2)):
        bm = np.random.default_rng(102).random(shape) > 0.4
        bm[..., 0] = True   # every row keeps a key block
        Ob, _ = oracle.attention_ext(q, k, v, 0.5, block_mask=bm, block_q=bq, block_k=bk)
        for h in range(2):
            full = np.kron(bm[0, h], np.ones((bq, bk), bool))[:10, :10]
            ref = F.scaled_dot_product_attention(torch.from_numpy(q[:, h:h + 1]),
                                                 torch.from_numpy(k[:, h:h + 1]),
                                                 torch.from_numpy(v[:, h:h + 1]),
                                                 attn_mask=torch.from_numpy(full), scale=0.5)
            np.testing.assert_allclose(Ob[:, h:h + 1], ref.numpy(), atol=1e-12, rtol=0)
    # a tiny softcap squeezes every score into (-c, c): the weights approach uniform
    Oc, Lc = oracle.attention_ext(q, k, v, 0.5, softcap=1e-9)
    np.testing.assert_allclose(Oc[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (10, 4)), atol=1e-8)
    np.testing.assert_allclose(Lc, np.log(10.0), atol=1e-8)


def pin_backward_torch_autograd():
    # the gradients equal torch's float64 autograd through its SDPA routine (dense, causal,
    # GQA through SDPA's own head mapping, and a window given as a boolean mask)
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    q, k, v = _rand((2, 4, 11, 8), 110), _rand((2, 2, 13, 8), 111), _rand((2, 2, 13, 8), 112)
    do = _rand((2, 4, 11, 8), 113)
    for causal, left, right in ((False, -1, -1), (True, -1, -1), (False, 3, 1)):
        dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.45, causal, left, right)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
        mask = None
        if causal:
            from torch.nn.attention.bias import causal_lower_right
            mask = causal_lower_right(11, 13)._materialize()
        elif left >= 0:
            i = torch.arange(11)[:, None] + 2
            j = torch.arange(13)[None, :]
            mask = (j >= i - left) & (j <= i + right)
        o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.45, enable_gqa=True)
        o.backward(torch.from_numpy(do))
        np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12, rtol=0)
        np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12, rtol=0)
        np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12, rtol=0)


def pin_backward_finite_differences():
    # central differences of L = sum(dO * O) through the oracle's forward, on every input
    # element of a tiny causal GQA problem with Nq < Nk
    q, k, v = _rand((1, 2, 3, 4), 114), _rand((1, 1, 5, 4), 115), _rand((1, 1, 5, 4), 116)
    do = _rand((1, 2, 3, 4), 117)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.8, causal=True)

    def loss(qq, kk, vv):
        return float((oracle.attention(qq, kk, vv, 0.8, causal=True)[0] * do).sum())

    eps = 1e-6
    for x, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            num[idx] = (up - loss(*args)) / (2 * eps)
        np.testing.assert_allclose(grad, num, atol=1e-7, rtol=0)


def pin_backward_masked_keys_and_rows():
    # keys no row sees get zero dK and dV; rows that see no key get zero dQ (causal Nq > Nk);
    # a row that sees a single key has P = 1 there, so dS = dP - D = 0 and its dQ is zero
    q, k, v = _rand((1, 1, 6, 3), 118), _rand((1, 1, 4, 3), 119), _rand((1, 1, 4, 3), 120)
    do = _rand((1, 1, 6, 3), 121)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.5, causal=True)
    assert np.all(dq[0, 0, :2] == 0)
    assert np.all(np.abs(dq[0, 0, 2]) < 1e-15)
    assert np.all(np.abs(dq[0, 0, 3:]).sum(axis=1) > 0)
    # Nq = 3, Nk = 4, off = 1, causal with window (0, 0): row i sees key i + 1 only, so
    # key 0 is seen by no row
    dq, dk, dv = oracle.attention_backward(q[:, :, :3], k, v, do[:, :, :3], 0.5, True, 0, 0)
    assert np.all(dk[0, 0, 0] == 0) and np.all(dv[0, 0, 0] == 0)


def _widen_by_fields(bits, dtype):
    """Value of 16-bit patterns from the IEEE binary16 / bfloat16 field definitions: sign,
    exponent (5 bits, bias 15 / 8 bits, bias 127), fraction (10 / 7 bits) with an implicit
    leading 1 for normal numbers; exponent 0 = subnormal, all ones = inf (fraction 0) or NaN.
    Integer fields and exact ldexp only."""
    b = np.asarray(bits, dtype=np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    ebits, fbits, bias = (5, 10, 15) if dtype == "f16" else (8, 7, 127)
    e = (b >> fbits) & ((1 << ebits) - 1)
    f = b & ((1 << fbits) - 1)
    emax = (1 << ebits) - 1
    normal = sign * np.ldexp((f + (1 << fbits)).astype(np.float64), e - bias - fbits)
    sub = sign * np.ldexp(f.astype(np.float64), 1 - bias - fbits)
    val = np.where(e == 0, sub, normal)
    special = np.where(f == 0, sign * np.inf, np.nan)
    return np.where(e == emax, special, val)


def pin_widen_every_bit_pattern():
    # widen turns the stored 16-bit patterns into float64 on both sides of every parity
    # check: all 65,536 patterns of each type against the field definitions and against
    # torch's own float16 / bfloat16 -> float64 conversions (NaNs compared as NaNs,
    # zeros by sign), plus fixed values that tell the two types apart
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        got = oracle.widen(bits, dt)
        ref = _widen_by_fields(bits, dt)
        ref_t = torch.from_numpy(bits.view(np.int16)).view(tdt).to(torch.float64).numpy()
        for r in (ref, ref_t):
            assert np.array_equal(np.isnan(got), np.isnan(r)), dt
            ok = ~np.isnan(r)
            assert np.array_equal(got[ok], r[ok]), dt
            assert np.array_equal(np.signbit(got[ok]), np.signbit(r[ok])), dt
    fixed = {
        "f16": {0x3C00: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -24, 0x7BFF: 65504.0, 0x7C00: np.inf,
                0xFC00: -np.inf, 0x3F80: 1.875, 0x0400: 2.0 ** -14, 0x3555: (1 + 0x155 / 1024) * 2.0 ** -2},
        "bf16": {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127,
                 0x7F80: np.inf, 0xFF80: -np.inf, 0x3C00: 2.0 ** -7, 0x0080: 2.0 ** -126},
    }
    for dt, table in fixed.items():
        pats = np.array(list(table), dtype=np.uint16)
        assert np.array_equal(oracle.widen(pats, dt), np.array(list(table.values()))), dt
    assert np.signbit(oracle.widen(np.array([0x8000], np.uint16), "f16")[0])
    assert np.isnan(oracle.widen(np.array([0x7E00], np.uint16), "f16")[0])
    assert np.isnan(oracle.widen(np.array([0x7FC0], np.uint16), "bf16")[0])


def pin_probs_gqa():
    # attention_probs with grouped query heads (g = 2, two distinct KV heads, Nq != Nk):
    # equal to the same call on explicitly repeated K heads (consecutive grouping), and
    # P V equal to the scalar path's output; one row against a brute-force softmax
    q, k, v = _rand((2, 4, 5, 3), 70), _rand((2, 2, 6, 3), 71), _rand((2, 2, 6, 3), 72)
    k_rep = np.repeat(k, 2, axis=1)
    for causal, left, right in [(False, -1, -1), (True, -1, -1), (True, 1, 0), (False, 0, 2)]:
        P = oracle.attention_probs(q, k, 0.8, causal, left, right)
        P_rep = oracle.attention_probs(q, k_rep, 0.8, causal, left, right)
        np.testing.assert_allclose(P, P_rep, atol=1e-15, rtol=0)
        Os, _ = attention_scalar(q.tolist(), k.tolist(), v.tolist(), 0.8, causal, left, right)
        for b in range(2):
            for h in range(4):
                np.testing.assert_allclose(P[b, h] @ v[b, h // 2], np.array(Os[b][h]), atol=1e-13,
                                           rtol=0)
    # row i = 4 of head 3 (KV head 1), non-causal: softmax of all 6 scaled scores
    P = oracle.attention_probs(q, k, 0.8)
    sc = [0.8 * _fsum_dot(q[1, 3, 4], k[1, 1, j]) for j in range(6)]
    z = math.fsum(math.exp(x) for x in sc)
    np.testing.assert_allclose(P[1, 3, 4], [math.exp(x) / z for x in sc], atol=1e-15, rtol=0)


PINS = [pin_golden, pin_single_key, pin_identical_keys, pin_causal_row0, pin_probs_sum_to_one,
        pin_lse_bruteforce, pin_scalar_oracle, pin_wide_window_is_full,
        pin_zero_window_is_identity, pin_gqa_is_repeated_mha, pin_affine_v, pin_torch_sdpa,
        pin_fully_masked_rows, pin_lse_merge_identity, pin_decode_paged, pin_visited_tiles,
        pin_window_workload_pairs, pin_varlen_block_diagonal, pin_varlen_lower_right,
        pin_varlen_window_scalar, pin_varlen_empty_and_isolated, pin_varlen_paged,
        pin_decode_multi, pin_ext_scalar, pin_ext_bias_torch, pin_ext_limits_and_blocks,
        pin_backward_torch_autograd, pin_backward_finite_differences,
        pin_backward_masked_keys_and_rows, pin_widen_every_bit_pattern, pin_probs_gqa]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ------------------------------------------------------------- planted mistakes

def _caught(monkeypatch_ctx, pins):
    """True if at least one pin fails under the planted mistake."""
    for pin in pins:
        try:
            pin()
        except AssertionError:
            return True
        except (ValueError, IndexError, FloatingPointError):
            return True
    return False


def _mut_exclusive_window(i, j, Nq, Nk, causal, left, right):
    # plausible mistake: exclusive left window end (P5-style "w keys" off by one)
    ok = _ORIG_VISIBLE(i, j, Nq, Nk, causal, left, right)
    if left >= 0:
        ok = ok & (np.asarray(j) > np.asarray(i) + (Nk - Nq) - left)
    return ok


def _mut_top_left_causal(i, j, Nq, Nk, causal, left, right):
    # plausible mistake: top-left causal alignment for Nq != Nk
    return _ORIG_VISIBLE(i, j, Nk, Nk, causal, left, right)


def _mut_rows_no_scale(qr, kk, vv, scale, vis):
    return _ORIG_ROWS(qr, kk, vv, 1.0, vis)


def _mut_rows_lse_no_max(qr, kk, vv, scale, vis):
    o, lse, p = _ORIG_ROWS(qr, kk, vv, scale, vis)
    s = scale * (qr @ kk.T)
    m = np.where(vis, s, -np.inf).max(axis=1, initial=-np.inf)
    return o, np.where(np.isfinite(lse), lse - np.where(np.isfinite(m), m, 0.0), lse), p


def _mut_rows_transposed_v(qr, kk, vv, scale, vis):
    # plausible mistake: contract P with V along the wrong axis when shapes allow it
    o, lse, p = _ORIG_ROWS(qr, kk, vv, scale, vis)
    if vv.shape[0] == vv.shape[1]:
        o = p @ vv.T
    return o, lse, p


def _mut_rows_sign(qr, kk, vv, scale, vis):
    return _ORIG_ROWS(qr, kk, vv, -scale, vis)


def _mut_merge_unweighted(parts):
    outs = [p[0] for p in parts]
    O, L = _ORIG_MERGE(parts)
    return np.mean(outs, axis=0), L


_ORIG_VISIBLE = OA.visible
_ORIG_ROWS = OA._rows_attention
_ORIG_MERGE = OA.lse_merge


def _gqa_mod_attention(q, k, v, scale, causal=False, left=-1, right=-1, rows=None, row_block=512):
    # plausible mistake: head h reads KV head h % Hkv instead of h // g
    Hq, Hkv = q.shape[1], k.shape[1]
    idx = np.arange(Hq) % Hkv
    return _ORIG_ATT(q, np.asarray(k)[:, idx], np.asarray(v)[:, idx], scale, causal, left, right,
                     rows, row_block)


_ORIG_ATT = OA.attention

def _mut_varlen_no_isolation(q, k, v, cu_q, cu_k, scale, causal=False, left=-1, right=-1,
                             rows=None):
    # plausible mistake: every sequence attends to the keys of the whole pack
    tk = np.asarray(k).shape[0]
    cq = np.asarray(cu_q)
    return _ORIG_VARLEN(q, k, v, cq, np.concatenate([[0], np.full(len(cq) - 1, tk)]), scale,
                        causal, left, right, rows)


def _mut_varlen_top_left(q, k, v, cu_q, cu_k, scale, causal=False, left=-1, right=-1, rows=None):
    # plausible mistake: top-left causal alignment inside each sequence (key j visible to
    # query i iff j <= i), i.e. only the first Lq_b keys of a longer sequence ever count
    cq, ck = np.asarray(cu_q), np.asarray(cu_k)
    lq = cq[1:] - cq[:-1]
    lk = ck[1:] - ck[:-1]
    keep = np.minimum(lk, lq) if causal else lk
    idx = np.concatenate([np.arange(ck[b], ck[b] + keep[b]) for b in range(len(lq))]).astype(int)
    ck2 = np.concatenate([[0], np.cumsum(keep)])
    return _ORIG_VARLEN(q, np.asarray(k)[idx], np.asarray(v)[idx], cq, ck2, scale, causal, left,
                        right, rows)


_ORIG_VARLEN = OA.attention_varlen


def _mut_varlen_paged_context_only(q, k_pages, v_pages, block_table, seq_lens_k, cu_seqlens_q,
                                  scale, page_size, causal=False, left=-1, right=-1, rows=None):
    # plausible mistake: the new tokens' own keys are left out (Lk = context length only)
    lq = np.diff(np.asarray(cu_seqlens_q))
    ctx = np.maximum(np.asarray(seq_lens_k) - lq, 0)
    return _ORIG_VARLEN_PAGED(q, k_pages, v_pages, block_table, ctx, cu_seqlens_q, scale,
                              page_size, causal, left, right, rows)


_ORIG_VARLEN_PAGED = OA.attention_varlen_paged
_ORIG_EXT = OA.attention_ext
_ORIG_BWD = OA.attention_backward


def _mut_bwd_no_dvec(q, k, v, dout, scale, causal=False, left=-1, right=-1):
    # plausible mistake: dS = P * dP (the D-vector term dropped)
    q64, k64, v64, do64 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    dq, dk, dv = _ORIG_BWD(q64, k64, v64, do64, scale, causal, left, right)
    O, _ = OA.attention(q64, k64, v64, scale, causal, left, right)
    # adding back the removed term: dQ gains scale * D_i * sum_j P_ij K_j = scale * D_i * (P K)_i
    Ok, _ = OA.attention(q64, k64, k64, scale, causal, left, right)
    dvec = (do64 * O).sum(axis=-1, keepdims=True)
    return dq + scale * dvec * Ok, dk, dv


def _mut_bwd_no_scale_dk(q, k, v, dout, scale, causal=False, left=-1, right=-1):
    # plausible mistake: dK without the softmax scale
    dq, dk, dv = _ORIG_BWD(q, k, v, dout, scale, causal, left, right)
    return dq, dk / scale, dv


def _mut_ext_softcap_unscaled(q, k, v, scale, causal=False, left=-1, right=-1, softcap=0.0,
                              alibi_slopes=None, bias=None, block_mask=None, block_q=0, block_k=0,
                              rows=None):
    # plausible mistake: softcap applied before the scale (tanh of the raw dot product)
    if softcap > 0:
        softcap = softcap * scale
    return _ORIG_EXT(q, k, v, scale, causal, left, right, softcap, alibi_slopes, bias, block_mask,
                     block_q, block_k, rows)


def _mut_ext_alibi_sign(q, k, v, scale, causal=False, left=-1, right=-1, softcap=0.0,
                        alibi_slopes=None, bias=None, block_mask=None, block_q=0, block_k=0,
                        rows=None):
    # plausible mistake: the ALiBi penalty added instead of subtracted
    if alibi_slopes is not None:
        alibi_slopes = [-x for x in alibi_slopes]
    return _ORIG_EXT(q, k, v, scale, causal, left, right, softcap, alibi_slopes, bias, block_mask,
                     block_q, block_k, rows)


def _mut_ext_block_transposed(q, k, v, scale, causal=False, left=-1, right=-1, softcap=0.0,
                              alibi_slopes=None, bias=None, block_mask=None, block_q=0, block_k=0,
                              rows=None):
    # plausible mistake: block mask indexed (key block, query block) -- for a square mask
    # the transpose, otherwise the two block sizes swapped
    if block_mask is not None:
        if block_mask.shape[-1] == block_mask.shape[-2]:
            block_mask = np.swapaxes(block_mask, -1, -2)
        else:
            block_q, block_k = block_k, block_q
    return _ORIG_EXT(q, k, v, scale, causal, left, right, softcap, alibi_slopes, bias, block_mask,
                     block_q, block_k, rows)


def _mut_decode_multi_top_left(q, k_pages, v_pages, block_table, seq_lens, scale, page_size):
    # plausible mistake: new token n sees only the first n + 1 cached keys (top-left)
    q = np.asarray(q, dtype=np.float64)
    B, Nq, Hq, D = q.shape
    O = np.zeros((B, Nq, Hq, D))
    L = np.full((B, Nq, Hq), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        kb = OA.gather_paged(k_pages, block_table, b, n, page_size).transpose(1, 0, 2)[None]
        vb = OA.gather_paged(v_pages, block_table, b, n, page_size).transpose(1, 0, 2)[None]
        o, lse = _ORIG_ATT(q[b].transpose(1, 0, 2)[None], kb[:, :, :Nq], vb[:, :, :Nq], scale,
                           causal=True)
        O[b] = o[0].transpose(1, 0, 2)
        L[b] = lse[0].T
    return O, L


_ORIG_WIDEN = OA.widen
_ORIG_PROBS = OA.attention_probs


def _mut_widen_bf16_shift(bits, dtype):
    # plausible mistake: the bf16 pattern shifted into the float32 word by the wrong amount
    if dtype == "bf16":
        return (np.asarray(bits).astype(np.uint32) << np.uint32(8)).view(np.float32).astype(np.float64)
    return _ORIG_WIDEN(bits, dtype)


def _mut_widen_swapped(bits, dtype):
    # plausible mistake: the two 16-bit types decoded with each other's layout
    return _ORIG_WIDEN(bits, "bf16" if dtype == "f16" else "f16")


def _mut_probs_gqa_modulo(q, k, scale, causal=False, left=-1, right=-1):
    # plausible mistake: query head h reads KV head h % Hkv
    q, k = np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64)
    Hq, Hkv = q.shape[1], k.shape[1]
    return np.concatenate([_ORIG_PROBS(q[:, h:h + 1], k[:, h % Hkv:h % Hkv + 1], scale, causal,
                                       left, right) for h in range(Hq)], axis=1)

MUTATIONS = {
    "exclusive_window": ("visible", _mut_exclusive_window),
    "top_left_causal": ("visible", _mut_top_left_causal),
    "dropped_scale": ("_rows_attention", _mut_rows_no_scale),
    "lse_missing_max": ("_rows_attention", _mut_rows_lse_no_max),
    "transposed_v": ("_rows_attention", _mut_rows_transposed_v),
    "wrong_sign": ("_rows_attention", _mut_rows_sign),
    "unweighted_merge": ("lse_merge", _mut_merge_unweighted),
    "gqa_modulo": ("attention", _gqa_mod_attention),
    "varlen_no_isolation": ("attention_varlen", _mut_varlen_no_isolation),
    "varlen_top_left": ("attention_varlen", _mut_varlen_top_left),
    "varlen_paged_context_only": ("attention_varlen_paged", _mut_varlen_paged_context_only),
    "decode_multi_top_left": ("decode_paged_multi", _mut_decode_multi_top_left),
    "ext_softcap_unscaled": ("attention_ext", _mut_ext_softcap_unscaled),
    "ext_alibi_sign": ("attention_ext", _mut_ext_alibi_sign),
    "ext_block_transposed": ("attention_ext", _mut_ext_block_transposed),
    "bwd_no_dvec": ("attention_backward", _mut_bwd_no_dvec),
    "bwd_unscaled_dk": ("attention_backward", _mut_bwd_no_scale_dk),
    "widen_bf16_wrong_shift": ("widen", _mut_widen_bf16_shift),
    "widen_types_swapped": ("widen", _mut_widen_swapped),
    "probs_gqa_modulo": ("attention_probs", _mut_probs_gqa_modulo),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(OA, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    assert _caught(monkeypatch, PINS), f"no pin catches the planted mistake {name!r}"
