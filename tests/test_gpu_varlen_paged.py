"""GPU parity of packed queries over a paged KV cache (mfa_fwd_varlen_paged through the
C ABI) against the oracle's attention_varlen_paged."""
import math

import numpy as np
import pytest

import attn_inputs as A
import oracle
from gpu_util import assert_close_lse, assert_close_o, to_bits, to_dev, to_f64

pytestmark = pytest.mark.gpu

ea = pytest.importorskip("exact_attention_amd")


def dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def run(p, scale, causal=True, left=-1, right=-1, block_table=None, k_pages=None, v_pages=None):
    import torch
    lq = np.diff(p.cu_seqlens_q)
    q = to_dev(p.q, p.dtype)
    kp = to_dev(p.k_pages if k_pages is None else k_pages, p.dtype)
    vp = to_dev(p.v_pages if v_pages is None else v_pages, p.dtype)
    bt = dev_i32(p.block_table if block_table is None else block_table)
    print(f"mfa_fwd_varlen_paged q={tuple(q.shape)} pool={tuple(kp.shape)} {p.dtype} "
          f"lq={lq.tolist()[:8]} lk={p.seq_lens_k.tolist()[:8]} causal={causal} "
          f"win=({left},{right})", flush=True)
    O, L = ea.mfa_fwd_varlen_paged(q, kp, vp, bt, dev_i32(p.seq_lens_k), dev_i32(p.cu_seqlens_q),
                                   int(max(1, lq.max())), int(max(1, p.seq_lens_k.max())),
                                   scale=scale, causal=causal,
                                   win_left=left, win_right=right)
    torch.cuda.synchronize()
    return O, L


def oracle_of(p, scale, causal=True, left=-1, right=-1, rows=None):
    qf, kf, vf = (oracle.widen(t, p.dtype) for t in (p.q, p.k_pages, p.v_pages))
    return oracle.attention_varlen_paged(qf, kf, vf, p.block_table, p.seq_lens_k, p.cu_seqlens_q,
                                         scale, p.page_size, causal, left, right, rows=rows)


def contiguous_tokens(p):
    """The cached tokens of every sequence, laid out back to back (host-side copy)."""
    ks, vs = [], []
    for b, L in enumerate(p.seq_lens_k):
        n = -(-int(L) // p.page_size)
        pages = p.block_table[b, :n]
        ks.append(p.k_pages[pages].reshape(-1, *p.k_pages.shape[2:])[:int(L)])
        vs.append(p.v_pages[pages].reshape(-1, *p.v_pages.shape[2:])[:int(L)])
    return np.concatenate(ks), np.concatenate(vs)


CASES = [
    # Hq, Hkv, D, dtype, new lengths, context lengths, causal, left, right
    (4, 2, 128, "bf16", [100, 1, 300, 64], [400, 77, 0, 1000], True, -1, -1),
    (8, 8, 128, "f16", [1, 1, 1, 1, 1], [15, 16, 17, 1000, 0], True, -1, -1),   # one-token chunks
    (2, 1, 64, "f16", [129, 250, 7], [3, 640, 33], True, -1, -1),
    (4, 4, 128, "f16", [200, 333], [500, 64], True, 100, 0),                    # window
    (2, 2, 64, "bf16", [90, 257], [10, 300], False, -1, -1),                    # non-causal
    (6, 2, 128, "bf16", [640], [0], True, -1, -1),                              # no context
    # many tiles: one 4-wave group per workgroup
    (64, 16, 128, "bf16", [300, 5, 700, 129], [700, 90, 0, 1500], True, -1, -1),
    (96, 48, 64, "f16", [129, 250, 7, 400], [3, 640, 33, 900], True, 200, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_paged_packs_match_oracle(case):
    Hq, Hkv, D, dtype, lq, ctx, causal, left, right = case
    p = A.paged_varlen_inputs(Hq, Hkv, D, dtype, 300 + sum(lq), seqlens_q=lq, ctx_lens=ctx,
                              extra_pages=3)
    O, L = run(p, 1 / math.sqrt(D), causal, left, right)
    Or, Lr = oracle_of(p, 1 / math.sqrt(D), causal, left, right)
    eo = assert_close_o(to_f64(O, dtype), Or, dtype, str(case))
    el = assert_close_lse(L.cpu().numpy(), Lr, str(case))
    info = ea.mfa_last_dispatch()
    assert info["op"] == 4 and ",varlen,paged" in info["kernel"]
    # (at most 64 sequences and Hkv a multiple of 8: sequence-major order)
    assert (",seq-major" in info["kernel"]) == (Hkv % 8 == 0 and len(lq) <= 64), info["kernel"]
    print(f"paged {case}: max|dO|={eo:.2e} max|dLSE|={el:.2e} {info['kernel']}")


@pytest.mark.parametrize("Hq,Hkv,layout", [(8, 2, "groups=2"), (96, 8, "groups=1")])
def test_paged_equals_contiguous_packed_bitwise(Hq, Hkv, layout):
    # the same tokens through pages or packed back to back: same tiles, same order, same
    # values (zeros past each sequence's end), hence bit-identical results (in both the
    # key-splitting and the one-group layout)
    import torch
    p = A.paged_varlen_inputs(Hq, Hkv, 128, "bf16", 17, seqlens_q=[300, 5, 129], ctx_lens=[700, 90, 0])
    O, L = run(p, 0.09)
    assert layout in ea.mfa_last_dispatch()["kernel"], ea.mfa_last_dispatch()["kernel"]
    k, v = contiguous_tokens(p)
    lk = p.seq_lens_k
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    Oc, Lc = ea.mfa_fwd_varlen(to_dev(p.q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                               dev_i32(p.cu_seqlens_q), dev_i32(cu_k), 300, int(lk.max()),
                               scale=0.09, causal=True)
    torch.cuda.synchronize()
    assert layout in ea.mfa_last_dispatch()["kernel"], ea.mfa_last_dispatch()["kernel"]
    assert np.array_equal(to_bits(O), to_bits(Oc))
    assert torch.equal(L, Lc)


def test_page_placement_bitwise():
    import torch
    p = A.paged_varlen_inputs(4, 1, 128, "f16", 23, seqlens_q=[64, 200], ctx_lens=[333, 17],
                              extra_pages=5)
    O0, L0 = run(p, 0.1)
    perm = np.random.default_rng(1).permutation(p.k_pages.shape[0])
    inv = np.argsort(perm)
    bt2 = np.where(p.block_table >= 0, inv[np.maximum(p.block_table, 0)], -1).astype(np.int32)
    O1, L1 = run(p, 0.1, block_table=bt2, k_pages=p.k_pages[perm], v_pages=p.v_pages[perm])
    assert np.array_equal(to_bits(O0), to_bits(O1))
    assert torch.equal(L0, L1)


def test_one_token_chunks_match_decode():
    # a chunk of one token is a decode step; the two kernels agree within the tolerance
    import torch
    p = A.paged_varlen_inputs(32, 8, 128, "bf16", 29, seqlens_q=[1] * 6,
                              ctx_lens=[0, 15, 16, 1000, 4095, 77])
    O, L = run(p, 1 / math.sqrt(128))
    q = to_dev(p.q, "bf16")
    Od, Ld = ea.mfa_decode_paged(q, to_dev(p.k_pages, "bf16"), to_dev(p.v_pages, "bf16"),
                                 dev_i32(p.block_table), dev_i32(p.seq_lens_k),
                                 scale=1 / math.sqrt(128))
    torch.cuda.synchronize()
    assert_close_o(to_f64(O, "bf16"), to_f64(Od, "bf16"), "bf16", "vs decode")
    assert_close_lse(L.t().cpu().numpy(), Ld.cpu().numpy().astype(np.float64), "vs decode")


def test_full_size_chunked_prefill_sampled():
    import torch
    c = A.workload("paged_chunked_prefill")
    p = A.workload_inputs("paged_chunked_prefill")
    O, L = run(p, c["scale"], c["causal"])
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(L).all())
    cu = p.cu_seqlens_q
    rows = set()
    for b in range(c["B"]):
        for t in (int(cu[b]), int(cu[b + 1]) - 1, (int(cu[b]) + int(cu[b + 1])) // 2):
            rows.add((t, 0))
            rows.add((t, c["Hq"] - 1))
    rng = np.random.default_rng(7)
    while len(rows) < 120:
        rows.add((int(rng.integers(int(cu[-1]))), int(rng.integers(c["Hq"]))))
    rows = sorted(rows)
    Or, Lr = oracle_of(p, c["scale"], c["causal"], rows=rows)
    t_idx, h_idx = (np.array(r) for r in zip(*rows))
    eo = assert_close_o(to_f64(O, c["dtype"])[t_idx, h_idx], Or, c["dtype"], "chunked prefill")
    el = assert_close_lse(L.cpu().numpy()[h_idx, t_idx], Lr, "chunked prefill")
    print(f"chunked prefill: max|dO|={eo:.2e} max|dLSE|={el:.2e} {ea.mfa_last_dispatch()['kernel']}")
