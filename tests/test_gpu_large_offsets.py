"""Addressing past 2^31 elements: tensors and page pools just over 4 GiB, with seeded
random data only in the heads, sequences or pages that sit on either side of element
2^31 (and at the ends), and zeros everywhere else.

A 32-bit element or byte offset that wrapped would read the zero region instead of the
random one, and the comparison with the oracle would fail.  The zero regions are checked
too, against closed forms: with Q = K = V = 0 every visible score is 0, so O = 0 exactly
and LSE = ln(number of visible keys), which is ln(i + 1) for causal row i (the
identical-keys case); with dO = 0 as well every gradient is exactly 0.

Each test holds up to about 35 GB of device memory and frees it before the next."""
import math

import numpy as np
import pytest

import attn_inputs as A
import oracle
from gpu_util import (assert_close_grads, assert_close_lse, assert_close_o, to_dev, to_f64)

pytestmark = pytest.mark.gpu

ea = pytest.importorskip("exact_attention_amd")

E31 = 2 ** 31


@pytest.fixture(autouse=True)
def _free_device_memory():
    yield
    import gc
    import torch
    gc.collect()
    torch.cuda.empty_cache()


def zeros(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=torch.float16 if dtype == "f16" else torch.bfloat16, device="cuda")


def dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def all_zero_bits(t):
    """True when every element of a 16-bit tensor is +0 (bit pattern 0)."""
    import torch
    return not bool(t.view(torch.int16).any())


def check_causal_zero_lse(L_rows, what):
    """Rows of a zero head / sequence: LSE[i] = ln(i + 1) (causal, Nq = Nk)."""
    import torch
    N = L_rows.shape[-1]
    ref = torch.log(torch.arange(1, N + 1, dtype=torch.float64, device=L_rows.device))
    err = float((L_rows.double() - ref).abs().max())
    print(f"  {what}: max |LSE - ln(i + 1)| = {err:.2e}")
    assert err <= 1e-5, f"{what}: {err:.3e}"


# ---- dense forward and backward: B=1, H=4112, N=4096, D=128 -> 2.156e9 elements ----------
H_BIG, N_BIG, D_BIG = 4112, 4096, 128
HEAD_AT_2_31 = E31 // (N_BIG * D_BIG)       # head 4096 starts exactly at element 2^31


def big_dense(heads, x, dtype, with_grad=None):
    """Q, K, V (and dO) of shape [1, H_BIG, N_BIG, D_BIG]: zeros, with x's heads at `heads`."""
    ts = []
    srcs = (x.q, x.k, x.v) + (() if with_grad is None else (with_grad,))
    for src in srcs:
        t = zeros((1, H_BIG, N_BIG, D_BIG), dtype)
        t[0, heads] = to_dev(src, dtype)[0]
        ts.append(t)
    return ts


def test_forward_past_2_31_elements():
    import torch
    assert H_BIG * N_BIG * D_BIG > E31
    heads = [0, HEAD_AT_2_31 - 1, HEAD_AT_2_31, H_BIG - 1]
    dt = "f16"
    x = A.dense_inputs(1, len(heads), len(heads), N_BIG, N_BIG, D_BIG, dt, 3101)
    q, k, v = big_dense(heads, x, dt)
    scale = 1 / math.sqrt(D_BIG)
    print(f"mfa_fwd q={tuple(q.shape)} f16 causal, random heads {heads}", flush=True)
    O, L = ea.mfa_fwd(q, k, v, scale=scale, causal=True)
    torch.cuda.synchronize()
    qf, kf, vf = (oracle.widen(t, dt) for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention(qf, kf, vf, scale, True)
    for n, h in enumerate(heads):
        assert_close_o(to_f64(O[:, h:h + 1], dt), Or[:, n:n + 1], dt, f"O head {h}")
        assert_close_lse(L[:, h:h + 1].cpu().numpy(), Lr[:, n:n + 1], f"LSE head {h}")
    zero = torch.ones(H_BIG, dtype=torch.bool, device="cuda")
    zero[heads] = False
    check_causal_zero_lse(L[0, zero], "zero heads")
    O[0, heads] = 0
    assert all_zero_bits(O), "a zero head has a nonzero output"


def test_backward_past_2_31_elements():
    import torch
    heads = [HEAD_AT_2_31 - 1, HEAD_AT_2_31, H_BIG - 1]
    dt = "bf16"
    x = A.dense_inputs(1, len(heads), len(heads), N_BIG, N_BIG, D_BIG, dt, 3102)
    dob = A.grad_inputs(1, len(heads), N_BIG, D_BIG, dt, 3103)
    q, k, v, do = big_dense(heads, x, dt, with_grad=dob)
    scale = 1 / math.sqrt(D_BIG)
    print(f"mfa_fwd + mfa_bwd q={tuple(q.shape)} bf16 causal, random heads {heads}", flush=True)
    O, L = ea.mfa_fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv = ea.mfa_bwd(q, k, v, O, do, L, scale=scale, causal=True)
    torch.cuda.synchronize()
    del O, L
    qf, kf, vf, dof = (oracle.widen(t, dt) for t in (x.q, x.k, x.v, dob))
    refs = oracle.attention_backward(qf, kf, vf, dof, scale, True)
    for n, h in enumerate(heads):
        assert_close_grads((f"dQ[{h}]", f"dK[{h}]", f"dV[{h}]"),
                           [to_f64(t[:, h:h + 1], dt) for t in (dq, dk, dv)],
                           [r[:, n:n + 1] for r in refs], dt)
    for name, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
        t[0, heads] = 0
        assert all_zero_bits(t), f"{name}: a zero head has a nonzero gradient"


# ---- packed sequences: 516 x 4096 tokens, Hq = Hkv = 8, D = 128 -> 2.164e9 elements ----
def test_varlen_past_2_31_elements():
    import torch
    H, D, Ls, nseq, dt = 8, 128, 4096, 516, "bf16"
    seq_at_2_31 = E31 // (Ls * H * D)          # sequence 512 starts exactly at element 2^31
    assert nseq * Ls * H * D > E31
    seqs = [0, seq_at_2_31 - 1, seq_at_2_31, nseq - 1]
    x = A.varlen_inputs(H, H, D, dt, 3104, seqlens_q=[Ls] * len(seqs))
    q, k, v = (zeros((nseq * Ls, H, D), dt) for _ in range(3))
    for n, s in enumerate(seqs):
        for big, src in ((q, x.q), (k, x.k), (v, x.v)):
            big[s * Ls:(s + 1) * Ls] = to_dev(src[n * Ls:(n + 1) * Ls], dt)
    cu = dev_i32(np.arange(nseq + 1) * Ls)
    scale = 1 / math.sqrt(D)
    print(f"mfa_fwd_varlen q={tuple(q.shape)} bf16 causal, {nseq} sequences of {Ls}, "
          f"random sequences {seqs}", flush=True)
    O, L = ea.mfa_fwd_varlen(q, k, v, cu, cu, Ls, Ls, scale=scale, causal=True)
    torch.cuda.synchronize()
    # sampled (token, head) rows of the random sequences, in the small packing's numbering
    rng = np.random.default_rng(3104)
    rows = [(n * Ls + i, h) for n in range(len(seqs)) for i in (0, 1, 127, 128, 2048, Ls - 1)
            for h in (0, H - 1)]
    rows += [(int(t), int(h)) for t, h in zip(rng.integers(0, len(seqs) * Ls, 64), rng.integers(0, H, 64))]
    qf, kf, vf = (oracle.widen(t, dt) for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention_varlen(qf, kf, vf, x.cu_seqlens_q, x.cu_seqlens_k, scale, True, rows=rows)
    big_tok = np.array([seqs[t // Ls] * Ls + t % Ls for t, _ in rows])
    hh = np.array([h for _, h in rows])
    Og = to_f64(O[torch.from_numpy(big_tok).cuda(), torch.from_numpy(hh).cuda()], dt)
    assert_close_o(Og, Or, dt, "varlen O")
    assert_close_lse(L.cpu().numpy()[hh, big_tok], Lr, "varlen LSE")
    zero = torch.ones(nseq, dtype=torch.bool, device="cuda")
    zero[seqs] = False
    check_causal_zero_lse(L.view(H, nseq, Ls)[:, zero], "zero sequences")
    for s in seqs:
        O[s * Ls:(s + 1) * Ls] = 0
    assert all_zero_bits(O), "a zero sequence has a nonzero output"


# ---- page pools across element 2^31 (a page of 16 x 8 x 128 is 2^14 elements) ------------
PAGE_AT_2_31 = E31 // (16 * 8 * 128)


def relocated_pool(pages, dtype):
    """A zero pool whose pages [base, base + P) hold `pages`, placed so that they straddle
    element 2^31; returns (pool, base)."""
    P = pages.shape[0]
    base = PAGE_AT_2_31 - P // 2
    pool = zeros((base + P,) + pages.shape[1:], dtype)
    pool[base:] = to_dev(pages, dtype)
    return pool, base


def shifted(block_table, base):
    bt = block_table.copy()
    bt[bt >= 0] += base
    return bt


def test_decode_pool_past_2_31_elements():
    import torch
    dt = "bf16"
    p = A.paged_inputs(6, 32, 8, 128, dt, 3105, len_lo=1, len_hi=5000, extra_pages=3)
    kp, base = relocated_pool(p.k_pages, dt)
    vp, _ = relocated_pool(p.v_pages, dt)
    assert kp.numel() > E31 and base < PAGE_AT_2_31 < base + p.k_pages.shape[0]
    scale = 1 / math.sqrt(128)
    print(f"mfa_decode_paged pool={tuple(kp.shape)} pages from {base}, seq_lens={p.seq_lens.tolist()}",
          flush=True)
    O, L = ea.mfa_decode_paged(to_dev(p.q, dt), kp, vp, dev_i32(shifted(p.block_table, base)),
                               dev_i32(p.seq_lens), scale=scale)
    torch.cuda.synchronize()
    Or, Lr = oracle.decode_paged(oracle.widen(p.q, dt), oracle.widen(p.k_pages, dt),
                                 oracle.widen(p.v_pages, dt), p.block_table, p.seq_lens, scale, 16)
    assert_close_o(to_f64(O, dt), Or, dt, "decode O")
    assert_close_lse(L.cpu().numpy(), Lr, "decode LSE")


def test_multi_decode_pool_past_2_31_elements():
    import torch
    dt = "bf16"
    p = A.paged_multi_inputs(5, 4, 32, 8, 128, dt, 3106, len_lo=4, len_hi=4000, extra_pages=2)
    kp, base = relocated_pool(p.k_pages, dt)
    vp, _ = relocated_pool(p.v_pages, dt)
    scale = 1 / math.sqrt(128)
    print(f"mfa_decode_paged_multi pool={tuple(kp.shape)} pages from {base}, "
          f"seq_lens={p.seq_lens.tolist()}", flush=True)
    O, L = ea.mfa_decode_paged_multi(to_dev(p.q, dt), kp, vp, dev_i32(shifted(p.block_table, base)),
                                     dev_i32(p.seq_lens), scale=scale)
    torch.cuda.synchronize()
    Or, Lr = oracle.decode_paged_multi(oracle.widen(p.q, dt), oracle.widen(p.k_pages, dt),
                                       oracle.widen(p.v_pages, dt), p.block_table, p.seq_lens, scale, 16)
    assert_close_o(to_f64(O, dt), Or, dt, "4-token decode O")
    assert_close_lse(L.cpu().numpy(), Lr, "4-token decode LSE")


def test_paged_prefill_pool_past_2_31_elements():
    import torch
    dt = "bf16"
    p = A.paged_varlen_inputs(32, 8, 128, dt, 3107, seqlens_q=[300, 1, 700], ctx_lens=[2000, 4000, 900])
    kp, base = relocated_pool(p.k_pages, dt)
    vp, _ = relocated_pool(p.v_pages, dt)
    lq = np.diff(p.cu_seqlens_q)
    scale = 1 / math.sqrt(128)
    print(f"mfa_fwd_varlen_paged pool={tuple(kp.shape)} pages from {base}, lq={lq.tolist()} "
          f"lk={p.seq_lens_k.tolist()}", flush=True)
    O, L = ea.mfa_fwd_varlen_paged(to_dev(p.q, dt), kp, vp, dev_i32(shifted(p.block_table, base)),
                                   dev_i32(p.seq_lens_k), dev_i32(p.cu_seqlens_q), int(lq.max()),
                                   int(p.seq_lens_k.max()), scale=scale, causal=True)
    torch.cuda.synchronize()
    qf, kf, vf = (oracle.widen(t, dt) for t in (p.q, p.k_pages, p.v_pages))
    Or, Lr = oracle.attention_varlen_paged(qf, kf, vf, p.block_table, p.seq_lens_k, p.cu_seqlens_q,
                                           scale, 16, True)
    assert_close_o(to_f64(O, dt), Or, dt, "paged prefill O")
    assert_close_lse(L.cpu().numpy(), Lr, "paged prefill LSE")


# ---- one very long context: 262144 cached tokens, 512 splits -----------------------------
def test_decode_long_context():
    import torch
    dt = "bf16"
    p = A.paged_inputs(2, 32, 8, 128, dt, 3108, len_lo=1, len_hi=262144, seq_lens=[262144, 37],
                       extra_pages=1)
    scale = 1 / math.sqrt(128)
    print(f"mfa_decode_paged pool={p.k_pages.shape} seq_lens={p.seq_lens.tolist()}", flush=True)
    O, L = ea.mfa_decode_paged(to_dev(p.q, dt), to_dev(p.k_pages, dt), to_dev(p.v_pages, dt),
                               dev_i32(p.block_table), dev_i32(p.seq_lens), scale=scale)
    torch.cuda.synchronize()
    info = ea.mfa_last_dispatch()
    print(f"  splits={info['num_splits']} chunk={info['chunk_tokens']}")
    assert info["num_splits"] * info["chunk_tokens"] >= 262144
    Or, Lr = oracle.decode_paged(oracle.widen(p.q, dt), oracle.widen(p.k_pages, dt),
                                 oracle.widen(p.v_pages, dt), p.block_table, p.seq_lens, scale, 16)
    assert_close_o(to_f64(O, dt), Or, dt, "long-context decode O")
    assert_close_lse(L.cpu().numpy(), Lr, "long-context decode LSE")
