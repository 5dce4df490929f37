"""GPU parity of the backward pass (mfa_bwd through the C ABI) against the oracle's
attention_backward.

Tolerance (the pages state none for gradients; derived from the arithmetic): P and dS are
rounded to the input type before each product (relative error u = 2^-9 for bf16, 2^-12
for f16), accumulation is fp32 and each gradient is rounded once more, so an element's
error is a few u times the magnitude of the terms it sums.  The test bounds
max |dX_gpu - dX_oracle| <= 8 u max |dX_oracle| for each of dQ, dK, dV."""
import math

import numpy as np
import pytest

import attn_inputs as A
import oracle
from gpu_util import assert_close_grads as check
from gpu_util import to_dev, to_f64

pytestmark = pytest.mark.gpu

ea = pytest.importorskip("exact_attention_amd")


def grads_case(B, Hq, Hkv, Nq, Nk, D, dtype, seed, causal=False, left=-1, right=-1, scale=None):
    import torch
    x = A.dense_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, seed)
    rng = np.random.default_rng(seed + 1)
    dout_bits = A.round_f32_to_bits(rng.standard_normal((B, Hq, Nq, D), dtype=np.float32), dtype)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
    do = to_dev(dout_bits, dtype)
    print(f"mfa_fwd + mfa_bwd q={tuple(q.shape)} k={tuple(k.shape)} {dtype} causal={causal} "
          f"win=({left},{right}) scale={scale:.4f}", flush=True)
    O, L = ea.mfa_fwd(q, k, v, scale=scale, causal=causal, win_left=left, win_right=right)
    dq, dk, dv = ea.mfa_bwd(q, k, v, O, do, L, scale=scale, causal=causal, win_left=left,
                            win_right=right)
    torch.cuda.synchronize()
    info = ea.mfa_last_dispatch()
    assert info["op"] == 7 and info["n_launches"] == 2
    return x, dout_bits, scale, (dq, dk, dv)


def full_check(B, Hq, Hkv, Nq, Nk, D, dtype, seed, causal=False, left=-1, right=-1, scale=None):
    x, dob, scale, (dq, dk, dv) = grads_case(B, Hq, Hkv, Nq, Nk, D, dtype, seed, causal, left, right,
                                             scale)
    qf, kf, vf, dof = (oracle.widen(t, dtype) for t in (x.q, x.k, x.v, dob))
    refs = oracle.attention_backward(qf, kf, vf, dof, scale, causal, left, right)
    check(("dQ", "dK", "dV"), [to_f64(t, dtype) for t in (dq, dk, dv)], refs, dtype)


CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, left, right
    (1, 2, 2, 128, 128, 64, "f16", False, -1, -1),
    (1, 4, 2, 257, 257, 128, "bf16", True, -1, -1),
    (2, 2, 1, 200, 333, 128, "f16", True, -1, -1),      # Nq < Nk, bottom-right
    (1, 2, 2, 300, 90, 64, "bf16", True, -1, -1),       # Nq > Nk: rows with no key
    (1, 2, 2, 500, 500, 128, "f16", True, 37, 0),       # window
    (1, 2, 2, 400, 400, 64, "bf16", False, 20, 45),     # two-sided window
    (1, 8, 2, 256, 256, 128, "bf16", True, -1, -1),     # GQA, g = 4
    (1, 3, 3, 33, 1, 128, "f16", False, -1, -1),        # one key
    (1, 2, 2, 1, 700, 128, "bf16", True, -1, -1),       # one query row
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_backward_vs_oracle(case):
    B, Hq, Hkv, Nq, Nk, D, dt, causal, left, right = case
    full_check(B, Hq, Hkv, Nq, Nk, D, dt, 900 + Nq + Nk, causal, left, right)


def test_negative_scale():
    full_check(1, 2, 2, 160, 160, 128, "f16", 5, True, scale=-0.09)


def test_deterministic():
    import torch
    _, _, _, g0 = grads_case(1, 8, 2, 384, 384, 128, "bf16", 3, True)
    _, _, _, g1 = grads_case(1, 8, 2, 384, 384, 128, "bf16", 3, True)
    for a, b in zip(g0, g1):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_masked_keys_get_zero_gradients():
    # window (0, 0) with Nq < Nk: keys 0 .. off - 1 are seen by no row
    import torch
    _, _, _, (dq, dk, dv) = grads_case(1, 2, 2, 100, 164, 64, "f16", 8, True, 0, 0)
    assert torch.all(dk[:, :, :64] == 0) and torch.all(dv[:, :, :64] == 0)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dense_causal_prefill_shape_two_heads(dtype):
    # the dense causal prefill shape (B=2, H=8, N=4096, D=128); the oracle recomputes two
    # (batch, head) pairs in full: each head's gradients depend on that head alone
    x, dob, scale, (dq, dk, dv) = grads_case(2, 8, 8, 4096, 4096, 128, dtype, 12, True)
    for b, h in ((0, 0), (1, 7)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        qf, kf, vf, dof = (oracle.widen(t[sl], dtype) for t in (x.q, x.k, x.v, dob))
        refs = oracle.attention_backward(qf, kf, vf, dof, scale, True)
        check((f"dQ[{b},{h}]", f"dK[{b},{h}]", f"dV[{b},{h}]"),
              [to_f64(t[sl], dtype) for t in (dq, dk, dv)], refs, dtype)


def test_gqa_long_sequence_one_kv_group():
    # GQA at a long sequence (B=1, Hq=8, Hkv=2, N=8192, bf16, causal): the oracle recomputes
    # KV head 0's whole group of 4 query heads (its dK, dV sum over all four), which checks
    # the group accumulation over the long descending walk of the dK/dV pass
    x, dob, scale, (dq, dk, dv) = grads_case(1, 8, 2, 8192, 8192, 128, "bf16", 21, True)
    sq, skv = (slice(0, 1), slice(0, 4)), (slice(0, 1), slice(0, 1))
    qf, dof = (oracle.widen(t[sq], "bf16") for t in (x.q, dob))
    kf, vf = (oracle.widen(t[skv], "bf16") for t in (x.k, x.v))
    refs = oracle.attention_backward(qf, kf, vf, dof, scale, True)
    check(("dQ[heads 0-3]", "dK[kv 0]", "dV[kv 0]"),
          [to_f64(dq[sq], "bf16"), to_f64(dk[skv], "bf16"), to_f64(dv[skv], "bf16")], refs, "bf16")
