"""The no-allocation decode entry point (mfa_decode_paged_noalloc) against mfa_decode_paged.

Both run the same split and combine kernels with the same split count; one keeps the split
partials in a caller workspace, the other in the library's fixed per-GPU scratch.  Two
calls in a row through the C ABI, the second on a smaller input (the scratch then holds the
first call's partials), must each give the workspace entry point's result bit for bit, and
both must match the oracle.  A request whose partials exceed the scratch is rejected.
"""
import math

import numpy as np
import pytest

import attn_inputs as A
import oracle
from gpu_util import assert_close_lse, assert_close_o, to_bits, to_dev, to_f64

pytestmark = pytest.mark.gpu

ea = pytest.importorskip("exact_attention_amd")


def _inputs(p):
    import torch
    return (to_dev(p.q, p.dtype), to_dev(p.k_pages, p.dtype), to_dev(p.v_pages, p.dtype),
            torch.from_numpy(p.block_table).to("cuda"), torch.from_numpy(p.seq_lens).to("cuda"))


def _call_noalloc(q, kp, vp, bt, sl, out, lse, scale, num_splits=0):
    """mfa_decode_paged_noalloc through the C ABI (raw pointers, the current stream)."""
    import torch
    B, Hq, D = q.shape
    P, page, Hkv, _ = kp.shape
    dt = ea.MFA_F16 if q.dtype == torch.float16 else ea.MFA_BF16
    return ea.lib().mfa_decode_paged_noalloc(
        q.data_ptr(), kp.data_ptr(), vp.data_ptr(), bt.data_ptr(), sl.data_ptr(), out.data_ptr(),
        lse.data_ptr(), B, Hq, Hkv, D, page, P, bt.shape[1], float(scale), int(num_splits), dt,
        torch.cuda.current_stream().cuda_stream)


CASES = [
    # the paged decode workload, then a smaller problem (D = 64, f16, short sequences)
    ("paged_splitkv_decode", None),
    ("small", dict(B=3, Hq=8, Hkv=2, D=64, dtype="f16", seed=901, len_lo=1, len_hi=700)),
]


def test_noalloc_two_calls_match_workspace_entry_point():
    import torch
    for name, kw in CASES:
        if kw is None:
            c = A.workload(name)
            p = A.workload_inputs(name)
            scale = c["scale"]
        else:
            p = A.paged_inputs(kw["B"], kw["Hq"], kw["Hkv"], kw["D"], kw["dtype"], kw["seed"],
                               len_lo=kw["len_lo"], len_hi=kw["len_hi"], extra_pages=2)
            scale = 1 / math.sqrt(kw["D"])
        q, kp, vp, bt, sl = _inputs(p)
        print(f"decode noalloc vs workspace: {name} q={tuple(q.shape)} pool={tuple(kp.shape)}",
              flush=True)
        Ow, Lw = ea.mfa_decode_paged(q, kp, vp, bt, sl, scale=scale)
        On = torch.empty_like(q)
        Ln = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
        st = _call_noalloc(q, kp, vp, bt, sl, On, Ln, scale)
        torch.cuda.synchronize()
        assert st == 0, ea.mfa_status_string(st)
        info = ea.mfa_last_dispatch()
        assert info["op"] == 2 and info["kernel"].startswith("mfa_decode_split_kernel"), info
        assert np.array_equal(to_bits(On), to_bits(Ow)), f"{name}: O differs from mfa_decode_paged"
        assert torch.equal(Ln, Lw), f"{name}: LSE differs from mfa_decode_paged"
        Or, Lr = oracle.decode_paged(oracle.widen(p.q, p.dtype), oracle.widen(p.k_pages, p.dtype),
                                     oracle.widen(p.v_pages, p.dtype), p.block_table, p.seq_lens,
                                     scale, p.page_size)
        assert_close_o(to_f64(On, p.dtype), Or, p.dtype, f"{name} O")
        assert_close_lse(Ln.cpu().numpy(), Lr, f"{name} LSE")


def test_noalloc_rejects_partials_beyond_the_scratch():
    # 64 sequences x 64 heads x 64 splits x 129 floats = 135 MB > 32 MiB: MFA_ERR_WORKSPACE,
    # with nothing launched (the outputs keep their contents)
    import torch
    B, Hq, Hkv, D = 64, 64, 8, 128
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros(4, 16, Hkv, D, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(B, 2048, dtype=torch.int32, device="cuda")
    sl = torch.ones(B, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 5.0)
    lse = torch.full((B, Hq), 7.0, dtype=torch.float32, device="cuda")
    assert ea.mfa_decode_workspace_bytes(B, Hq, D, 16, 2048, 0) > 32 << 20
    st = _call_noalloc(q, kp, kp, bt, sl, out, lse, 0.1)
    torch.cuda.synchronize()
    assert st == -8, ea.mfa_status_string(st)
    assert bool((out == 5.0).all()) and bool((lse == 7.0).all())
