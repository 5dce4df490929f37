"""GPU parity of the multi-token paged decode (mfa_decode_paged_multi through the C ABI)
against the oracle's decode_paged_multi."""
import math

import numpy as np
import pytest

import attn_inputs as A
import oracle
from gpu_util import assert_close_lse, assert_close_o, to_bits, to_dev, to_f64

pytestmark = pytest.mark.gpu

ea = pytest.importorskip("exact_attention_amd")


class Dev:
    def __init__(self, p):
        import torch
        self.p = p
        self.q = to_dev(p.q, p.dtype)
        self.kp = to_dev(p.k_pages, p.dtype)
        self.vp = to_dev(p.v_pages, p.dtype)
        self.bt = torch.from_numpy(p.block_table).to("cuda")
        self.sl = torch.from_numpy(p.seq_lens).to("cuda")


def run(d, scale, num_splits=0, bt=None, kp=None, vp=None):
    import torch
    print(f"mfa_decode_paged_multi q={tuple(d.q.shape)} pool={tuple(d.kp.shape)} "
          f"lens={d.p.seq_lens.tolist()[:8]} splits={num_splits}", flush=True)
    O, L = ea.mfa_decode_paged_multi(d.q, d.kp if kp is None else kp, d.vp if vp is None else vp,
                                     d.bt if bt is None else bt, d.sl, scale=scale,
                                     num_splits=num_splits)
    torch.cuda.synchronize()
    return O, L


def ref(p, scale):
    return oracle.decode_paged_multi(oracle.widen(p.q, p.dtype), oracle.widen(p.k_pages, p.dtype),
                                     oracle.widen(p.v_pages, p.dtype), p.block_table, p.seq_lens,
                                     scale, p.page_size)


CASES = [
    # B, Nq, Hq, Hkv, D, dtype, len_lo, len_hi, seq_lens
    (3, 4, 8, 2, 128, "bf16", 1, 300, None),
    (4, 4, 32, 8, 128, "bf16", 1000, 3000, None),
    (3, 2, 4, 4, 64, "f16", 1, 100, None),          # g = 1
    (5, 3, 16, 2, 128, "f16", 1, 2000, [1, 15, 16, 17, 2000]),   # L < Nq: masked rows
    (2, 4, 6, 2, 64, "bf16", 50, 600, None),        # g = 3: one head per workgroup
    (3, 2, 16, 2, 128, "bf16", 100, 900, None),     # g = 8, Nq = 2: four heads per workgroup
    (2, 1, 8, 2, 128, "f16", 100, 700, None),       # one token
    (1, 4, 2, 1, 128, "f16", 4096, 4096, None),     # g = 2
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_multi_decode_vs_oracle(case):
    B, Nq, Hq, Hkv, D, dt, lo, hi, sl = case
    p = A.paged_multi_inputs(B, Nq, Hq, Hkv, D, dt, 700 + B + Hq + Nq, len_lo=lo, len_hi=hi,
                             extra_pages=3, seq_lens=sl)
    scale = 1 / math.sqrt(D)
    d = Dev(p)
    O, L = run(d, scale)
    Or, Lr = ref(p, scale)
    eo = assert_close_o(to_f64(O, dt), Or, dt, f"multi decode O {case}")
    el = assert_close_lse(L.cpu().numpy(), Lr, f"multi decode LSE {case}")
    info = ea.mfa_last_dispatch()
    assert info["op"] == 5 and info["kernel"].startswith("mfa_decode_mq_split_kernel")
    print(f"multi {case}: max|dO|={eo:.2e} max|dLSE|={el:.2e} {info['kernel']}")


@pytest.mark.parametrize("B", [256, 257])
def test_both_grids(B):
    # the flattened grid of non-empty chunks (B <= 256) and the (chunk, head group, sequence)
    # grid, with sequences shorter than the new tokens among them
    lens = np.random.default_rng(B).integers(0, 300, size=B)
    lens[:3] = [0, 2, 17]
    p = A.paged_multi_inputs(B, 3, 4, 2, 64, "f16", 80 + B, len_lo=0, len_hi=300, seq_lens=lens,
                             extra_pages=1)
    O, L = run(Dev(p), 0.12)
    info = ea.mfa_last_dispatch()
    assert (",flat" in info["kernel"]) == (B <= 256), info["kernel"]
    Or, Lr = ref(p, 0.12)
    assert_close_o(to_f64(O, "f16"), Or, "f16", f"multi decode O B={B}")
    assert_close_lse(L.cpu().numpy(), Lr, f"multi decode LSE B={B}")


def test_fully_masked_rows():
    # with 2 cached tokens and 4 new ones, tokens 0 and 1 see nothing: O = 0, LSE = -inf
    import torch
    p = A.paged_multi_inputs(2, 4, 8, 2, 128, "bf16", 5, len_lo=1, len_hi=40, seq_lens=[2, 40])
    O, L = run(Dev(p), 0.1)
    assert torch.all(O[0, :2] == 0) and torch.all(torch.isneginf(L[0, :2]))
    Or, Lr = ref(p, 0.1)
    assert_close_o(to_f64(O, "bf16"), Or, "bf16")
    assert_close_lse(L.cpu().numpy(), Lr)


@pytest.mark.parametrize("num_splits", [1, 3, 64])
def test_split_counts(num_splits):
    p = A.paged_multi_inputs(3, 4, 16, 4, 128, "f16", 11, len_lo=200, len_hi=3000)
    O, L = run(Dev(p), 0.08, num_splits=num_splits)
    Or, Lr = ref(p, 0.08)
    assert_close_o(to_f64(O, "f16"), Or, "f16", f"splits={num_splits}")
    assert_close_lse(L.cpu().numpy(), Lr, f"splits={num_splits}")


def test_page_placement_bitwise():
    import torch
    p = A.paged_multi_inputs(3, 4, 8, 2, 128, "bf16", 13, len_lo=30, len_hi=700, extra_pages=4)
    d = Dev(p)
    O0, L0 = run(d, 0.1)
    perm = np.random.default_rng(2).permutation(p.k_pages.shape[0])
    inv = np.argsort(perm)
    bt2 = np.where(p.block_table >= 0, inv[np.maximum(p.block_table, 0)], -1).astype(np.int32)
    O1, L1 = run(d, 0.1, bt=torch.from_numpy(bt2).cuda(), kp=to_dev(p.k_pages[perm], "bf16"),
                 vp=to_dev(p.v_pages[perm], "bf16"))
    assert np.array_equal(to_bits(O0), to_bits(O1)) and torch.equal(L0, L1)


def test_one_token_matches_single_query_kernel():
    import torch
    p = A.paged_multi_inputs(4, 1, 32, 8, 128, "bf16", 17, len_lo=100, len_hi=5000)
    d = Dev(p)
    O, L = run(d, 0.088)
    Os, Ls = ea.mfa_decode_paged(d.q[:, 0].contiguous(), d.kp, d.vp, d.bt, d.sl, scale=0.088)
    torch.cuda.synchronize()
    assert_close_o(to_f64(O[:, 0], "bf16"), to_f64(Os, "bf16"), "bf16", "vs single-query kernel")
    assert_close_lse(L[:, 0].cpu().numpy(), Ls.cpu().numpy().astype(np.float64))


def test_deterministic():
    import torch
    p = A.paged_multi_inputs(4, 4, 32, 8, 128, "bf16", 19, len_lo=500, len_hi=4000)
    d = Dev(p)
    O0, L0 = run(d, 0.09)
    O1, L1 = run(d, 0.09)
    assert torch.equal(O0.view(torch.int16), O1.view(torch.int16)) and torch.equal(L0, L1)


def test_full_size_verification_workload():
    # 4 new tokens per sequence over the decode workload's cache shape, every row checked
    import torch
    c = A.workload("paged_multi_query_decode")
    p = A.workload_inputs("paged_multi_query_decode")
    O, L = run(Dev(p), c["scale"])
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(L).all())
    Or, Lr = ref(p, c["scale"])
    eo = assert_close_o(to_f64(O, c["dtype"]), Or, c["dtype"], "verification workload")
    el = assert_close_lse(L.cpu().numpy(), Lr, "verification workload")
    print(f"verification workload: max|dO|={eo:.2e} max|dLSE|={el:.2e} "
          f"{ea.mfa_last_dispatch()['kernel']}")
