"""GPU parity of the forward kernel (mfa_fwd through the C ABI) against the oracle."""
import math

import numpy as np
import pytest

import attn_inputs as A
import oracle
from gpu_util import assert_close_lse, assert_close_o, to_dev, to_f64, torch_dtype

pytestmark = pytest.mark.gpu

ea = pytest.importorskip("exact_attention_amd")


def run(q, k, v, scale, causal=False, left=-1, right=-1):
    print(f"mfa_fwd q={tuple(q.shape)} k={tuple(k.shape)} {q.dtype} causal={causal} "
          f"win=({left},{right})", flush=True)
    O, L = ea.mfa_fwd(q, k, v, scale=scale, causal=causal, win_left=left, win_right=right)
    import torch
    torch.cuda.synchronize()
    return O, L


def dense_case(B, Hq, Hkv, Nq, Nk, D, dtype, seed, causal, left=-1, right=-1, scale=None):
    x = A.dense_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, seed)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
    O, L = run(q, k, v, scale, causal, left, right)
    qf, kf, vf = (oracle.widen(t, dtype) for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention(qf, kf, vf, scale, causal, left, right)
    eo = assert_close_o(to_f64(O, dtype), Or, dtype, "O")
    el = assert_close_lse(L.cpu().numpy(), Lr, "LSE")
    info = ea.mfa_last_dispatch()
    assert info["op"] == 1 and info["kernel"].startswith("mfa_fwd_kernel<D=%d" % D)
    return eo, el


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_workload(causal):
    c = A.workload("tiny_dense")
    eo, el = dense_case(c["B"], c["Hq"], c["Hkv"], c["Nq"], c["Nk"], c["D"], c["dtype"], c["seed"],
                        causal)
    print(f"tiny workload causal={causal}: max|dO|={eo:.2e} max|dLSE|={el:.2e}")


EDGE = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, left, right
    (1, 2, 2, 200, 333, 128, "f16", False, -1, -1),
    (1, 2, 2, 333, 333, 128, "f16", True, -1, -1),
    (2, 4, 1, 259, 259, 64, "bf16", True, -1, -1),
    (1, 8, 2, 130, 517, 128, "bf16", True, -1, -1),     # Nq < Nk: bottom-right causal
    (1, 2, 2, 300, 90, 128, "f16", True, -1, -1),       # Nq > Nk: fully masked rows
    (1, 2, 1, 1, 1, 128, "f16", False, -1, -1),
    (1, 2, 2, 1, 777, 64, "f16", True, -1, -1),         # one query row
    (1, 3, 3, 64, 1, 64, "bf16", False, -1, -1),        # one key
    (1, 2, 2, 500, 500, 128, "f16", True, 37, 0),       # window
    (1, 2, 2, 500, 500, 64, "bf16", False, 20, 45),     # two-sided window
    (1, 2, 2, 400, 400, 128, "f16", False, 0, 0),       # diagonal only
    (1, 4, 4, 260, 260, 128, "bf16", False, -1, 3),     # right-only window
    (2, 4, 2, 384, 384, 128, "f16", False, -1, -1),     # exact multiples of the tiles
]


@pytest.mark.parametrize("case", EDGE, ids=[str(i) for i in range(len(EDGE))])
def test_edge_shapes(case):
    B, Hq, Hkv, Nq, Nk, D, dtype, causal, left, right = case
    dense_case(B, Hq, Hkv, Nq, Nk, D, dtype, 1000 + Nq + Nk, causal, left, right)


@pytest.mark.parametrize("case", [
    (500, 128, "f16", True, 37, 0),      # row windows starting in the upper lane half of a block
    (500, 64, "bf16", False, 20, 45),
    (333, 128, "bf16", True, -1, -1),
])
def test_both_workgroup_layouts(case):
    # a small grid takes two key-splitting wave groups per workgroup, a large one a single
    # group; both must agree with the oracle (first and last head checked)
    N, D, dtype, causal, left, right = case
    for H, groups in ((2, 2), (240, 1)):
        x = A.dense_inputs(1, H, H, N, N, D, dtype, 31 + H)
        q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
        O, L = run(q, k, v, 1 / math.sqrt(D), causal, left, right)
        info = ea.mfa_last_dispatch()
        assert f"groups={groups}" in info["kernel"], info["kernel"]
        for h in (0, H - 1):
            qf, kf, vf = (oracle.widen(t[:, h:h + 1], dtype) for t in (x.q, x.k, x.v))
            Or, Lr = oracle.attention(qf, kf, vf, 1 / math.sqrt(D), causal, left, right)
            assert_close_o(to_f64(O[:, h:h + 1], dtype), Or, dtype, f"O H={H} h={h}")
            assert_close_lse(L[:, h:h + 1].cpu().numpy(), Lr, f"LSE H={H} h={h}")


@pytest.mark.parametrize("case", [
    # Hq, Hkv, Nq, Nk, D, dtype, causal, left, right, chained
    (4, 4, 512, 512, 128, "f16", True, -1, -1, True),      # 4 tiles: pairs (3, 0), (2, 1)
    (4, 2, 400, 400, 128, "bf16", True, -1, -1, True),     # partial last tile, GQA
    (2, 2, 256, 700, 64, "f16", True, -1, -1, True),       # Nq < Nk (bottom-right)
    (2, 1, 512, 512, 128, "bf16", False, -1, -1, True),    # no mask: equal tiles
    (4, 4, 768, 768, 128, "f16", True, 200, 0, True),      # window
    (2, 2, 384, 384, 128, "f16", True, -1, -1, False),     # 3 tiles: not chained
])
def test_chained_tiles(case):
    # a small grid of 8-wave workgroups with an even number of query tiles runs two
    # complementary query tiles per workgroup; every row against the oracle
    Hq, Hkv, Nq, Nk, D, dtype, causal, left, right, chained = case
    x = A.dense_inputs(1, Hq, Hkv, Nq, Nk, D, dtype, 60 + Nq + Hq)
    q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
    O, L = run(q, k, v, 1 / math.sqrt(D), causal, left, right)
    info = ea.mfa_last_dispatch()
    assert "groups=2" in info["kernel"] and (",chained" in info["kernel"]) == chained, info["kernel"]
    qf, kf, vf = (oracle.widen(t, dtype) for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention(qf, kf, vf, 1 / math.sqrt(D), causal, left, right)
    assert_close_o(to_f64(O, dtype), Or, dtype, "chained O")
    assert_close_lse(L.cpu().numpy(), Lr, "chained LSE")


def test_fully_masked_rows_exact():
    import torch
    x = A.dense_inputs(1, 2, 2, 300, 90, 128, "f16", 5)
    q, k, v = (to_dev(t, "f16") for t in (x.q, x.k, x.v))
    O, L = run(q, k, v, 0.1, causal=True)
    # rows i < Nq - Nk see no key: O = 0 exactly, LSE = -inf
    assert torch.all(O[:, :, :210] == 0)
    assert torch.all(torch.isneginf(L[:, :, :210]))
    assert torch.all(torch.isfinite(L[:, :, 210:]))


@pytest.mark.parametrize("D,dtype", [(128, "f16"), (64, "bf16"), (128, "bf16")])
def test_causal_row0_bitexact(D, dtype):
    # row 0 sees key 0 only: P = exp2(0) = 1, l = 1, so O[0] is V[0] bit for bit
    x = A.dense_inputs(2, 4, 2, 257, 257, D, dtype, 7)
    q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
    O, L = run(q, k, v, 1 / math.sqrt(D), causal=True)
    import torch
    Ob = O[:, :, 0].contiguous().view(torch.int16).cpu().numpy()
    Vb = v[:, [0, 0, 1, 1], 0].contiguous().view(torch.int16).cpu().numpy()
    assert np.array_equal(Ob, Vb)


@pytest.mark.parametrize("case", [
    (700, 700, 128, True, -1, -1), (700, 700, 64, True, 100, 0), (600, 900, 128, True, -1, -1),
    (1000, 1000, 128, False, 60, 90), (300, 1000, 128, False, -1, -1), (129, 5, 64, True, -1, -1),
    (4096, 4096, 128, True, -1, -1), (8192, 8192, 128, True, 512, 0),
])
def test_tile_visits_match_plan_and_oracle(case):
    import torch
    Nq, Nk, D, causal, left, right = case
    x = A.dense_inputs(1, 2, 1, Nq, Nk, D, "f16", 11)
    q, k, v = (to_dev(t, "f16") for t in (x.q, x.k, x.v))
    plan, ranges = ea.mfa_plan_fwd(Nq, Nk, D, ea.MFA_F16, causal, left, right)
    log = torch.full((1 * 2 * plan["n_q_tiles"] * 4,), -7, dtype=torch.int32, device="cuda")
    print(f"tilelog {case}", flush=True)
    ea.mfa_fwd(q, k, v, scale=0.1, causal=causal, win_left=left, win_right=right, tile_log=log)
    torch.cuda.synchronize()
    # the logging kernel takes the layout the plain call would: on these small grids two
    # wave groups, chaining two query tiles per workgroup when their number is even
    kern = ea.mfa_last_dispatch()["kernel"]
    assert ",tilelog" in kern and "groups=2" in kern, kern
    assert (",chained" in kern) == (plan["n_q_tiles"] % 2 == 0), kern
    log = log.view(2, plan["n_q_tiles"], 4).cpu().numpy()
    ref = oracle.visited_tiles(Nq, Nk, plan["BM"], plan["BN"], causal, left, right)
    for h in range(2):
        for t in range(plan["n_q_tiles"]):
            first, count, edge, end = log[h, t]
            tiles = ref[t]
            assert count == len(tiles), (h, t, count, tiles)
            if tiles:
                assert first == tiles[0] and end == tiles[-1] + 1
                assert (first, end) == ranges[t]
            else:
                assert first == -1 and end == -1
    assert int(log[..., 1].sum()) == 2 * plan["visited"]
    assert int(log[..., 2].sum()) == 2 * plan["edge"]


@pytest.mark.parametrize("mode", ["causal", "window"])
def test_perturbation_invariance_bitwise(mode):
    # keys invisible to a block of rows may hold anything finite: those rows' outputs
    # stay bit-identical
    import torch
    N, D, r = 640, 128, 300
    x = A.dense_inputs(1, 2, 2, N, N, D, "f16", 21)
    q, k, v = (to_dev(t, "f16") for t in (x.q, x.k, x.v))
    if mode == "causal":
        O0, L0 = run(q, k, v, 0.09, causal=True)
        k2, v2 = k.clone(), v.clone()
        k2[:, :, r + 1:] = 7.0
        v2[:, :, r + 1:] = -3.0
        O1, L1 = run(q, k2, v2, 0.09, causal=True)
        rows = slice(0, r + 1)
    else:
        left = 50
        O0, L0 = run(q, k, v, 0.09, causal=True, left=left, right=0)
        k2, v2 = k.clone(), v.clone()
        k2[:, :, : r - left] = 5.0
        v2[:, :, : r - left] = 11.0
        O1, L1 = run(q, k2, v2, 0.09, causal=True, left=left, right=0)
        rows = slice(r, N)
    assert torch.equal(O0[:, :, rows].view(torch.int16), O1[:, :, rows].view(torch.int16))
    assert torch.equal(L0[:, :, rows], L1[:, :, rows])
    # and the perturbation is visible elsewhere (the test would be vacuous otherwise)
    assert not torch.equal(O0, O1)


def test_deterministic():
    import torch
    x = A.dense_inputs(2, 8, 2, 1000, 1000, 128, "bf16", 3)
    q, k, v = (to_dev(t, "bf16") for t in (x.q, x.k, x.v))
    O0, L0 = run(q, k, v, 0.08, causal=True)
    O1, L1 = run(q, k, v, 0.08, causal=True)
    assert torch.equal(O0.view(torch.int16), O1.view(torch.int16)) and torch.equal(L0, L1)


def test_prepared_call_holds_its_tensors():
    # ea.prepare() repeats a call with marshalled raw pointers; the callable must keep the
    # tensors behind them (inputs, and outputs the binding allocated itself) alive after the
    # caller drops its references, or their memory would be handed to other tensors
    import torch

    def make():
        x = A.dense_inputs(1, 4, 2, 300, 300, 128, "f16", 41)
        q, k, v = (to_dev(t, "f16") for t in (x.q, x.k, x.v))
        return ea.prepare(ea.mfa_fwd, q, k, v, scale=0.09, causal=True), x

    step, x = make()
    junk = [torch.full((1 << 20,), 7.0, dtype=torch.float16, device="cuda") for _ in range(8)]
    step()
    torch.cuda.synchronize()
    out, lse = step.keep[2][3], step.keep[2][4]   # held in marshalling order: q, k, v, out, lse
    assert tuple(out.shape) == (1, 4, 300, 128) and tuple(lse.shape) == (1, 4, 300)
    qf, kf, vf = (oracle.widen(t, "f16") for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention(qf, kf, vf, 0.09, True)
    assert_close_o(to_f64(out, "f16"), Or, "f16", "prepared O")
    assert_close_lse(lse.cpu().numpy(), Lr, "prepared LSE")
    del junk


# Dense GQA on a large grid (more than two query tiles per CU) runs one 8-wave workgroup
# per pair of query heads that share a KV head (both groups walk the same key tiles from one K/V stream in LDS); an odd group
# size keeps the 4-wave layout.  Hq, Hkv, Nq, Nk, D, dtype, causal, left, right, scale, pairs
PAIR_CASES = [
    (128, 64, 520, 520, 128, "f16", True, -1, -1, None, True),      # g = 2, ragged last tile
    (96, 16, 700, 800, 64, "bf16", False, 40, 17, None, True),      # g = 6, window, Nk > Nq
    (128, 32, 600, 600, 128, "f16", True, -1, -1, -0.1, True),      # g = 4, negative scale
    (64, 16, 1100, 1100, 128, "bf16", True, 300, 0, None, True),    # g = 4, causal window
    (192, 64, 300, 300, 128, "bf16", True, -1, -1, None, False),    # g = 3: 4-wave groups
]


@pytest.mark.parametrize("case", PAIR_CASES, ids=[str(i) for i in range(len(PAIR_CASES))])
def test_head_pairs(case):
    import torch
    Hq, Hkv, Nq, Nk, D, dtype, causal, left, right, scale, pairs = case
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    x = A.dense_inputs(1, Hq, Hkv, Nq, Nk, D, dtype, 900 + Hq + Nq)
    q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
    O, L = run(q, k, v, scale, causal, left, right)
    kern = ea.mfa_last_dispatch()["kernel"]
    assert (",head-pairs" in kern) == pairs and ("groups=2" in kern) == pairs, kern
    # (one 4-wave group with Hkv a multiple of 8: head-major order per XCD)
    assert (",head-major" in kern) == (not pairs and Hkv % 8 == 0), kern
    # both heads of the first and the last pair, and one pair in the middle
    g = Hq // Hkv
    heads = sorted({0, 1, Hq // 2, Hq // 2 + 1, Hq - 2, Hq - 1})
    for h in heads:
        kv = h // g
        qf = oracle.widen(x.q[:, h:h + 1], dtype)
        kf, vf = (oracle.widen(t[:, kv:kv + 1], dtype) for t in (x.k, x.v))
        Or, Lr = oracle.attention(qf, kf, vf, scale, causal, left, right)
        assert_close_o(to_f64(O[:, h:h + 1], dtype), Or, dtype, f"O h={h}")
        assert_close_lse(L[:, h:h + 1].cpu().numpy(), Lr, f"LSE h={h}")
    # the per-tile visit record: each group writes its own head's records
    plan, ranges = ea.mfa_plan_fwd(Nq, Nk, D, ea.MFA_F16 if dtype == "f16" else ea.MFA_BF16,
                                   causal, left, right)
    log = torch.full((Hq * plan["n_q_tiles"] * 4,), -7, dtype=torch.int32, device="cuda")
    ea.mfa_fwd(q, k, v, scale=scale, causal=causal, win_left=left, win_right=right, tile_log=log)
    torch.cuda.synchronize()
    assert (",head-pairs" in ea.mfa_last_dispatch()["kernel"]) == pairs
    log = log.view(Hq, plan["n_q_tiles"], 4).cpu().numpy()
    ref = oracle.visited_tiles(Nq, Nk, plan["BM"], plan["BN"], causal, left, right)
    for t in range(plan["n_q_tiles"]):
        want = (ref[t][0], len(ref[t]), ref[t][-1] + 1) if ref[t] else (-1, 0, -1)
        assert np.all(log[:, t, 0] == want[0]) and np.all(log[:, t, 1] == want[1]), (t, log[:, t])
        assert np.all(log[:, t, 3] == want[2]), (t, log[:, t])
    assert int(log[..., 2].sum()) == Hq * plan["edge"]
