"""GPU parity of the packed variable-length forward (mfa_fwd_varlen through the C ABI)
against the oracle's attention_varlen."""
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


def run(x, scale, causal=False, left=-1, right=-1, max_q=None, max_k=None, out=None,
        tile_log=None):
    import torch
    lq = np.diff(x.cu_seqlens_q)
    lk = np.diff(x.cu_seqlens_k)
    max_q = int(max(1, lq.max())) if max_q is None else max_q
    max_k = int(max(1, lk.max())) if max_k is None else max_k
    q, k, v = (to_dev(t, x.dtype) for t in (x.q, x.k, x.v))
    print(f"mfa_fwd_varlen q={tuple(q.shape)} k={tuple(k.shape)} {x.dtype} B={len(lq)} "
          f"lq={lq.tolist()[:8]} lk={lk.tolist()[:8]} causal={causal} win=({left},{right})",
          flush=True)
    O, L = ea.mfa_fwd_varlen(q, k, v, dev_i32(x.cu_seqlens_q), dev_i32(x.cu_seqlens_k), max_q, max_k,
                             scale=scale, causal=causal, win_left=left, win_right=right, out=out,
                             tile_log=tile_log)
    torch.cuda.synchronize()
    return O, L


def oracle_of(x, scale, causal, left=-1, right=-1, rows=None):
    qf, kf, vf = (oracle.widen(t, x.dtype) for t in (x.q, x.k, x.v))
    return oracle.attention_varlen(qf, kf, vf, x.cu_seqlens_q, x.cu_seqlens_k, scale, causal,
                                   left, right, rows=rows)


def in_seq_tokens(x):
    return int(x.cu_seqlens_q[-1])


def check(x, scale, causal, left=-1, right=-1, what="", **kw):
    O, L = run(x, scale, causal, left, right, **kw)
    Or, Lr = oracle_of(x, scale, causal, left, right)
    T = in_seq_tokens(x)
    eo = assert_close_o(to_f64(O, x.dtype)[:T], Or[:T], x.dtype, f"O {what}")
    el = assert_close_lse(L.cpu().numpy()[:, :T], Lr[:, :T], f"LSE {what}")
    info = ea.mfa_last_dispatch()
    assert info["op"] == 3 and ",varlen" in info["kernel"] and info["planned"] == -1
    return O, L, eo, el


PACKS = [
    # Hq, Hkv, D, dtype, seqlens_q, seqlens_k (None = same), causal, left, right
    (4, 4, 128, "f16", [1, 130, 257, 64, 500, 3], None, True, -1, -1),
    (4, 2, 64, "bf16", [1, 130, 257, 64, 500, 3], None, False, -1, -1),
    (8, 2, 128, "bf16", [100, 1, 300, 64], [500, 77, 300, 1000], True, -1, -1),   # chunked prefill
    (2, 1, 128, "f16", [300, 129, 2], [90, 129, 700], True, -1, -1),             # Lq > Lk rows
    (4, 4, 128, "f16", [400, 700, 33], None, True, 37, 0),                        # window
    (2, 2, 64, "bf16", [256, 511, 128], [256, 600, 1], False, 20, 45),            # two-sided
    (3, 1, 128, "bf16", [0, 200, 0, 77, 1], [10, 0, 5, 77, 1], True, -1, -1),     # empty parts
    (2, 2, 128, "f16", [640], [640], False, -1, 3),                               # one sequence
]


@pytest.mark.parametrize("case", PACKS, ids=[str(i) for i in range(len(PACKS))])
def test_packs_match_oracle(case):
    Hq, Hkv, D, dtype, lq, lk, causal, left, right = case
    x = A.varlen_inputs(Hq, Hkv, D, dtype, 200 + sum(lq), seqlens_q=lq, seqlens_k=lk)
    _, L, eo, el = check(x, 1 / math.sqrt(D), causal, left, right, what=str(case))
    print(f"pack {case}: max|dO|={eo:.2e} max|dLSE|={el:.2e} {ea.mfa_last_dispatch()['kernel']}")


def test_keyless_rows_and_padding_untouched():
    # a sequence with queries but no keys gives O = 0 and LSE = -inf; tokens after the last
    # sequence belong to none and their output rows are not written
    import torch
    x = A.varlen_inputs(2, 2, 128, "f16", 5, seqlens_q=[70, 90, 40], seqlens_k=[100, 0, 40],
                        pad_q=50, pad_k=20)
    T = in_seq_tokens(x)
    out = torch.full(x.q.shape, 3.0, dtype=torch.float16, device="cuda")
    O, L = run(x, 0.1, True, out=out)
    Ob = O.cpu()
    assert torch.all(Ob[70:160] == 0) and torch.all(torch.isneginf(L[:, 70:160].cpu()))
    assert torch.all(Ob[T:] == 3.0)
    Or, Lr = oracle_of(x, 0.1, True)
    assert_close_o(to_f64(O, "f16")[:T], Or[:T], "f16", "keyless")
    assert_close_lse(L.cpu().numpy()[:, :T], Lr[:, :T], "keyless")


def test_both_workgroup_layouts():
    # few query tiles: two key-splitting wave groups per workgroup; many: one group (packed
    # sequences take no head pairs, whatever the group size)
    for Hq, Hkv, layout in ((2, 2, "groups=2"), (64, 2, "groups=1"), (72, 24, "groups=1")):
        x = A.varlen_inputs(Hq, Hkv, 128, "bf16", 40 + Hq, seqlens_q=[900, 1, 640, 459])
        O, L = run(x, 0.09, True)
        info = ea.mfa_last_dispatch()
        assert layout in info["kernel"], info["kernel"]
        g = Hq // Hkv
        for h in sorted({0, 1, Hq - 2, Hq - 1}):
            kv = h // g
            sub = A.VarlenInputs(x.q[:, h:h + 1], x.k[:, kv:kv + 1], x.v[:, kv:kv + 1],
                                 x.cu_seqlens_q, x.cu_seqlens_k, "bf16")
            Or, Lr = oracle_of(sub, 0.09, True)
            assert_close_o(to_f64(O[:, h:h + 1], "bf16"), Or, "bf16", f"Hq={Hq} h={h}")
            assert_close_lse(L[h:h + 1].cpu().numpy(), Lr, f"Hq={Hq} h={h}")


@pytest.mark.parametrize("causal,left,right", [(True, -1, -1), (True, 100, 0), (False, 60, 90)])
def test_tile_visits_per_sequence(causal, left, right):
    import torch
    lq, lk = [700, 1, 300, 129, 0], [700, 900, 1000, 5, 3]
    x = A.varlen_inputs(2, 1, 128, "f16", 11, seqlens_q=lq, seqlens_k=lk)
    plan, _ = ea.mfa_plan_fwd(max(lq), max(lk), 128, ea.MFA_F16, causal, left, right, False)
    BM, BN = plan["BM"], plan["BN"]
    nqt = math.ceil(max(lq) / BM)
    log = torch.full((len(lq) * 2 * nqt * 4,), -7, dtype=torch.int32, device="cuda")
    run(x, 0.1, causal, left, right, tile_log=log)
    log = log.view(len(lq), 2, nqt, 4).cpu().numpy()
    for b in range(len(lq)):
        ref = oracle.visited_tiles(lq[b], lk[b], BM, BN, causal, left, right) if lq[b] else []
        for h in range(2):
            for t in range(nqt):
                first, count, edge, end = log[b, h, t]
                tiles = ref[t] if t < len(ref) else []
                assert count == len(tiles), (b, h, t, count, tiles)
                assert 0 <= edge <= count
                if tiles:
                    assert first == tiles[0] and end == tiles[-1] + 1
                else:
                    assert first == -1 and end == -1


def test_sequences_isolated_bitwise():
    # changing the tokens of one sequence leaves every other sequence's rows bit-identical
    import torch
    x = A.varlen_inputs(4, 2, 128, "bf16", 8, seqlens_q=[300, 200, 257], seqlens_k=[300, 500, 257])
    O0, L0 = run(x, 0.08, True)
    y = A.VarlenInputs(x.q.copy(), x.k.copy(), x.v.copy(), x.cu_seqlens_q, x.cu_seqlens_k, "bf16")
    y.q[300:500] = A.round_f32_to_bits(np.full((200, 4, 128), 2.0, np.float32), "bf16")
    y.k[300:800] = A.round_f32_to_bits(np.full((500, 2, 128), -1.5, np.float32), "bf16")
    y.v[300:800] = A.round_f32_to_bits(np.full((500, 2, 128), 9.0, np.float32), "bf16")
    O1, L1 = run(y, 0.08, True)
    for sl in (slice(0, 300), slice(500, 757)):
        assert torch.equal(O0[sl].view(torch.int16), O1[sl].view(torch.int16))
        assert torch.equal(L0[:, sl], L1[:, sl])
    assert not torch.equal(O0[300:500], O1[300:500])


def test_single_sequence_equals_dense_entry_point():
    # one packed sequence with one head is the dense problem [1, 1, N, D]: the same tiles
    # in the same order, hence bit-identical results
    import torch
    N = 777
    x = A.varlen_inputs(1, 1, 128, "f16", 9, seqlens_q=[N], seqlens_k=[N])
    O, L = run(x, 0.1, True, 50, 0)
    q, k, v = (to_dev(t, "f16").permute(1, 0, 2).unsqueeze(0).contiguous() for t in (x.q, x.k, x.v))
    Od, Ld = ea.mfa_fwd(q, k, v, scale=0.1, causal=True, win_left=50, win_right=0)
    torch.cuda.synchronize()
    assert "groups=2" in ea.mfa_last_dispatch()["kernel"]
    assert np.array_equal(to_bits(O[:, 0]), to_bits(Od[0, 0]))
    assert torch.equal(L[0], Ld[0, 0])


def test_deterministic():
    import torch
    x = A.varlen_inputs(8, 2, 128, "bf16", 3, B=6, len_lo=1, len_hi=900)
    O0, L0 = run(x, 0.08, True)
    O1, L1 = run(x, 0.08, True)
    assert torch.equal(O0.view(torch.int16), O1.view(torch.int16)) and torch.equal(L0, L1)


def test_full_size_packed_workload_sampled():
    # the packed causal prefill workload at full size, checked on sampled rows: the first,
    # the last and a middle token of every sequence (first and last head) plus random rows
    import torch
    c = A.workload("packed_varlen_causal_prefill")
    x = A.workload_inputs("packed_varlen_causal_prefill")
    O, L = run(x, c["scale"], c["causal"])
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(L).all())
    cu = x.cu_seqlens_q
    rows = set()
    for b in range(c["B"]):
        for t in (int(cu[b]), int(cu[b + 1]) - 1, (int(cu[b]) + int(cu[b + 1])) // 2):
            rows.add((t, 0))
            rows.add((t, c["Hq"] - 1))
    rng = np.random.default_rng(6)
    while len(rows) < 160:
        rows.add((int(rng.integers(int(cu[-1]))), int(rng.integers(c["Hq"]))))
    rows = sorted(rows)
    Or, Lr = oracle_of(x, c["scale"], c["causal"], rows=rows)
    t_idx, h_idx = (np.array(r) for r in zip(*rows))
    Og = to_f64(O, c["dtype"])[t_idx, h_idx]
    Lg = L.cpu().numpy()[h_idx, t_idx]
    eo = assert_close_o(Og, Or, c["dtype"], "packed workload")
    el = assert_close_lse(Lg, Lr, "packed workload")
    print(f"packed workload: max|dO|={eo:.2e} max|dLSE|={el:.2e} kernel={ea.mfa_last_dispatch()['kernel']}")


# Sequence-major order (at most 64 sequences, Hkv a multiple of 8): each XCD takes whole KV
# heads and runs the sequences longest first, a sequence's tiles of one KV head back to
# back; every (sequence, head, tile) must still be computed exactly once, and the tile
# records of empty sequences are written by each XCD's first workgroup.
# Hq, Hkv, lq, lk, causal, left, right, dtype
SEQ_MAJOR = [
    (16, 8, [700, 1, 300, 129, 0, 1000], [700, 900, 1000, 5, 3, 1200], True, -1, -1, "bf16"),
    (32, 16, [257, 513, 0, 40], [257, 600, 7, 40], True, 100, 0, "f16"),
    (8, 8, [200] * 64, [300] * 64, False, -1, -1, "bf16"),    # 64 sequences: the limit
    (24, 8, [0, 0, 129], [10, 0, 129], True, -1, -1, "f16"),   # mostly empty, g = 3
]


@pytest.mark.parametrize("case", SEQ_MAJOR, ids=[str(i) for i in range(len(SEQ_MAJOR))])
def test_sequence_major_order(case):
    import torch
    Hq, Hkv, lq, lk, causal, left, right, dt = case
    x = A.varlen_inputs(Hq, Hkv, 128, dt, 60 + Hq + len(lq), seqlens_q=lq, seqlens_k=lk)
    O, L = run(x, 0.09, causal, left, right)
    assert ",seq-major" in ea.mfa_last_dispatch()["kernel"], ea.mfa_last_dispatch()["kernel"]
    Or, Lr = oracle_of(x, 0.09, causal, left, right)
    T = in_seq_tokens(x)
    assert_close_o(to_f64(O, dt)[:T], Or[:T], dt, "seq-major O")
    assert_close_lse(L.cpu().numpy()[:, :T], Lr[:, :T], "seq-major LSE")
    # per-tile visit records of every (sequence, head)
    plan, _ = ea.mfa_plan_fwd(max(max(lq), 1), max(max(lk), 1), 128,
                              ea.MFA_F16 if dt == "f16" else ea.MFA_BF16, causal, left, right, False)
    BM, BN = plan["BM"], plan["BN"]
    nqt = max(1, math.ceil(max(lq) / BM))
    log = torch.full((len(lq) * Hq * nqt * 4,), -7, dtype=torch.int32, device="cuda")
    run(x, 0.09, causal, left, right, tile_log=log)
    assert ",seq-major" in ea.mfa_last_dispatch()["kernel"]
    log = log.view(len(lq), Hq, nqt, 4).cpu().numpy()
    for b in range(len(lq)):
        ref = oracle.visited_tiles(lq[b], lk[b], BM, BN, causal, left, right) if lq[b] else []
        for t in range(nqt):
            tiles = ref[t] if t < len(ref) else []
            want = (tiles[0], len(tiles), tiles[-1] + 1) if tiles else (-1, 0, -1)
            got = log[b, :, t]
            assert np.all(got[:, 0] == want[0]) and np.all(got[:, 1] == want[1]), (b, t, got, want)
            assert np.all(got[:, 3] == want[2]), (b, t, got, want)


def test_sequence_major_limits():
    # more than 64 sequences, or Hkv not a multiple of 8: the round order
    for Hq, Hkv, B in ((8, 8, 65), (8, 4, 10)):
        x = A.varlen_inputs(Hq, Hkv, 64, "f16", 70 + B, seqlens_q=[33] * B, seqlens_k=[40] * B)
        O, L = run(x, 0.125, True)
        assert ",seq-major" not in ea.mfa_last_dispatch()["kernel"]
        Or, Lr = oracle_of(x, 0.125, True)
        T = in_seq_tokens(x)
        assert_close_o(to_f64(O, "f16")[:T], Or[:T], "f16", f"B={B} Hkv={Hkv}")
        assert_close_lse(L.cpu().numpy()[:, :T], Lr[:, :T], f"B={B} Hkv={Hkv}")
