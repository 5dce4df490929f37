"""GPU parity of the paged split-KV decode (mfa_decode_paged through the C ABI)."""
import math

import numpy as np
import pytest

import attn_inputs as A
import oracle
from gpu_util import assert_close_lse, assert_close_o, to_dev, to_f64

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


def run(d, scale, num_splits=0, workspace=None, bt=None, kp=None, vp=None):
    import torch
    print(f"mfa_decode_paged B={d.q.shape[0]} Hq={d.q.shape[1]} pool={tuple(d.kp.shape)} "
          f"splits={num_splits}", flush=True)
    O, L = ea.mfa_decode_paged(d.q, d.kp if kp is None else kp, d.vp if vp is None else vp,
                               d.bt if bt is None else bt, d.sl, scale=scale,
                               num_splits=num_splits, workspace=workspace)
    torch.cuda.synchronize()
    return O, L


def ref(p, scale):
    return oracle.decode_paged(oracle.widen(p.q, p.dtype), oracle.widen(p.k_pages, p.dtype),
                               oracle.widen(p.v_pages, p.dtype), p.block_table, p.seq_lens, scale,
                               p.page_size)


CASES = [
    # B, Hq, Hkv, D, dtype, len_lo, len_hi, seq_lens
    (3, 8, 2, 128, "bf16", 1, 300, None),
    (4, 32, 8, 128, "bf16", 1000, 3000, None),
    (2, 4, 4, 64, "f16", 1, 100, None),
    (5, 16, 2, 128, "f16", 1, 2000, [1, 15, 16, 17, 2000]),
    (2, 6, 2, 64, "bf16", 50, 600, None),      # g = 3
    (3, 16, 2, 128, "bf16", 100, 900, None),   # g = 8: two head groups per KV head
    (1, 2, 1, 128, "f16", 4096, 4096, None),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_decode_vs_oracle(case):
    B, Hq, Hkv, D, dt, lo, hi, sl = case
    p = A.paged_inputs(B, Hq, Hkv, D, dt, 500 + B + Hq, len_lo=lo, len_hi=hi, extra_pages=3,
                       seq_lens=sl)
    scale = 1 / math.sqrt(D)
    d = Dev(p)
    O, L = run(d, scale)
    Or, Lr = ref(p, scale)
    assert_close_o(to_f64(O, dt), Or, dt, "decode O")
    assert_close_lse(L.cpu().numpy(), Lr, "decode LSE")
    info = ea.mfa_last_dispatch()
    assert info["op"] == 2 and info["kernel"].startswith("mfa_decode_split_kernel")
    assert info["num_splits"] == ea.mfa_decode_num_splits(16, p.block_table.shape[1], 0)


@pytest.mark.parametrize("B", [256, 257])
def test_both_grids(B):
    # up to 256 sequences the split kernel's grid lists only the non-empty chunks (each
    # workgroup finds its item from seq_lens); above, the grid is (chunk, head group,
    # sequence) and empty chunks return at once.  Both against the oracle, with zero-length
    # and single-token sequences among them.
    lens = np.random.default_rng(B).integers(0, 400, size=B)
    lens[:3] = [0, 1, 16]
    p = A.paged_inputs(B, 4, 1, 64, "bf16", 60 + B, len_lo=0, len_hi=400, seq_lens=lens,
                       extra_pages=1)
    d = Dev(p)
    O, L = run(d, 0.11)
    info = ea.mfa_last_dispatch()
    assert (",flat" in info["kernel"]) == (B <= 256), info["kernel"]
    Or, Lr = ref(p, 0.11)
    assert_close_o(to_f64(O, "bf16"), Or, "bf16", f"decode O B={B}")
    assert_close_lse(L.cpu().numpy(), Lr, f"decode LSE B={B}")


def test_empty_sequence():
    import torch
    p = A.paged_inputs(3, 8, 2, 128, "bf16", 9, len_lo=1, len_hi=200, seq_lens=[0, 33, 200])
    d = Dev(p)
    O, L = run(d, 0.1)
    assert torch.all(O[0] == 0) and torch.all(torch.isneginf(L[0]))
    Or, Lr = ref(p, 0.1)
    assert_close_o(to_f64(O, "bf16")[1:], Or[1:], "bf16")
    assert_close_lse(L.cpu().numpy()[1:], Lr[1:])


def test_paged_decode_workload_full():
    c = A.workload("paged_splitkv_decode")
    p = A.workload_inputs("paged_splitkv_decode")
    d = Dev(p)
    O, L = run(d, c["scale"])
    Or, Lr = ref(p, c["scale"])
    eo = assert_close_o(to_f64(O, "bf16"), Or, "bf16", "paged decode workload")
    el = assert_close_lse(L.cpu().numpy(), Lr, "paged decode workload")
    print(f"paged decode workload: max|dO|={eo:.2e} max|dLSE|={el:.2e} seq_lens={p.seq_lens.tolist()}")


def test_split_count_invariance():
    import torch
    p = A.paged_inputs(4, 16, 4, 128, "bf16", 77, len_lo=100, len_hi=2500)
    d = Dev(p)
    max_pages = p.block_table.shape[1]
    outs = []
    for ns in (1, 2, 0, max_pages):
        O, L = run(d, 0.09, num_splits=ns)
        outs.append((ns, O.float(), L))
    O0, L0 = outs[0][1], outs[0][2]
    for ns, O, L in outs[1:]:
        # different splits differ only by fp32 rounding before the final bf16 rounding
        assert float((O - O0).abs().max()) <= 2 ** -7, ns
        assert float((L - L0).abs().max()) <= 1e-5, ns


def test_page_permutation_bitwise():
    import torch
    p = A.paged_inputs(4, 8, 2, 128, "f16", 31, len_lo=10, len_hi=1500, extra_pages=5)
    d = Dev(p)
    O0, L0 = run(d, 0.1)
    P = p.k_pages.shape[0]
    perm = np.random.default_rng(3).permutation(P)
    inv = np.argsort(perm)
    bt2 = np.where(p.block_table >= 0, inv[np.maximum(p.block_table, 0)], -1).astype(np.int32)
    kp2 = to_dev(p.k_pages[perm], "f16")
    vp2 = to_dev(p.v_pages[perm], "f16")
    O1, L1 = run(d, 0.1, bt=torch.from_numpy(bt2).to("cuda"), kp=kp2, vp=vp2)
    assert torch.equal(O0.view(torch.int16), O1.view(torch.int16)) and torch.equal(L0, L1)


def test_decode_equals_last_prefill_row():
    # decode of sequence L with query q equals the bottom-right causal prefill row
    import torch
    p = A.paged_inputs(2, 8, 2, 128, "bf16", 13, len_lo=700, len_hi=1300)
    d = Dev(p)
    Od, Ld = run(d, 0.1)
    for b in range(2):
        n = int(p.seq_lens[b])
        kk = oracle.gather_paged(p.k_pages, p.block_table, b, n, 16).transpose(1, 0, 2)[None]
        vv = oracle.gather_paged(p.v_pages, p.block_table, b, n, 16).transpose(1, 0, 2)[None]
        q = to_dev(p.q[b][None, :, None, :], "bf16")
        Of, Lf = ea.mfa_fwd(q, to_dev(np.ascontiguousarray(kk), "bf16"),
                            to_dev(np.ascontiguousarray(vv), "bf16"), scale=0.1, causal=True)
        torch.cuda.synchronize()
        assert float((Of[0, :, 0].float() - Od[b].float()).abs().max()) <= 1.5e-2
        assert float((Lf[0, :, 0] - Ld[b]).abs().max()) <= 1e-3


def test_workspace_slot_scan():
    # pattern-fill the workspace: exactly the slots of non-empty splits get written
    import torch
    p = A.paged_inputs(3, 8, 2, 128, "bf16", 55, len_lo=1, len_hi=1000, seq_lens=[1, 513, 1000])
    d = Dev(p)
    B, Hq, D = 3, 8, 128
    max_pages = p.block_table.shape[1]
    for ns in (0, 3, max_pages):
        S = ea.mfa_decode_num_splits(16, max_pages, ns)
        nbytes = ea.mfa_decode_workspace_bytes(B, Hq, D, 16, max_pages, ns)
        ws = torch.full((nbytes // 4,), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
        run(d, 0.1, num_splits=ns, workspace=ws)
        info = ea.mfa_last_dispatch()
        chunk_pages = info["chunk_tokens"] // 16
        raw = ws.cpu().numpy()
        wo = raw[: B * Hq * S * D].reshape(B, Hq, S, D)
        wl = raw[B * Hq * S * D:].reshape(B, Hq, S)
        for b in range(B):
            used = -(-(-(-int(p.seq_lens[b]) // 16)) // chunk_pages)
            written = wl[b, :, :used].view(np.float32)
            assert np.all(np.isfinite(written)), (ns, b)
            assert np.all(np.isfinite(wo[b, :, :used].view(np.float32)))
            assert np.all(wl[b, :, used:] == 0x7F7F7F7F), (ns, b, "stray write")
            assert np.all(wo[b, :, used:] == 0x7F7F7F7F), (ns, b, "stray write")


def test_decode_deterministic():
    import torch
    p = A.paged_inputs(4, 32, 8, 128, "bf16", 99, len_lo=1, len_hi=4000)
    d = Dev(p)
    O0, L0 = run(d, 0.1)
    O1, L1 = run(d, 0.1)
    assert torch.equal(O0.view(torch.int16), O1.view(torch.int16)) and torch.equal(L0, L1)
