"""The work counts bench.py divides by, checked by brute force on small shapes (CPU only)."""
import os
import sys

import numpy as np

import attn_inputs as A
import oracle

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_visible_pairs_brute_force():
    for Nq, Nk, causal, left, right in ((300, 300, True, -1, -1), (100, 700, True, 50, 0),
                                        (500, 200, False, 30, 7), (64, 64, False, -1, -1)):
        vis = oracle.visible(np.arange(Nq)[:, None], np.arange(Nk)[None, :], Nq, Nk, causal, left,
                             right)
        assert bench.visible_pairs(Nq, Nk, causal, left, right) == int(vis.sum())


def test_block_sparse_pairs_brute_force():
    bm = A.block_mask_inputs(1, 3, 768, 768, 128, 128, 0.35, 9)
    vis = oracle.visible(np.arange(768)[:, None], np.arange(768)[None, :], 768, 768, True, -1, -1)
    ref = sum(int((vis & np.kron(bm[0, h].astype(bool), np.ones((128, 128), bool))).sum())
              for h in range(3))
    assert bench.block_sparse_pairs(bm, 768, 768, 128, 128) == ref


def test_decode_bytes_counts_every_cached_token_once():
    p = A.paged_inputs(3, 8, 2, 64, "bf16", 3, len_lo=1, len_hi=100)
    L = p.seq_lens.astype(np.int64)
    expect = int(L.sum()) * 2 * 64 * 2 * 2 + 2 * 3 * 8 * 64 * 2 + 3 * 8 * 4 + 4 * int(np.ceil(L / 16).sum()) + 12
    assert bench.decode_bytes(p, 2, 64, 8) == expect


def test_prefill_bytes_and_roofline_model():
    # bytes of the seeded arrays themselves: q, k, v, out (2 bytes per element) and fp32 LSE
    c = dict(B=1, Hq=4, Hkv=2, Nq=96, Nk=160, D=64)
    x = A.dense_inputs(c["B"], c["Hq"], c["Hkv"], c["Nq"], c["Nk"], c["D"], "f16", 5)
    expect = x.q.nbytes * 2 + x.k.nbytes + x.v.nbytes + c["B"] * c["Hq"] * c["Nq"] * 4
    assert bench.prefill_bytes(c) == expect
    # below the ridge the attainable rate is intensity x bandwidth, above it the MFMA peak
    lo = bench.roofline_model(flop=100e9, nbytes=1e9, tflops=200.0)
    assert lo["bound"] == "hbm" and abs(lo["attainable_tflops"] - 800.0) < 1e-9
    assert abs(lo["frac_of_attainable"] - 0.25) < 1e-12
    hi = bench.roofline_model(flop=1000e9, nbytes=1e9, tflops=500.0)
    assert hi["bound"] == "mfma" and hi["attainable_tflops"] == bench.PEAK_MFMA_F16
    assert abs(hi["frac_of_attainable"] - 0.2) < 1e-12
