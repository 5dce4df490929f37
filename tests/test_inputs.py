"""The seeded generator: determinism, rounding and the paged layout.  CPU only."""
import numpy as np
import pytest

import attn_inputs as A


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [np.inf, -np.inf, 0.0, -0.0]
    ours = A.round_f32_to_bits(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    assert A.round_f32_to_bits(np.array([np.nan], np.float32), "bf16")[0] == 0x7FC0


def test_f16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 300
    ours = A.round_f32_to_bits(x, "f16")
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_dense_deterministic():
    a = A.dense_inputs(1, 2, 1, 5, 7, 8, "bf16", 3)
    b = A.dense_inputs(1, 2, 1, 5, 7, 8, "bf16", 3)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        np.testing.assert_array_equal(x, y)
    assert a.q.shape == (1, 2, 5, 8) and a.k.shape == (1, 1, 7, 8)


def test_paged_layout():
    p = A.paged_inputs(4, 4, 2, 16, "f16", 9, len_lo=1, len_hi=70, extra_pages=2)
    assert p.block_table.dtype == np.int32 and p.seq_lens.dtype == np.int32
    used = np.concatenate([p.block_table[b, : -(-int(L) // 16)] for b, L in enumerate(p.seq_lens)])
    # every page is dealt to at most one sequence, all in range
    assert len(set(used.tolist())) == len(used) and used.min() >= 0
    assert used.max() < p.k_pages.shape[0]
    for b, L in enumerate(p.seq_lens):
        n = -(-int(L) // 16)
        assert np.all(p.block_table[b, n:] == -1)
        tail = int(L) - 16 * (n - 1)
        last = p.block_table[b, n - 1]
        assert np.all(p.k_pages[last, tail:] == A.NAN_BITS["f16"])
        assert not np.any(p.k_pages[last, :tail] == A.NAN_BITS["f16"])
    unused = sorted(set(range(p.k_pages.shape[0])) - set(used.tolist()))
    assert len(unused) == 2
    assert np.all(p.v_pages[unused] == A.NAN_BITS["f16"])


def test_paged_decode_workload_shape():
    c = A.workload("paged_splitkv_decode")
    assert (c["B"], c["Hq"], c["Hkv"], c["D"], c["page_size"]) == (16, 32, 8, 128, 16)
    assert abs(c["scale"] - 128 ** -0.5) < 1e-15


def test_varlen_layout():
    a = A.varlen_inputs(4, 2, 8, "bf16", 11, B=5, len_lo=1, len_hi=40, pad_q=3, pad_k=2)
    b = A.varlen_inputs(4, 2, 8, "bf16", 11, B=5, len_lo=1, len_hi=40, pad_q=3, pad_k=2)
    np.testing.assert_array_equal(a.q, b.q)
    assert a.cu_seqlens_q.dtype == np.int32 and a.cu_seqlens_q[0] == 0
    assert np.all(np.diff(a.cu_seqlens_q) >= 1) and np.array_equal(a.cu_seqlens_q, a.cu_seqlens_k)
    tq = int(a.cu_seqlens_q[-1])
    assert a.q.shape == (tq + 3, 4, 8) and a.k.shape == (tq + 2, 2, 8)
    assert np.all(a.q[tq:] == A.NAN_BITS["bf16"]) and np.all(a.v[tq:] == A.NAN_BITS["bf16"])
    assert not np.any(a.q[:tq] == A.NAN_BITS["bf16"])
    c = A.varlen_inputs(2, 1, 8, "f16", 12, seqlens_q=[3, 0, 5], seqlens_k=[7, 2, 5])
    assert c.cu_seqlens_q.tolist() == [0, 3, 3, 8] and c.cu_seqlens_k.tolist() == [0, 7, 9, 14]


def test_packed_prefill_workload_shape():
    c = A.workload("packed_varlen_causal_prefill")
    assert (c["B"], c["Hq"], c["Hkv"], c["D"], c["causal"]) == (16, 32, 8, 128, True)
    x = A.workload_inputs("packed_varlen_causal_prefill")
    L = np.diff(x.cu_seqlens_q)
    assert L.min() >= 256 and L.max() <= 4096 and x.q.shape[1:] == (32, 128)


def test_paged_varlen_layout():
    p = A.paged_varlen_inputs(4, 2, 8, "f16", 13, seqlens_q=[3, 20, 1], ctx_lens=[0, 17, 40],
                              extra_pages=2)
    assert p.seq_lens_k.tolist() == [3, 37, 41] and p.cu_seqlens_q.tolist() == [0, 3, 23, 24]
    assert p.q.shape == (24, 4, 8) and p.k_pages.shape == (1 + 3 + 3 + 2, 16, 2, 8)
    assert p.block_table.shape == (3, 3) and p.block_table[0, 1] == -1
    used = np.concatenate([p.block_table[b, : -(-int(L) // 16)] for b, L in enumerate(p.seq_lens_k)])
    assert len(set(used.tolist())) == len(used) == 7
    c = A.workload("paged_chunked_prefill")
    assert (c["B"], c["Hq"], c["Hkv"], c["D"], c["page_size"]) == (8, 32, 8, 128, 16)


def test_grad_inputs_and_backward_workload():
    c = A.workload("dense_causal_backward")
    assert (c["B"], c["Hq"], c["Hkv"], c["Nq"], c["Nk"], c["D"]) == (2, 8, 8, 4096, 4096, 128)
    assert c["dtype"] == "bf16" and c["causal"]
    g0 = A.grad_inputs(1, 2, 64, 128, "bf16", 5)
    g1 = A.grad_inputs(1, 2, 64, 128, "bf16", 5)
    assert g0.shape == (1, 2, 64, 128) and g0.dtype == np.uint16 and np.array_equal(g0, g1)
    x = (g0.astype(np.uint32) << np.uint32(16)).view(np.float32)
    assert abs(x.mean()) < 0.05 and 0.95 < x.std() < 1.05


def test_output_step_is_one_ulp():
    # one step of the output type at |x|: bf16 keeps 8 significant bits, f16 11
    from gpu_util import output_step
    xs = np.array([1.0, 1.5, 2.0, 3.99, 4.0, -2.5, 0.25])
    assert np.array_equal(output_step("bf16", xs), [2 ** -7, 2 ** -7, 2 ** -6, 2 ** -6, 2 ** -5, 2 ** -6, 2 ** -9])
    assert np.array_equal(output_step("f16", xs), [2 ** -10, 2 ** -10, 2 ** -9, 2 ** -9, 2 ** -8, 2 ** -9, 2 ** -12])
    # the next representable value above x is x + step (checked through the generators' rounding)
    for x in (1.0, 2.0, 3.0, 6.0):
        up = A.round_f32_to_bits(np.float32([x + output_step("bf16", np.array([x]))[0]]), "bf16")
        same = A.round_f32_to_bits(np.float32([x + 0.49 * output_step("bf16", np.array([x]))[0]]), "bf16")
        assert up[0] != A.round_f32_to_bits(np.float32([x]), "bf16")[0]
        assert same[0] == A.round_f32_to_bits(np.float32([x]), "bf16")[0]
