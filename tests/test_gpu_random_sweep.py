"""Seeded random sweep: shapes, head grouping, masks, windows, scales, dtypes and
sequence layouts drawn at random, every entry point against the oracle, at sizes the
float64 oracle finishes in about a second.  Each case prints its draw before the GPU
call, so a failure names it.

Tolerances: those of the fixed cases, except that an element of O may also be off by
what the rounding of the arithmetic allows at its magnitude (gpu_util.assert_close_o with
the oracle's attention over |V|).  Large scales make the softmax peaked, so O approaches
single V rows, with |O| above 2.  There one bf16 step (2^-6) alone exceeds the 1.5e-2
bound, and P rounded to bf16 before P V adds up to 2^-8 of sum_j P_ij |V_jd|."""
import math

import numpy as np
import pytest

import attn_inputs as A
import oracle
from gpu_util import assert_close_grads, assert_close_lse, assert_close_o, to_dev, to_f64

pytestmark = pytest.mark.gpu

ea = pytest.importorskip("exact_attention_amd")


def dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def dev_u8(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")


def draw_common(rng):
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    Hkv = int(rng.integers(1, 4))
    g = int(rng.choice([1, 2, 3, 4, 8]))
    return D, dtype, Hkv * g, Hkv


def draw_mask(rng, D):
    causal = bool(rng.integers(0, 2))
    left = int(rng.integers(0, 300)) if rng.random() < 0.3 else -1
    right = int(rng.integers(0, 300)) if rng.random() < 0.3 else -1
    u = rng.random()
    scale = 1.0 / math.sqrt(D) if u < 0.5 else (float(rng.uniform(0.02, 0.3)) if u < 0.8
                                                 else -float(rng.uniform(0.02, 0.2)))
    return causal, left, right, scale


def sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("i", range(128))
def test_random_forward(i):
    rng = np.random.default_rng(7000 + i)
    D, dtype, Hq, Hkv = draw_common(rng)
    B, Nq, Nk = int(rng.integers(1, 3)), int(rng.integers(1, 700)), int(rng.integers(1, 700))
    causal, left, right, scale = draw_mask(rng, D)
    print(f"mfa_fwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} D={D} {dtype} causal={causal} "
          f"win=({left},{right}) scale={scale:.4f}", flush=True)
    x = A.dense_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, 7100 + i)
    q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
    O, L = ea.mfa_fwd(q, k, v, scale=scale, causal=causal, win_left=left, win_right=right)
    sync()
    qf, kf, vf = (oracle.widen(t, dtype) for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention(qf, kf, vf, scale, causal, left, right)
    Oa, _ = oracle.attention(qf, kf, np.abs(vf), scale, causal, left, right)
    assert_close_o(to_f64(O, dtype), Or, dtype, "O", ref_pabs=Oa)
    assert_close_lse(L.cpu().numpy(), Lr, "LSE")


@pytest.mark.parametrize("i", range(64))
def test_random_backward(i):
    rng = np.random.default_rng(7200 + i)
    D, dtype, Hq, Hkv = draw_common(rng)
    B, Nq, Nk = int(rng.integers(1, 3)), int(rng.integers(1, 400)), int(rng.integers(1, 400))
    causal, left, right, scale = draw_mask(rng, D)
    print(f"mfa_fwd + mfa_bwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} D={D} {dtype} "
          f"causal={causal} win=({left},{right}) scale={scale:.4f}", flush=True)
    x = A.dense_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, 7300 + i)
    dob = A.grad_inputs(B, Hq, Nq, D, dtype, 7400 + i)
    q, k, v, do = (to_dev(t, dtype) for t in (x.q, x.k, x.v, dob))
    O, L = ea.mfa_fwd(q, k, v, scale=scale, causal=causal, win_left=left, win_right=right)
    dq, dk, dv = ea.mfa_bwd(q, k, v, O, do, L, scale=scale, causal=causal, win_left=left,
                            win_right=right)
    sync()
    qf, kf, vf, dof = (oracle.widen(t, dtype) for t in (x.q, x.k, x.v, dob))
    refs = oracle.attention_backward(qf, kf, vf, dof, scale, causal, left, right)
    assert_close_grads(("dQ", "dK", "dV"), [to_f64(t, dtype) for t in (dq, dk, dv)], refs, dtype)


@pytest.mark.parametrize("i", range(48))
def test_random_varlen(i):
    rng = np.random.default_rng(7500 + i)
    D, dtype, Hq, Hkv = draw_common(rng)
    B = int(rng.integers(1, 6))
    lq = rng.integers(0, 500, size=B)
    # keys: as many as the queries (self-attention packing) or a longer prefix (chunked)
    lk = lq + (rng.integers(0, 400, size=B) if rng.random() < 0.5 else 0)
    causal, left, right, scale = draw_mask(rng, D)
    print(f"mfa_fwd_varlen Hq={Hq} Hkv={Hkv} D={D} {dtype} lq={lq.tolist()} lk={lk.tolist()} "
          f"causal={causal} win=({left},{right}) scale={scale:.4f}", flush=True)
    x = A.varlen_inputs(Hq, Hkv, D, dtype, 7600 + i, seqlens_q=lq, seqlens_k=lk)
    if x.q.shape[0] == 0 or x.k.shape[0] == 0:
        pytest.skip("drew no tokens")
    q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
    O, L = ea.mfa_fwd_varlen(q, k, v, dev_i32(x.cu_seqlens_q), dev_i32(x.cu_seqlens_k),
                             int(max(1, lq.max())), int(max(1, lk.max())), scale=scale,
                             causal=causal, win_left=left, win_right=right)
    sync()
    qf, kf, vf = (oracle.widen(t, dtype) for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention_varlen(qf, kf, vf, x.cu_seqlens_q, x.cu_seqlens_k, scale, causal,
                                     left, right)
    Oa, _ = oracle.attention_varlen(qf, kf, np.abs(vf), x.cu_seqlens_q, x.cu_seqlens_k, scale, causal,
                                    left, right)
    assert_close_o(to_f64(O, dtype), Or, dtype, "varlen O", ref_pabs=Oa)
    assert_close_lse(L.cpu().numpy(), Lr, "varlen LSE")


@pytest.mark.parametrize("i", range(32))
def test_random_paged_prefill(i):
    rng = np.random.default_rng(7700 + i)
    D, dtype, Hq, Hkv = draw_common(rng)
    B = int(rng.integers(1, 5))
    lq = rng.integers(1, 300, size=B)
    ctx = rng.integers(0, 1500, size=B)
    causal, left, right, scale = draw_mask(rng, D)
    causal = True if rng.random() < 0.7 else causal
    print(f"mfa_fwd_varlen_paged Hq={Hq} Hkv={Hkv} D={D} {dtype} lq={lq.tolist()} "
          f"ctx={ctx.tolist()} causal={causal} win=({left},{right}) scale={scale:.4f}", flush=True)
    p = A.paged_varlen_inputs(Hq, Hkv, D, dtype, 7800 + i, seqlens_q=lq, ctx_lens=ctx,
                              extra_pages=int(rng.integers(0, 4)))
    O, L = ea.mfa_fwd_varlen_paged(to_dev(p.q, dtype), to_dev(p.k_pages, dtype), to_dev(p.v_pages, dtype),
                                   dev_i32(p.block_table), dev_i32(p.seq_lens_k),
                                   dev_i32(p.cu_seqlens_q), int(lq.max()), int(p.seq_lens_k.max()),
                                   scale=scale, causal=causal, win_left=left, win_right=right)
    sync()
    qf, kf, vf = (oracle.widen(t, dtype) for t in (p.q, p.k_pages, p.v_pages))
    Or, Lr = oracle.attention_varlen_paged(qf, kf, vf, p.block_table, p.seq_lens_k, p.cu_seqlens_q,
                                           scale, p.page_size, causal, left, right)
    Oa, _ = oracle.attention_varlen_paged(qf, kf, np.abs(vf), p.block_table, p.seq_lens_k,
                                          p.cu_seqlens_q, scale, p.page_size, causal, left, right)
    assert_close_o(to_f64(O, dtype), Or, dtype, "paged prefill O", ref_pabs=Oa)
    assert_close_lse(L.cpu().numpy(), Lr, "paged prefill LSE")


@pytest.mark.parametrize("i", range(48))
def test_random_decode(i):
    rng = np.random.default_rng(7900 + i)
    D, dtype, Hq, Hkv = draw_common(rng)
    B = int(rng.integers(1, 7))
    hi = int(rng.choice([50, 700, 3000]))
    splits = int(rng.choice([0, 0, 1, 3, 7]))
    scale = 1.0 / math.sqrt(D) if rng.random() < 0.7 else float(rng.uniform(0.02, 0.3))
    p = A.paged_inputs(B, Hq, Hkv, D, dtype, 8000 + i, len_lo=0, len_hi=hi,
                       extra_pages=int(rng.integers(0, 4)))
    print(f"mfa_decode_paged B={B} Hq={Hq} Hkv={Hkv} D={D} {dtype} lens={p.seq_lens.tolist()} "
          f"splits={splits} scale={scale:.4f}", flush=True)
    O, L = ea.mfa_decode_paged(to_dev(p.q, dtype), to_dev(p.k_pages, dtype), to_dev(p.v_pages, dtype),
                               dev_i32(p.block_table), dev_i32(p.seq_lens), scale=scale,
                               num_splits=splits)
    sync()
    qf, kf, vf = (oracle.widen(t, dtype) for t in (p.q, p.k_pages, p.v_pages))
    Or, Lr = oracle.decode_paged(qf, kf, vf, p.block_table, p.seq_lens, scale, p.page_size)
    Oa, _ = oracle.decode_paged(qf, kf, np.abs(vf), p.block_table, p.seq_lens, scale, p.page_size)
    assert_close_o(to_f64(O, dtype), Or, dtype, "decode O", ref_pabs=Oa)
    assert_close_lse(L.cpu().numpy(), Lr, "decode LSE")


@pytest.mark.parametrize("i", range(32))
def test_random_multi_decode(i):
    rng = np.random.default_rng(8100 + i)
    D, dtype, Hq, Hkv = draw_common(rng)
    B, Nq = int(rng.integers(1, 6)), int(rng.integers(1, 5))
    hi = int(rng.choice([60, 800, 2500]))
    splits = int(rng.choice([0, 0, 1, 2, 5]))
    scale = 1.0 / math.sqrt(D)
    p = A.paged_multi_inputs(B, Nq, Hq, Hkv, D, dtype, 8200 + i, len_lo=0, len_hi=hi,
                             extra_pages=int(rng.integers(0, 3)))
    print(f"mfa_decode_paged_multi B={B} Nq={Nq} Hq={Hq} Hkv={Hkv} D={D} {dtype} "
          f"lens={p.seq_lens.tolist()} splits={splits}", flush=True)
    O, L = ea.mfa_decode_paged_multi(to_dev(p.q, dtype), to_dev(p.k_pages, dtype),
                                     to_dev(p.v_pages, dtype), dev_i32(p.block_table),
                                     dev_i32(p.seq_lens), scale=scale, num_splits=splits)
    sync()
    qf, kf, vf = (oracle.widen(t, dtype) for t in (p.q, p.k_pages, p.v_pages))
    Or, Lr = oracle.decode_paged_multi(qf, kf, vf, p.block_table, p.seq_lens, scale, p.page_size)
    Oa, _ = oracle.decode_paged_multi(qf, kf, np.abs(vf), p.block_table, p.seq_lens, scale, p.page_size)
    assert_close_o(to_f64(O, dtype), Or, dtype, "multi decode O", ref_pabs=Oa)
    assert_close_lse(L.cpu().numpy(), Lr, "multi decode LSE")


@pytest.mark.parametrize("i", range(48))
def test_random_ext(i):
    rng = np.random.default_rng(8300 + i)
    D, dtype, Hq, Hkv = draw_common(rng)
    B, Nq, Nk = int(rng.integers(1, 3)), int(rng.integers(1, 600)), int(rng.integers(1, 600))
    causal, left, right, scale = draw_mask(rng, D)
    softcap = float(rng.choice([0.0, 5.0, 30.0]))
    slopes = 2.0 ** (-8.0 * (np.arange(Hq) + 1) / Hq) if rng.random() < 0.4 else None
    bias = None
    kind = int(rng.integers(0, 4))
    if kind == 1:
        bias = rng.standard_normal(Nk)
    elif kind == 2:
        bias = rng.standard_normal((Hq, Nk))
    elif kind == 3:
        bias = rng.standard_normal((B, Hq, Nk))
    bm, bq, bk = None, 0, 0
    if rng.random() < 0.5:
        bq, bk = int(rng.choice([32, 64, 128])), int(rng.choice([32, 64, 128]))
        nqb, nkb = -(-Nq // bq), -(-Nk // bk)
        bm = (rng.random((B, Hq if rng.random() < 0.5 else 1, nqb, nkb)) < 0.6).astype(np.uint8)
    print(f"mfa_fwd_ext B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} D={D} {dtype} causal={causal} "
          f"win=({left},{right}) scale={scale:.4f} softcap={softcap} alibi={slopes is not None} "
          f"bias={kind} mask={None if bm is None else bm.shape} blocks=({bq},{bk})", flush=True)
    x = A.dense_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, 8400 + i)
    q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
    O, L = ea.mfa_fwd_ext(q, k, v, scale=scale, causal=causal, win_left=left, win_right=right,
                          softcap=softcap, alibi_slopes=None if slopes is None else dev_f32(slopes),
                          bias=None if bias is None else dev_f32(bias),
                          block_mask=None if bm is None else dev_u8(bm), block_q=bq, block_k=bk)
    sync()
    qf, kf, vf = (oracle.widen(t, dtype) for t in (x.q, x.k, x.v))
    bias_full = None if bias is None else np.broadcast_to(bias, (B, Hq, Nk))
    bm_full = None if bm is None else np.broadcast_to(bm, (B, Hq) + bm.shape[-2:])
    kw = dict(softcap=softcap, alibi_slopes=slopes, bias=bias_full, block_mask=bm_full, block_q=bq,
              block_k=bk)
    Or, Lr = oracle.attention_ext(qf, kf, vf, scale, causal, left, right, **kw)
    Oa, _ = oracle.attention_ext(qf, kf, np.abs(vf), scale, causal, left, right, **kw)
    assert_close_o(to_f64(O, dtype), Or, dtype, "ext O", ref_pabs=Oa)
    assert_close_lse(L.cpu().numpy(), Lr, "ext LSE")


@pytest.mark.parametrize("i", range(8))
def test_random_forward_many_heads(i):
    # grids of more than two query tiles per CU with an even group size take one 8-wave
    # workgroup per pair of query heads sharing a KV head; sampled rows against the oracle
    rng = np.random.default_rng(8500 + i)
    D, dtype, _, _ = draw_common(rng)
    Hkv = int(rng.choice([32, 64]))
    Hq = Hkv * int(rng.choice([2, 4]))
    B, Nq = 1, int(rng.integers(1100, 1600))      # >= 9 query tiles x >= 64 heads > 2 x 256
    Nk = Nq if rng.random() < 0.6 else int(rng.integers(300, 2000))
    causal, left, right, scale = draw_mask(rng, D)
    print(f"mfa_fwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} D={D} {dtype} causal={causal} "
          f"win=({left},{right}) scale={scale:.4f}", flush=True)
    x = A.dense_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, 8600 + i)
    q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
    O, L = ea.mfa_fwd(q, k, v, scale=scale, causal=causal, win_left=left, win_right=right)
    sync()
    # (an even group size: one 8-wave workgroup per pair of query heads)
    assert "groups=2" in ea.mfa_last_dispatch()["kernel"] and ",head-pairs" in ea.mfa_last_dispatch()["kernel"]
    rows = sorted({(0, int(h), int(r)) for h, r in zip(rng.integers(0, Hq, 200), rng.integers(0, Nq, 200))}
                  | {(0, 0, 0), (0, Hq - 1, Nq - 1)})
    qf, kf, vf = (oracle.widen(t, dtype) for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention(qf, kf, vf, scale, causal, left, right, rows=rows)
    Oa, _ = oracle.attention(qf, kf, np.abs(vf), scale, causal, left, right, rows=rows)
    idx = tuple(np.array(rows).T)
    assert_close_o(to_f64(O, dtype)[idx], Or, dtype, "O", ref_pabs=Oa)
    assert_close_lse(L.cpu().numpy()[idx], Lr, "LSE")


# Workgroup orders that pin KV heads to XCDs (Hkv a multiple of 8): sequence-major for
# packed and paged sequences, head-major for dense layouts with one 4-wave group.
def draw_xcd_heads(rng, gs=(1, 2, 3)):
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    Hkv = int(rng.choice([8, 16]))
    return D, dtype, Hkv * int(rng.choice(gs)), Hkv


@pytest.mark.parametrize("i", range(16))
def test_random_varlen_seq_major(i):
    rng = np.random.default_rng(9100 + i)
    D, dtype, Hq, Hkv = draw_xcd_heads(rng)
    B = int(rng.integers(1, 25))
    lq = rng.integers(0, 300, size=B)
    lk = lq + (rng.integers(0, 300, size=B) if rng.random() < 0.5 else 0)
    causal, left, right, scale = draw_mask(rng, D)
    print(f"mfa_fwd_varlen (seq-major) B={B} Hq={Hq} Hkv={Hkv} D={D} {dtype} lq={lq.tolist()} "
          f"lk={lk.tolist()} causal={causal} win=({left},{right}) scale={scale:.4f}", flush=True)
    x = A.varlen_inputs(Hq, Hkv, D, dtype, 9200 + i, seqlens_q=lq, seqlens_k=lk)
    if x.q.shape[0] == 0 or x.k.shape[0] == 0:
        pytest.skip("drew no tokens")
    q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
    O, L = ea.mfa_fwd_varlen(q, k, v, dev_i32(x.cu_seqlens_q), dev_i32(x.cu_seqlens_k),
                             int(max(1, lq.max())), int(max(1, lk.max())), scale=scale,
                             causal=causal, win_left=left, win_right=right)
    sync()
    assert ",seq-major" in ea.mfa_last_dispatch()["kernel"], ea.mfa_last_dispatch()["kernel"]
    qf, kf, vf = (oracle.widen(t, dtype) for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention_varlen(qf, kf, vf, x.cu_seqlens_q, x.cu_seqlens_k, scale, causal,
                                     left, right)
    Oa, _ = oracle.attention_varlen(qf, kf, np.abs(vf), x.cu_seqlens_q, x.cu_seqlens_k, scale, causal,
                                    left, right)
    assert_close_o(to_f64(O, dtype), Or, dtype, "varlen O", ref_pabs=Oa)
    assert_close_lse(L.cpu().numpy(), Lr, "varlen LSE")


@pytest.mark.parametrize("i", range(12))
def test_random_paged_seq_major(i):
    rng = np.random.default_rng(9300 + i)
    D, dtype, Hq, Hkv = draw_xcd_heads(rng)
    B = int(rng.integers(1, 17))
    lq = rng.integers(1, 200, size=B)
    ctx = rng.integers(0, 800, size=B)
    causal, left, right, scale = draw_mask(rng, D)
    causal = True if rng.random() < 0.7 else causal
    print(f"mfa_fwd_varlen_paged (seq-major) B={B} Hq={Hq} Hkv={Hkv} D={D} {dtype} "
          f"lq={lq.tolist()} ctx={ctx.tolist()} causal={causal} win=({left},{right}) "
          f"scale={scale:.4f}", flush=True)
    p = A.paged_varlen_inputs(Hq, Hkv, D, dtype, 9400 + i, seqlens_q=lq, ctx_lens=ctx,
                              extra_pages=int(rng.integers(0, 4)))
    O, L = ea.mfa_fwd_varlen_paged(to_dev(p.q, dtype), to_dev(p.k_pages, dtype), to_dev(p.v_pages, dtype),
                                   dev_i32(p.block_table), dev_i32(p.seq_lens_k),
                                   dev_i32(p.cu_seqlens_q), int(lq.max()), int(p.seq_lens_k.max()),
                                   scale=scale, causal=causal, win_left=left, win_right=right)
    sync()
    assert ",seq-major" in ea.mfa_last_dispatch()["kernel"], ea.mfa_last_dispatch()["kernel"]
    qf, kf, vf = (oracle.widen(t, dtype) for t in (p.q, p.k_pages, p.v_pages))
    Or, Lr = oracle.attention_varlen_paged(qf, kf, vf, p.block_table, p.seq_lens_k, p.cu_seqlens_q,
                                           scale, p.page_size, causal, left, right)
    Oa, _ = oracle.attention_varlen_paged(qf, kf, np.abs(vf), p.block_table, p.seq_lens_k,
                                          p.cu_seqlens_q, scale, p.page_size, causal, left, right)
    assert_close_o(to_f64(O, dtype), Or, dtype, "paged prefill O", ref_pabs=Oa)
    assert_close_lse(L.cpu().numpy(), Lr, "paged prefill LSE")


@pytest.mark.parametrize("i", range(12))
def test_random_head_major(i):
    # dense layouts with one 4-wave group (odd group sizes, more than two query tiles per
    # CU), with score modifiers and a block mask on every other draw; four heads checked
    rng = np.random.default_rng(9500 + i)
    D, dtype, Hq, Hkv = draw_xcd_heads(rng, gs=(1, 3))
    B = int(rng.integers(1, 3))
    tiles = 512 // (B * Hq) + 1
    Nq = int(rng.integers(128 * tiles - 100, 128 * tiles + 300))
    Nk = Nq if rng.random() < 0.6 else int(rng.integers(max(1, Nq // 2), Nq + 400))
    causal, left, right, scale = draw_mask(rng, D)
    ext = i % 2 == 1
    print(f"{'mfa_fwd_ext' if ext else 'mfa_fwd'} (head-major) B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} "
          f"Nk={Nk} D={D} {dtype} causal={causal} win=({left},{right}) scale={scale:.4f}", flush=True)
    x = A.dense_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, 9600 + i)
    q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
    kw = {}
    if ext:
        bq, bk = 64, 64
        bm = (rng.random((B, Hq, math.ceil(Nq / bq), math.ceil(Nk / bk))) < 0.5).astype(np.uint8)
        kw = dict(softcap=float(rng.uniform(5, 40)), block_mask=bm, block_q=bq, block_k=bk)
        O, L = ea.mfa_fwd_ext(q, k, v, scale=scale, causal=causal, win_left=left, win_right=right,
                              softcap=kw["softcap"], block_mask=dev_u8(bm), block_q=bq, block_k=bk)
    else:
        O, L = ea.mfa_fwd(q, k, v, scale=scale, causal=causal, win_left=left, win_right=right)
    sync()
    assert ",head-major" in ea.mfa_last_dispatch()["kernel"], ea.mfa_last_dispatch()["kernel"]
    g = Hq // Hkv
    heads = sorted({0, Hq - 1} | {int(h) for h in rng.integers(0, Hq, 2)})
    for b in range(B):
        for h in heads:
            qf = oracle.widen(x.q[b:b + 1, h:h + 1], dtype)
            kf, vf = (oracle.widen(t[b:b + 1, h // g:h // g + 1], dtype) for t in (x.k, x.v))
            if ext:
                bmh = kw["block_mask"][b:b + 1, h:h + 1]
                Or, Lr = oracle.attention_ext(qf, kf, vf, scale, causal, left, right,
                                              softcap=kw["softcap"], block_mask=bmh, block_q=64, block_k=64)
                Oa, _ = oracle.attention_ext(qf, kf, np.abs(vf), scale, causal, left, right,
                                             softcap=kw["softcap"], block_mask=bmh, block_q=64, block_k=64)
            else:
                Or, Lr = oracle.attention(qf, kf, vf, scale, causal, left, right)
                Oa, _ = oracle.attention(qf, kf, np.abs(vf), scale, causal, left, right)
            assert_close_o(to_f64(O[b:b + 1, h:h + 1], dtype), Or, dtype, f"O b={b} h={h}", ref_pabs=Oa)
            assert_close_lse(L[b:b + 1, h:h + 1].cpu().numpy(), Lr, f"LSE b={b} h={h}")
