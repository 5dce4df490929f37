"""Guard bands around every output and workspace (race and out-of-bounds detection).

The MXFlashAttn 1.5.0 page traces a split-KV bug to lanes of invalid query heads writing
into the next split's scratch slot.  Writes outside a tensor are the same class of fault:
here each output (and workspace) sits inside a larger buffer whose extra words, before and
after it, are filled with a canary bit pattern; after the call the canaries must be intact.
Inside the outputs, the rows the library documents as not written (tokens outside every
packed sequence) must keep the canary too.  The cases put partial query tiles, partial key
tiles and short last pages at the ends of the buffers, and every result is also checked
against the oracle.
"""
import math

import numpy as np
import pytest

import attn_inputs as A
import oracle
from gpu_util import assert_close_grads, assert_close_lse, assert_close_o, to_dev, to_f64

pytestmark = pytest.mark.gpu

ea = pytest.importorskip("exact_attention_amd")

GUARD = 1024          # canary words on each side (a multiple of 8: alignment is kept)
CANARY16 = 0x7E5A     # a NaN pattern of both 16-bit types
CANARY32 = 0x7FC05A5A  # a float32 NaN pattern


class Guarded:
    """A device tensor of `shape` placed GUARD words into a canary-filled buffer."""

    def __init__(self, shape, dtype):
        import torch
        self.n = int(np.prod(shape))
        self.bits = torch.int16 if dtype in (torch.float16, torch.bfloat16) else torch.int32
        self.canary = CANARY16 if self.bits == torch.int16 else CANARY32
        self.buf = torch.full((self.n + 2 * GUARD,), self.canary, dtype=self.bits, device="cuda")
        self.t = self.buf[GUARD:GUARD + self.n].view(dtype).view(shape)

    def check(self, what):
        raw = self.buf.cpu().numpy()
        assert np.all(raw[:GUARD] == self.canary), f"{what}: write before the buffer"
        assert np.all(raw[GUARD + self.n:] == self.canary), f"{what}: write past the buffer"

    def untouched(self):
        """Boolean array (shape of the tensor): elements still holding the canary."""
        return (self.buf[GUARD:GUARD + self.n].cpu().numpy() == self.canary).reshape(self.t.shape)


def guarded_bytes(nbytes):
    import torch
    return Guarded((-(-nbytes // 4),), torch.int32)


DENSE = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, left, right
    (2, 4, 2, 259, 333, 128, "f16", True, -1, -1),      # partial query and key tiles
    (1, 2, 2, 500, 500, 64, "bf16", True, 37, 0),       # window, partial tiles, D = 64
    (1, 240, 240, 259, 259, 128, "bf16", True, -1, -1),  # many heads: one wave group
    (1, 4, 4, 512, 512, 128, "f16", True, -1, -1),      # chained complementary tiles
    (1, 2, 1, 1, 777, 128, "f16", True, -1, -1),        # one query row
    (1, 128, 32, 520, 520, 64, "bf16", True, -1, -1),   # head pairs, D = 64, partial tile
    (1, 128, 64, 650, 600, 128, "f16", True, -1, -1),   # head pairs, Nk < Nq
]


@pytest.mark.parametrize("case", DENSE, ids=[str(i) for i in range(len(DENSE))])
def test_forward_guards(case):
    import torch
    B, Hq, Hkv, Nq, Nk, D, dt, causal, left, right = case
    x = A.dense_inputs(B, Hq, Hkv, Nq, Nk, D, dt, 3000 + Nq + Hq)
    q, k, v = (to_dev(t, dt) for t in (x.q, x.k, x.v))
    tdt = q.dtype
    out, lse = Guarded((B, Hq, Nq, D), tdt), Guarded((B, Hq, Nq), torch.float32)
    print(f"guarded mfa_fwd {case}", flush=True)
    ea.mfa_fwd(q, k, v, scale=1 / math.sqrt(D), causal=causal, win_left=left, win_right=right,
               out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check("O")
    lse.check("LSE")
    qf, kf, vf = (oracle.widen(t, dt) for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention(qf, kf, vf, 1 / math.sqrt(D), causal, left, right)
    assert_close_o(to_f64(out.t, dt), Or, dt, "O")
    assert_close_lse(lse.t.cpu().numpy(), Lr, "LSE")


def test_backward_guards():
    import torch
    B, Hq, Hkv, Nq, Nk, D, dt = 1, 4, 2, 259, 333, 128, "bf16"
    x = A.dense_inputs(B, Hq, Hkv, Nq, Nk, D, dt, 3101)
    q, k, v = (to_dev(t, dt) for t in (x.q, x.k, x.v))
    dob = A.grad_inputs(B, Hq, Nq, D, dt, 3102)
    do = to_dev(dob, dt)
    O, L = ea.mfa_fwd(q, k, v, scale=0.09, causal=True)
    dq, dk, dv = (Guarded(t.shape, t.dtype) for t in (q, k, v))
    need = int(ea.lib().mfa_bwd_workspace_bytes(B, Hq, Nq))
    ws = guarded_bytes(need)
    print("guarded mfa_bwd", flush=True)
    ea.mfa_bwd(q, k, v, O, do, L, scale=0.09, causal=True, dq=dq.t, dk=dk.t, dv=dv.t,
               workspace=ws.t)
    torch.cuda.synchronize()
    for g, n in ((dq, "dQ"), (dk, "dK"), (dv, "dV"), (ws, "workspace")):
        g.check(n)
    refs = oracle.attention_backward(*(oracle.widen(t, dt) for t in (x.q, x.k, x.v, dob)), 0.09,
                                     True)
    assert_close_grads(["dQ", "dK", "dV"], [to_f64(g.t, dt) for g in (dq, dk, dv)], refs, dt)


def test_varlen_guards_and_padding():
    # tokens after the last sequence belong to none: their O rows and LSE columns stay
    # untouched, as does everything outside the buffers
    import torch
    x = A.varlen_inputs(4, 2, 128, "f16", 3201, seqlens_q=[70, 259, 1, 130],
                        seqlens_k=[70, 300, 1, 400], pad_q=37, pad_k=11)
    T = int(x.cu_seqlens_q[-1])
    q, k, v = (to_dev(t, "f16") for t in (x.q, x.k, x.v))
    cq = torch.from_numpy(x.cu_seqlens_q).to("cuda")
    ck = torch.from_numpy(x.cu_seqlens_k).to("cuda")
    out, lse = Guarded(q.shape, q.dtype), Guarded((q.shape[1], q.shape[0]), torch.float32)
    print("guarded mfa_fwd_varlen", flush=True)
    ea.mfa_fwd_varlen(q, k, v, cq, ck, 259, 400, scale=0.1, causal=True, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check("O")
    lse.check("LSE")
    assert np.all(out.untouched()[T:]) and np.all(lse.untouched()[:, T:]), "padding rows written"
    assert not np.any(out.untouched()[:T]) and not np.any(lse.untouched()[:, :T])
    qf, kf, vf = (oracle.widen(t, "f16") for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention_varlen(qf, kf, vf, x.cu_seqlens_q, x.cu_seqlens_k, 0.1, True)
    assert_close_o(to_f64(out.t, "f16")[:T], Or[:T], "f16", "packed O")
    assert_close_lse(lse.t.cpu().numpy()[:, :T], Lr[:, :T], "packed LSE")


def test_varlen_paged_guards():
    import torch
    p = A.paged_varlen_inputs(8, 2, 128, "bf16", 3301, seqlens_q=[1, 259, 70],
                              ctx_lens=[15, 300, 1000])
    T = int(p.cu_seqlens_q[-1])
    q = to_dev(p.q, "bf16")
    kp, vp = to_dev(p.k_pages, "bf16"), to_dev(p.v_pages, "bf16")
    bt = torch.from_numpy(p.block_table).to("cuda")
    sl = torch.from_numpy(p.seq_lens_k).to("cuda")
    cq = torch.from_numpy(p.cu_seqlens_q).to("cuda")
    lq = np.diff(p.cu_seqlens_q)
    out, lse = Guarded(q.shape, q.dtype), Guarded((q.shape[1], q.shape[0]), torch.float32)
    print("guarded mfa_fwd_varlen_paged", flush=True)
    ea.mfa_fwd_varlen_paged(q, kp, vp, bt, sl, cq, int(lq.max()), int(p.seq_lens_k.max()),
                            scale=0.09, causal=True, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check("O")
    lse.check("LSE")
    qf, kf, vf = (oracle.widen(t, "bf16") for t in (p.q, p.k_pages, p.v_pages))
    Or, Lr = oracle.attention_varlen_paged(qf, kf, vf, p.block_table, p.seq_lens_k,
                                           p.cu_seqlens_q, 0.09, 16, True)
    assert_close_o(to_f64(out.t, "bf16")[:T], Or[:T], "bf16", "paged prefill O")
    assert_close_lse(lse.t.cpu().numpy()[:, :T], Lr[:, :T], "paged prefill LSE")


@pytest.mark.parametrize("nq", [1, 3])
def test_decode_guards(nq):
    import torch
    B, Hq, Hkv, D = 5, 16, 4, 128
    seq_lens = [1, 15, 17, 513, 2000]
    if nq == 1:
        p = A.paged_inputs(B, Hq, Hkv, D, "bf16", 3401, len_lo=1, len_hi=2000, seq_lens=seq_lens,
                           extra_pages=2)
        oshape, lshape = (B, Hq, D), (B, Hq)
    else:
        p = A.paged_multi_inputs(B, nq, Hq, Hkv, D, "bf16", 3402, len_lo=1, len_hi=2000,
                                 seq_lens=seq_lens, extra_pages=2)
        oshape, lshape = (B, nq, Hq, D), (B, nq, Hq)
    q = to_dev(p.q, "bf16")
    kp, vp = to_dev(p.k_pages, "bf16"), to_dev(p.v_pages, "bf16")
    bt = torch.from_numpy(p.block_table).to("cuda")
    sl = torch.from_numpy(p.seq_lens).to("cuda")
    max_pages = p.block_table.shape[1]
    if nq == 1:
        need = ea.mfa_decode_workspace_bytes(B, Hq, D, 16, max_pages, 0)
    else:
        need = ea.mfa_decode_multi_workspace_bytes(B, nq, Hq, D, 16, max_pages, 0)
    out, lse, ws = Guarded(oshape, q.dtype), Guarded(lshape, torch.float32), guarded_bytes(need)
    print(f"guarded decode nq={nq}", flush=True)
    if nq == 1:
        ea.mfa_decode_paged(q, kp, vp, bt, sl, scale=0.08, out=out.t, lse=lse.t, workspace=ws.t)
    else:
        ea.mfa_decode_paged_multi(q, kp, vp, bt, sl, scale=0.08, out=out.t, lse=lse.t,
                                  workspace=ws.t)
    torch.cuda.synchronize()
    for g, n in ((out, "O"), (lse, "LSE"), (ws, "workspace")):
        g.check(n)
    args = (oracle.widen(p.q, "bf16"), oracle.widen(p.k_pages, "bf16"),
            oracle.widen(p.v_pages, "bf16"), p.block_table, p.seq_lens, 0.08, 16)
    Or, Lr = oracle.decode_paged(*args) if nq == 1 else oracle.decode_paged_multi(*args)
    assert_close_o(to_f64(out.t, "bf16"), Or, "bf16", "decode O")
    assert_close_lse(lse.t.cpu().numpy(), Lr, "decode LSE")


def test_ext_guards():
    import torch
    B, Hq, Hkv, Nq, Nk, D, dt = 1, 4, 2, 300, 333, 128, "f16"
    x = A.dense_inputs(B, Hq, Hkv, Nq, Nk, D, dt, 3501)
    q, k, v = (to_dev(t, dt) for t in (x.q, x.k, x.v))
    bm = A.block_mask_inputs(B, Hq, Nq, Nk, 64, 64, 0.5, 3502)
    slopes = np.array([0.5, 0.25, 0.125, 0.0625], np.float32)
    out, lse = Guarded(q.shape, q.dtype), Guarded((B, Hq, Nq), torch.float32)
    print("guarded mfa_fwd_ext", flush=True)
    ea.mfa_fwd_ext(q, k, v, scale=0.09, causal=True, softcap=20.0,
                   alibi_slopes=torch.from_numpy(slopes).to("cuda"),
                   block_mask=torch.from_numpy(bm).to("cuda"), block_q=64, block_k=64,
                   out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check("O")
    lse.check("LSE")
    qf, kf, vf = (oracle.widen(t, dt) for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention_ext(qf, kf, vf, 0.09, True, softcap=20.0, alibi_slopes=slopes,
                                  block_mask=bm, block_q=64, block_k=64)
    assert_close_o(to_f64(out.t, dt), Or, dt, "ext O")
    assert_close_lse(lse.t.cpu().numpy(), Lr, "ext LSE")
