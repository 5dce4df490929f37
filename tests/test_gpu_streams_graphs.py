"""The library launches on the stream it is given (the binding passes torch's current
stream) and issues nothing but kernel launches (no allocation, memset or synchronisation),
so its calls can run on any stream and be captured in a HIP graph.  Results are
deterministic, so every comparison here is bitwise."""
import math

import numpy as np
import pytest

import attn_inputs as A

pytestmark = pytest.mark.gpu

ea = pytest.importorskip("exact_attention_amd")


def to_dev(bits, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16)


def same(a, b):
    import torch
    if a.dtype in (torch.float16, torch.bfloat16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


class Problem:
    """Forward + backward inputs (dense causal, GQA) and a paged decode batch."""

    def __init__(self, seed):
        import torch
        x = A.dense_inputs(2, 4, 2, 300, 300, 128, "bf16", seed)
        self.q, self.k, self.v = (to_dev(t, "bf16") for t in (x.q, x.k, x.v))
        self.do = to_dev(A.grad_inputs(2, 4, 300, 128, "bf16", seed + 1), "bf16")
        p = A.paged_inputs(3, 8, 2, 128, "bf16", seed + 2, len_lo=1, len_hi=900, extra_pages=2)
        self.dq = to_dev(p.q, "bf16")
        self.kp, self.vp = to_dev(p.k_pages, "bf16"), to_dev(p.v_pages, "bf16")
        self.bt = torch.from_numpy(p.block_table).cuda()
        self.sl = torch.from_numpy(p.seq_lens).cuda()

    def refill(self, seed):
        """New seeded N(0, 1) values in the same buffers (the block table and sequence
        lengths stay; the kernels never read past a sequence's length)."""
        import torch
        gen = torch.Generator().manual_seed(seed)
        for name in ("q", "k", "v", "do", "dq", "kp", "vp"):
            t = getattr(self, name)
            t.copy_(torch.randn(t.shape, generator=gen).to(t.dtype))


def run_all(p, outs=None):
    """mfa_fwd, mfa_bwd and mfa_decode_paged on p; into preallocated outs if given."""
    import torch
    scale = 1 / math.sqrt(128)
    if outs is None:
        outs = {
            "o": torch.empty_like(p.q),
            "lse": torch.empty(p.q.shape[:3], dtype=torch.float32, device="cuda"),
            "gq": torch.empty_like(p.q), "gk": torch.empty_like(p.k), "gv": torch.empty_like(p.v),
            "bws": torch.empty(int(ea.lib().mfa_bwd_workspace_bytes(2, 4, 300)), dtype=torch.uint8,
                               device="cuda"),
            "do_": torch.empty_like(p.dq),
            "dlse": torch.empty(p.dq.shape[:2], dtype=torch.float32, device="cuda"),
            "dws": torch.empty(ea.mfa_decode_workspace_bytes(3, 8, 128, 16, p.bt.shape[1], 0),
                               dtype=torch.uint8, device="cuda"),
        }
    ea.mfa_fwd(p.q, p.k, p.v, scale=scale, causal=True, out=outs["o"], lse=outs["lse"])
    ea.mfa_bwd(p.q, p.k, p.v, outs["o"], p.do, outs["lse"], scale=scale, causal=True,
               dq=outs["gq"], dk=outs["gk"], dv=outs["gv"], workspace=outs["bws"])
    ea.mfa_decode_paged(p.dq, p.kp, p.vp, p.bt, p.sl, scale=scale, out=outs["do_"],
                        lse=outs["dlse"], workspace=outs["dws"])
    return outs


def test_side_stream_matches_default_stream():
    import torch
    p = Problem(31)
    ref = run_all(p)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = run_all(p)
    s.synchronize()
    for key in ref:
        if key in ("bws", "dws"):
            continue
        assert same(ref[key], got[key]), key


def test_graph_capture_replays_match_eager():
    import torch
    p = Problem(41)
    outs = run_all(p)                     # buffers the graph writes into
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):            # warm-up outside the capture
        run_all(p, outs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all(p, outs)
    for r in range(3):
        # new data in the captured input buffers, then a replay and an eager run on it,
        # with eager work and synchronisation between the replays
        p.refill(50 + r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {key: t.clone() for key, t in outs.items() if key not in ("bws", "dws")}
        ref = run_all(p)
        torch.cuda.synchronize()
        for key, t in got.items():
            assert same(t, ref[key]), (r, key)


def test_repeated_calls_bitwise():
    # 30 back-to-back calls of the chained forward (an even number of query tiles on a
    # small grid) and of the backward give the first call's result bit for bit
    import torch
    x = A.dense_inputs(2, 4, 2, 512, 512, 128, "bf16", 61)
    q, k, v = (to_dev(t, "bf16") for t in (x.q, x.k, x.v))
    do = to_dev(A.grad_inputs(2, 4, 512, 128, "bf16", 62), "bf16")
    scale = 1 / math.sqrt(128)
    O0, L0 = ea.mfa_fwd(q, k, v, scale=scale, causal=True)
    assert ",chained" in ea.mfa_last_dispatch()["kernel"]
    g0 = ea.mfa_bwd(q, k, v, O0, do, L0, scale=scale, causal=True)
    torch.cuda.synchronize()
    for _ in range(30):
        O, L = ea.mfa_fwd(q, k, v, scale=scale, causal=True)
        g = ea.mfa_bwd(q, k, v, O, do, L, scale=scale, causal=True)
        assert same(O, O0) and same(L, L0)
        assert all(same(a, b) for a, b in zip(g, g0))
