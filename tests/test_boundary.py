"""Host side of the C ABI, without a GPU: the library loads and exports every
declared entry point; the tile plan equals the oracle's brute-force visited-tile set;
malformed arguments get their documented status before anything is launched."""
import math
import os
import re
import threading

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mfa.h")

ea = pytest.importorskip("exact_attention_amd")
if not os.path.exists(ea.LIB_PATH):
    pytest.skip("libmfa.so not built", allow_module_level=True)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\**\s+\**(mfa_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 9, names
    L = ea.lib()
    for n in names:
        assert hasattr(L, n), f"libmfa.so does not export {n}"
    assert set(names) == set(ea.EXPORTS), "binding and header disagree"


def test_version_and_status_strings():
    assert ea.mfa_version() >= 100
    for code in range(-13, 1):
        s = ea.mfa_status_string(code)
        assert s and s != "unknown status"
    assert ea.mfa_status_string(5) == "unknown status"


def _plan_vs_oracle(Nq, Nk, D, causal, left, right):
    plan, ranges = ea.mfa_plan_fwd(Nq, Nk, D, ea.MFA_F16, causal, left, right)
    ref = oracle.visited_tiles(Nq, Nk, plan["BM"], plan["BN"], causal, left, right)
    assert len(ranges) == len(ref) == math.ceil(Nq / plan["BM"])
    for t, ((lo, hi), tiles) in enumerate(zip(ranges, ref)):
        assert list(range(lo, hi)) == tiles, (Nq, Nk, D, causal, left, right, t)
    assert plan["visited"] == sum(len(t) for t in ref)
    assert 0 <= plan["edge"] <= plan["visited"]
    return plan


@pytest.mark.parametrize("case", [
    (128, 128, 64, False, -1, -1), (128, 128, 64, True, -1, -1), (4096, 4096, 128, True, -1, -1),
    (8192, 8192, 128, True, 512, 0), (1, 1, 128, True, -1, -1), (1, 5000, 128, True, -1, -1),
    (300, 100, 64, True, -1, -1), (1000, 1000, 128, False, 3, 7), (777, 1234, 128, False, 0, 0),
    (513, 513, 64, True, 0, -1), (200, 4000, 128, False, -1, 0), (4000, 200, 128, False, 50, -1),
])
def test_plan_matches_oracle(case):
    _plan_vs_oracle(*case)


def test_plan_random():
    rng = np.random.default_rng(0)
    for _ in range(60):
        Nq, Nk = (int(x) for x in rng.integers(1, 700, size=2))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        left = int(rng.choice([-1, 0, 1, 17, 130, 1000]))
        right = int(rng.choice([-1, 0, 1, 33, 300]))
        _plan_vs_oracle(Nq, Nk, D, causal, left, right)


def test_plan_headline_counts():
    # causal N=4096 with 128x64 tiles: query tile t visits 2(t+1) tiles -> 1056 of 2048
    plan, _ = ea.mfa_plan_fwd(4096, 4096, 128, ea.MFA_F16, True)
    assert (plan["BM"], plan["BN"]) == (128, 64)
    assert plan["visited"] == 1056 and plan["n_k_tiles"] * plan["n_q_tiles"] == 2048
    # the diagonal of a 128-row tile crosses two 64-key tiles: both are masked
    assert plan["edge"] == 64
    # window (512, 0): query tile t visits key tiles max(0, 2t-8) .. 2t+1 -> 620 in all
    plan, _ = ea.mfa_plan_fwd(8192, 8192, 128, ea.MFA_F16, True, 512, 0)
    assert plan["visited"] == sum(min(2 * t + 2, 10) for t in range(64)) == 620


def test_plan_errors():
    P = ea.mfa_plan
    import ctypes
    p = P()
    L = ea.lib()
    assert L.mfa_plan_fwd(10, 10, 96, 0, 0, -1, -1, ctypes.byref(p), None, 0) == -4
    assert L.mfa_plan_fwd(10, 10, 64, 3, 0, -1, -1, ctypes.byref(p), None, 0) == -5
    assert L.mfa_plan_fwd(0, 10, 64, 0, 0, -1, -1, ctypes.byref(p), None, 0) == -2
    assert L.mfa_plan_fwd(10, 10, 64, 0, 0, -2, -1, ctypes.byref(p), None, 0) == -6
    assert L.mfa_plan_fwd(10, 10, 64, 0, 0, -1, -1, None, None, 0) == -1
    buf = (ctypes.c_int32 * 1)()
    assert L.mfa_plan_fwd(1000, 10, 64, 0, 0, -1, -1, ctypes.byref(p), ctypes.cast(buf, ctypes.c_void_p), 1) == -13


# fake, aligned device addresses: every case below must fail validation before any
# HIP call, so they are never dereferenced
A1, A2, A3, A4, A5 = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000


def fwd(**kw):
    a = dict(q=A1, k=A2, v=A3, out=A4, lse=A5, B=1, Hq=4, Hkv=2, Nq=64, Nk=64, D=128, scale=0.1,
             causal=0, left=-1, right=-1, dtype=0, stream=None)
    a.update(kw)
    return ea.lib().mfa_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                            a["Nq"], a["Nk"], a["D"], a["scale"], a["causal"], a["left"], a["right"],
                            a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(out=None), -1),
    (dict(dtype=2), -5), (dict(dtype=-1), -5), (dict(D=96), -4), (dict(D=256), -4),
    (dict(B=0), -2), (dict(Hq=0), -2), (dict(Hkv=0), -2), (dict(Nq=0), -2), (dict(Nk=0), -2),
    (dict(Hq=3, Hkv=2), -3), (dict(left=-2), -6), (dict(right=-5), -6),
    (dict(scale=float("nan")), -7), (dict(scale=float("inf")), -7),
    (dict(q=A1 + 2), -12), (dict(out=A4 + 8), -12), (dict(lse=A5 + 2), -12),
    (dict(causal=2), -13), (dict(B=65536, Hq=65536, Hkv=1, Nq=128), -10),
])
def test_fwd_validation(kw, code):
    assert fwd(**kw) == code


def fwd_varlen(**kw):
    a = dict(q=A1, k=A2, v=A3, out=A4, lse=A5, cq=0x60000, ck=0x70000, B=3, Hq=4, Hkv=2, tq=300,
             tk=400, mq=200, mk=250, D=64, scale=0.1, causal=1, left=-1, right=-1, dtype=1,
             stream=None)
    a.update(kw)
    return ea.lib().mfa_fwd_varlen(a["q"], a["k"], a["v"], a["out"], a["lse"], a["cq"], a["ck"],
                                   a["B"], a["Hq"], a["Hkv"], a["tq"], a["tk"], a["mq"], a["mk"],
                                   a["D"], a["scale"], a["causal"], a["left"], a["right"],
                                   a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(cq=None), -1), (dict(ck=None), -1), (dict(out=None), -1),
    (dict(dtype=2), -5), (dict(D=32), -4), (dict(B=0), -2), (dict(tq=0), -2), (dict(tk=0), -2),
    (dict(mq=0), -2), (dict(mk=0), -2), (dict(Hq=6, Hkv=4), -3), (dict(left=-3), -6),
    (dict(scale=float("nan")), -7), (dict(q=A1 + 2), -12), (dict(cq=0x60002), -12),
    (dict(lse=A5 + 1), -12), (dict(causal=-1), -13),
    (dict(mq=1 << 24, Hq=64, Hkv=64), -10), (dict(mk=1 << 24, Hkv=4), -10),
    (dict(B=1 << 20, Hq=64, Hkv=64, mq=1 << 20), -10),
])
def test_fwd_varlen_validation(kw, code):
    assert fwd_varlen(**kw) == code


def fwd_paged(**kw):
    a = dict(q=A1, kp=A2, vp=A3, bt=A4, sl=A5, cq=0x60000, out=0x70000, lse=0x80000, B=3, Hq=4,
             Hkv=2, tq=300, mq=200, mk=320, D=128, page=16, num_pages=50, max_pages=20, scale=0.1,
             causal=1, left=-1, right=-1, dtype=0, stream=None)
    a.update(kw)
    return ea.lib().mfa_fwd_varlen_paged(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["cq"],
                                         a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["tq"],
                                         a["mq"], a["mk"], a["D"], a["page"], a["num_pages"],
                                         a["max_pages"], a["scale"], a["causal"], a["left"],
                                         a["right"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(kp=None), -1), (dict(bt=None), -1), (dict(sl=None), -1),
    (dict(cq=None), -1), (dict(out=None), -1), (dict(dtype=7), -5), (dict(D=96), -4),
    (dict(B=0), -2), (dict(tq=0), -2), (dict(mq=0), -2), (dict(mk=0), -2), (dict(Hq=5, Hkv=2), -3),
    (dict(right=-2), -6), (dict(scale=float("inf")), -7), (dict(page=32), -9),
    (dict(num_pages=0), -9), (dict(max_pages=0), -9), (dict(kp=A2 + 8), -12),
    (dict(sl=A5 + 2), -12), (dict(cq=0x60001), -12), (dict(causal=3), -13),
    (dict(mq=1 << 24, Hq=64, Hkv=64), -10), (dict(max_pages=1 << 27), -10),
])
def test_fwd_varlen_paged_validation(kw, code):
    assert fwd_paged(**kw) == code


def fwd_ext(ext_kw, **kw):
    import ctypes
    e = ea.mfa_fwd_ext_args()
    for k_, v_ in ext_kw.items():
        setattr(e, k_, v_)
    a = dict(q=A1, k=A2, v=A3, out=A4, lse=A5, B=1, Hq=4, Hkv=2, Nq=64, Nk=64, D=128, scale=0.1,
             causal=0, left=-1, right=-1, dtype=0, stream=None)
    a.update(kw)
    return ea.lib().mfa_fwd_ext(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"],
                                a["Hkv"], a["Nq"], a["Nk"], a["D"], a["scale"], a["causal"],
                                a["left"], a["right"], ctypes.byref(e), a["dtype"], a["stream"])


@pytest.mark.parametrize("ext_kw,kw,code", [
    (dict(softcap=-1.0), {}, -13), (dict(softcap=float("inf")), {}, -13),
    (dict(softcap=float("nan")), {}, -13),
    (dict(block_mask=0x90000, block_q=16, block_k=32, mask_q_blocks=4, mask_k_blocks=2), {}, -13),
    (dict(block_mask=0x90000, block_q=32, block_k=48, mask_q_blocks=2, mask_k_blocks=2), {}, -13),
    (dict(block_mask=0x90000, block_q=32, block_k=32, mask_q_blocks=1, mask_k_blocks=2), {}, -13),
    (dict(block_mask=0x90000, block_q=32, block_k=32, mask_q_blocks=2, mask_k_blocks=1), {}, -13),
    (dict(block_mask=0x90000, block_q=32, block_k=32, mask_q_blocks=2, mask_k_blocks=8192,
          mask_stride_h=-1), {}, -13),
    (dict(block_mask=0x90000, block_q=32, block_k=32, mask_q_blocks=2, mask_k_blocks=8192),
     dict(Nk=200000), -10),
    (dict(bias=0x90002), {}, -12), (dict(alibi_slopes=0x90001), {}, -12),
    (dict(bias=0x90000, bias_stride_b=-4), {}, -13),
    ({}, dict(D=96), -4), ({}, dict(q=None), -1), ({}, dict(Hq=3), -3),
])
def test_fwd_ext_validation(ext_kw, kw, code):
    assert fwd_ext(ext_kw, **kw) == code


def test_fwd_ext_null_args():
    assert ea.lib().mfa_fwd_ext(A1, A2, A3, A4, A5, 1, 4, 2, 64, 64, 128, 0.1, 0, -1, -1, None, 0,
                                None) == -1


def bwd(**kw):
    a = dict(q=A1, k=A2, v=A3, o=A4, do=A5, lse=0x60000, dq=0x70000, dk=0x80000, dv=0x90000,
             ws=0xa0000, ws_bytes=1 << 20, B=1, Hq=4, Hkv=2, Nq=64, Nk=80, D=128, scale=0.1,
             causal=1, left=-1, right=-1, dtype=1, stream=None)
    a.update(kw)
    return ea.lib().mfa_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                            a["dv"], a["ws"], a["ws_bytes"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                            a["Nk"], a["D"], a["scale"], a["causal"], a["left"], a["right"],
                            a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(do=None), -1), (dict(lse=None), -1),
    (dict(dq=None), -1), (dict(dk=None), -1), (dict(dv=None), -1), (dict(dtype=3), -5),
    (dict(D=80), -4), (dict(Nq=0), -2), (dict(Hq=3), -3), (dict(left=-4), -6),
    (dict(scale=float("nan")), -7), (dict(ws=None), -8), (dict(ws_bytes=2 * 4 * 64 * 4 - 1), -8),
    (dict(dk=0x80008), -12), (dict(lse=0x60002), -12), (dict(causal=5), -13),
])
def test_bwd_validation(kw, code):
    assert bwd(**kw) == code


def test_bwd_workspace_bytes():
    assert ea.lib().mfa_bwd_workspace_bytes(2, 8, 4096) == 2 * 2 * 8 * 4096 * 4
    assert ea.lib().mfa_bwd_workspace_bytes(0, 8, 4096) == 0


def dec(**kw):
    a = dict(q=A1, kp=A2, vp=A3, bt=A4, sl=A5, out=0x60000, lse=0x70000, B=2, Hq=8, Hkv=2, D=128,
             page_size=16, num_pages=10, max_pages=4, scale=0.1, num_splits=0, ws=0x80000,
             ws_bytes=1 << 30, dtype=1, stream=None)
    a.update(kw)
    return ea.lib().mfa_decode_paged(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["out"], a["lse"],
                                     a["B"], a["Hq"], a["Hkv"], a["D"], a["page_size"],
                                     a["num_pages"], a["max_pages"], a["scale"], a["num_splits"],
                                     a["ws"], a["ws_bytes"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(bt=None), -1), (dict(sl=None), -1), (dict(out=None), -1),
    (dict(dtype=5), -5), (dict(D=80), -4), (dict(B=0), -2), (dict(Hkv=3), -3),
    (dict(page_size=32), -9), (dict(num_pages=0), -9), (dict(max_pages=0), -9),
    (dict(scale=float("-inf")), -7), (dict(num_splits=-1), -13), (dict(ws=None), -8),
    (dict(ws_bytes=16), -8), (dict(q=A1 + 4), -12), (dict(bt=A4 + 2), -12),
])
def test_decode_validation(kw, code):
    assert dec(**kw) == code


def dec_multi(**kw):
    a = dict(q=A1, kp=A2, vp=A3, bt=A4, sl=A5, out=0x60000, lse=0x70000, B=2, Nq=4, Hq=8, Hkv=2,
             D=128, page_size=16, num_pages=10, max_pages=4, scale=0.1, num_splits=0, ws=0x80000,
             ws_bytes=1 << 30, dtype=1, stream=None)
    a.update(kw)
    return ea.lib().mfa_decode_paged_multi(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["out"],
                                           a["lse"], a["B"], a["Nq"], a["Hq"], a["Hkv"], a["D"],
                                           a["page_size"], a["num_pages"], a["max_pages"],
                                           a["scale"], a["num_splits"], a["ws"], a["ws_bytes"],
                                           a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(sl=None), -1), (dict(dtype=5), -5), (dict(D=80), -4),
    (dict(Nq=0), -2), (dict(Nq=5), -2), (dict(B=0), -2), (dict(Hkv=3), -3),
    (dict(page_size=8), -9), (dict(scale=float("nan")), -7), (dict(num_splits=-2), -13),
    (dict(ws=None), -8), (dict(ws_bytes=100), -8), (dict(out=0x60004), -12),
])
def test_decode_multi_validation(kw, code):
    assert dec_multi(**kw) == code


def test_multi_workspace_bytes():
    # B * Nq * Hq * S * (D + 1) floats.  One token: the single-token decode's split count;
    # with explicit num_splits the same count for every Nq; auto with Nq > 1: 2048 pages in
    # chunks of 88 (24 splits)
    one = ea.mfa_decode_workspace_bytes(16, 32, 128, 16, 2048, 0)
    assert ea.mfa_decode_multi_workspace_bytes(16, 1, 32, 128, 16, 2048, 0) == one
    for nq in (1, 2, 3, 4):
        assert ea.mfa_decode_multi_workspace_bytes(16, nq, 32, 128, 16, 2048, 7) == \
            nq * ea.mfa_decode_workspace_bytes(16, 32, 128, 16, 2048, 7)
    for nq in (2, 3, 4):
        assert ea.mfa_decode_multi_workspace_bytes(16, nq, 32, 128, 16, 2048, 0) == \
            16 * nq * 32 * 24 * 129 * 4
    assert ea.mfa_decode_multi_workspace_bytes(16, 5, 32, 128, 16, 2048, 0) == 0
    assert ea.mfa_decode_multi_workspace_bytes(16, 0, 32, 128, 16, 2048, 0) == 0


def test_workspace_and_splits():
    for max_pages, ns in [(2048, 0), (64, 0), (4, 0), (2048, 1), (2048, 7), (100, 3), (9, 1000)]:
        S = ea.mfa_decode_num_splits(16, max_pages, ns)
        assert 1 <= S <= max_pages
        if ns > 0:
            assert S <= ns
        assert ea.mfa_decode_workspace_bytes(16, 32, 128, 16, max_pages, ns) == 16 * 32 * S * 129 * 4
    assert ea.mfa_decode_num_splits(16, 2048, 0) == 32   # auto: 64-page chunks
    assert ea.mfa_decode_workspace_bytes(16, 32, 128, 8, 2048, 0) == 0
    with pytest.raises(ea.MfaError):
        ea.mfa_decode_num_splits(16, 0, 0)


def test_last_dispatch_is_per_thread():
    out = {}

    def run():
        try:
            ea.mfa_last_dispatch()
            out["r"] = "ok"
        except ea.MfaError as e:
            out["r"] = e.status

    t = threading.Thread(target=run)
    t.start()
    t.join()
    assert out["r"] == -13


# ---- the torch binding checks every buffer against the sizes it passes to the C ABI,
# before touching the device (CPU tensors here: a check that let them through would fail
# later with "must be a device tensor" instead)

def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.float16)


def _binding_error(fn, *args, match, **kw):
    kw.setdefault("scale", 0.1)
    with pytest.raises((ValueError, TypeError), match=match):
        fn(*args, **kw)


def test_binding_requires_scale():
    # the scale multiplies Q K^T and has no default: omitting it, or passing None, is an error
    # raised before anything reaches the library
    import torch
    q, k = _t(1, 2, 64, 64), _t(1, 2, 64, 64)
    o, do, lse = _t(1, 2, 64, 64), _t(1, 2, 64, 64), _t(1, 2, 64, dtype=torch.float32)
    cu = torch.tensor([0, 64], dtype=torch.int32)
    kp, bt, sl = _t(4, 16, 2, 64), torch.zeros(1, 4, dtype=torch.int32), torch.ones(1, dtype=torch.int32)
    calls = [
        (ea.mfa_fwd, (q, k, k)), (ea.mfa_fwd_ext, (q, k, k)), (ea.mfa_bwd, (q, k, k, o, do, lse)),
        (ea.mfa_fwd_varlen, (q[0].transpose(0, 1).contiguous(),) * 3 + (cu, cu, 64, 64)),
        (ea.mfa_fwd_varlen_paged, (q[0].transpose(0, 1).contiguous(), kp, kp, bt, sl, cu, 64, 64)),
        (ea.mfa_decode_paged, (_t(1, 2, 64), kp, kp, bt, sl)),
        (ea.mfa_decode_paged_multi, (_t(1, 1, 2, 64), kp, kp, bt, sl)),
    ]
    for fn, args in calls:
        with pytest.raises(TypeError, match="scale"):
            fn(*args)
        with pytest.raises(ValueError, match="scale is required"):
            fn(*args, scale=None)


def test_binding_checks_backward_shapes_and_types():
    import torch
    q, k, v = _t(1, 4, 64, 64), _t(1, 2, 80, 64), _t(1, 2, 80, 64)
    o, do, lse = _t(1, 4, 64, 64), _t(1, 4, 64, 64), _t(1, 4, 64, dtype=torch.float32)
    _binding_error(ea.mfa_bwd, q, _t(2, 2, 80, 64), _t(2, 2, 80, 64), o, do, lse, match="shape mismatch")
    _binding_error(ea.mfa_bwd, q, _t(1, 2, 80, 128), _t(1, 2, 80, 128), o, do, lse, match="shape mismatch")
    _binding_error(ea.mfa_bwd, q, k.bfloat16(), v.bfloat16(), o, do, lse, match="one dtype")
    _binding_error(ea.mfa_bwd, q, k, v, o, do, lse, dk=_t(1, 2, 64, 64), match="dk must be")
    _binding_error(ea.mfa_bwd, q, k, v, o, do, lse, dq=_t(1, 4, 64, 64).bfloat16(), match="dq must be")
    _binding_error(ea.mfa_bwd, q, k, v, o, do, lse, dv=_t(1, 2, 80, 32), match="dv must be")


def test_binding_checks_forward_ext_and_tile_logs():
    import torch
    q, k, v = _t(1, 4, 300, 128), _t(1, 2, 300, 128), _t(1, 2, 300, 128)
    _binding_error(ea.mfa_fwd_ext, q, _t(1, 2, 300, 64), _t(1, 2, 300, 64), match="shape mismatch")
    _binding_error(ea.mfa_fwd_ext, q, k.bfloat16(), v.bfloat16(), match="one dtype")
    _binding_error(ea.mfa_fwd_ext, q, k, v, out=_t(1, 4, 299, 128), match="out must be")
    _binding_error(ea.mfa_fwd_ext, q, k, v, lse=_t(1, 4, 300, dtype=torch.float32)[:, :, :10],
                   match="lse must be")
    # 300 rows = 3 query tiles: 1 * 4 * 3 * 4 = 48 int32 records
    short = torch.zeros(47, dtype=torch.int32)
    _binding_error(ea.mfa_fwd, q, k, v, tile_log=short, match="at least 48")
    _binding_error(ea.mfa_fwd_ext, q, k, v, tile_log=short, match="at least 48")
    _binding_error(ea.mfa_fwd, q, k, v, tile_log=torch.zeros(48, dtype=torch.int64), match="int32")
    # varlen: tiles counted from max_seqlen_q (300 -> 3), B = 2 sequences: 2 * 4 * 3 * 4 = 96
    cu = torch.tensor([0, 100, 300], dtype=torch.int32)
    _binding_error(ea.mfa_fwd_varlen, _t(300, 4, 128), _t(300, 2, 128), _t(300, 2, 128), cu, cu,
                   300, 300, tile_log=torch.zeros(95, dtype=torch.int32), match="at least 96")


def test_binding_checks_decode_outputs():
    import torch
    q = _t(2, 8, 128).bfloat16()
    kp = _t(10, 16, 2, 128).bfloat16()
    bt = torch.zeros(2, 4, dtype=torch.int32)
    sl = torch.ones(2, dtype=torch.int32)
    _binding_error(ea.mfa_decode_paged, q, kp, kp, bt, sl, out=_t(2, 8, 128), match="out must be")
    _binding_error(ea.mfa_decode_paged, q, kp, kp, bt, sl, lse=_t(2, 4, dtype=torch.float32),
                   match="lse must be")
    q4 = _t(2, 4, 8, 128).bfloat16()
    _binding_error(ea.mfa_decode_paged_multi, q4, kp, kp, bt, sl, out=_t(2, 4, 8, 64).bfloat16(),
                   match="out must be")
    _binding_error(ea.mfa_decode_paged_multi, q4, kp, kp, bt, sl, lse=_t(2, 8, 4, dtype=torch.float32),
                   match="lse must be")
