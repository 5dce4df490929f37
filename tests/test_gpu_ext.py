"""GPU parity of the forward with score modifiers and block-sparse masks (mfa_fwd_ext
through the C ABI) against the oracle's attention_ext."""
import math

import numpy as np
import pytest

import attn_inputs as A
import oracle
from gpu_util import assert_close_lse, assert_close_o, to_dev, to_f64

pytestmark = pytest.mark.gpu

ea = pytest.importorskip("exact_attention_amd")


def dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def dev_u8(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")


def case(B, Hq, Hkv, Nq, Nk, D, dtype, seed, causal=False, left=-1, right=-1, softcap=0.0,
         slopes=None, bias=None, bmask=None, bq=0, bk=0, scale=None, tile_log=None):
    import torch
    x = A.dense_inputs(B, Hq, Hkv, Nq, Nk, D, dtype, seed)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v = (to_dev(t, dtype) for t in (x.q, x.k, x.v))
    print(f"mfa_fwd_ext q={tuple(q.shape)} k={tuple(k.shape)} {dtype} causal={causal} "
          f"win=({left},{right}) softcap={softcap} alibi={slopes is not None} "
          f"bias={None if bias is None else bias.shape} mask={None if bmask is None else bmask.shape}"
          f" blocks=({bq},{bk})", flush=True)
    O, L = ea.mfa_fwd_ext(q, k, v, scale=scale, causal=causal, win_left=left, win_right=right,
                          softcap=softcap,
                          alibi_slopes=None if slopes is None else dev_f32(slopes),
                          bias=None if bias is None else dev_f32(bias),
                          block_mask=None if bmask is None else dev_u8(bmask), block_q=bq,
                          block_k=bk, tile_log=tile_log)
    torch.cuda.synchronize()
    qf, kf, vf = (oracle.widen(t, dtype) for t in (x.q, x.k, x.v))
    bias_full = None if bias is None else np.broadcast_to(bias, (B, Hq, Nk))
    bm_full = None if bmask is None else np.broadcast_to(bmask, (B, Hq) + bmask.shape[-2:])
    Or, Lr = oracle.attention_ext(qf, kf, vf, scale, causal, left, right, softcap=softcap,
                                  alibi_slopes=slopes, bias=bias_full, block_mask=bm_full,
                                  block_q=bq, block_k=bk)
    eo = assert_close_o(to_f64(O, dtype), Or, dtype, "ext O")
    el = assert_close_lse(L.cpu().numpy(), Lr, "ext LSE")
    info = ea.mfa_last_dispatch()
    assert info["op"] == 6 and ",ext" in info["kernel"]
    return eo, el, O, L


MOD_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, left, right, softcap, alibi, bias shape
    (1, 4, 2, 300, 300, 128, "f16", True, -1, -1, 30.0, False, None),
    (2, 2, 2, 257, 400, 64, "bf16", True, -1, -1, 5.0, False, None),
    (1, 4, 4, 333, 333, 128, "bf16", True, -1, -1, 0.0, True, None),
    (1, 2, 1, 200, 517, 128, "f16", False, 60, 40, 0.0, True, None),
    (1, 4, 2, 300, 300, 128, "f16", False, -1, -1, 0.0, False, "key"),
    (2, 4, 2, 190, 260, 64, "bf16", True, -1, -1, 0.0, False, "head"),
    (2, 4, 4, 190, 190, 128, "f16", True, 100, 0, 0.0, False, "full"),
    (2, 8, 2, 400, 400, 128, "bf16", True, -1, -1, 20.0, True, "full"),
]


@pytest.mark.parametrize("c", MOD_CASES, ids=[str(i) for i in range(len(MOD_CASES))])
def test_modifiers(c):
    B, Hq, Hkv, Nq, Nk, D, dt, causal, left, right, sc, alibi, bshape = c
    rng = np.random.default_rng(Nq + Nk)
    slopes = 2.0 ** (-8.0 * (np.arange(Hq) + 1) / Hq) if alibi else None
    bias = None
    if bshape == "key":
        bias = rng.standard_normal(Nk)
    elif bshape == "head":
        bias = rng.standard_normal((Hq, Nk))
    elif bshape == "full":
        bias = rng.standard_normal((B, Hq, Nk))
    eo, el, _, _ = case(B, Hq, Hkv, Nq, Nk, D, dt, 40 + Nq, causal, left, right, sc, slopes, bias)
    print(f"modifiers {c}: max|dO|={eo:.2e} max|dLSE|={el:.2e}")


def test_negative_scale_with_softcap():
    case(1, 2, 2, 200, 200, 128, "f16", 41, True, softcap=10.0, scale=-0.2)


BLOCK_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, left, right, bq, bk, density, mask per head
    (1, 4, 2, 512, 512, 128, "f16", True, -1, -1, 32, 32, 0.5, True),
    (2, 2, 2, 700, 700, 64, "bf16", False, -1, -1, 64, 64, 0.4, False),
    (1, 2, 1, 333, 900, 128, "bf16", True, -1, -1, 32, 64, 0.6, True),
    (1, 4, 4, 640, 640, 128, "f16", True, 200, 0, 128, 32, 0.7, True),
    # more than two query tiles per CU with Hkv a multiple of 8: head-major order per XCD
    (1, 64, 16, 1100, 1100, 128, "f16", True, -1, -1, 128, 128, 0.3, True),
    (1, 48, 48, 1500, 1500, 64, "bf16", True, 200, 0, 64, 32, 0.5, False),
]


def visited_tiles_masked(Nq, Nk, causal, left, right, bm, bq, bk, BM=128, BN=64):
    """Brute force: per query tile, the key tiles holding a visible, unmasked pair."""
    ii = np.arange(Nq)[:, None]
    jj = np.arange(Nk)[None, :]
    vis = oracle.visible(ii, jj, Nq, Nk, causal, left, right)
    vis &= np.kron(bm.astype(bool), np.ones((bq, bk), bool))[:Nq, :Nk]
    out = []
    for qt in range(math.ceil(Nq / BM)):
        cols = vis[qt * BM:(qt + 1) * BM].any(axis=0)
        out.append([kt for kt in range(math.ceil(Nk / BN)) if cols[kt * BN:(kt + 1) * BN].any()])
    return out


@pytest.mark.parametrize("c", BLOCK_CASES, ids=[str(i) for i in range(len(BLOCK_CASES))])
def test_block_sparse(c):
    import torch
    B, Hq, Hkv, Nq, Nk, D, dt, causal, left, right, bq, bk, dens, per_head = c
    nqb, nkb = math.ceil(Nq / bq), math.ceil(Nk / bk)
    rng = np.random.default_rng(nqb * 31 + nkb)
    bm = (rng.random((B, Hq if per_head else 1, nqb, nkb)) < dens).astype(np.uint8)
    nqt = math.ceil(Nq / 128)
    log = torch.full((B * Hq * nqt * 4,), -7, dtype=torch.int32, device="cuda")
    eo, el, _, _ = case(B, Hq, Hkv, Nq, Nk, D, dt, 50 + Nq, causal, left, right, bmask=bm, bq=bq,
                        bk=bk, tile_log=log)
    kern = ea.mfa_last_dispatch()["kernel"]
    one_group = B * Hq * nqt > 2 * 256
    assert (",head-major" in kern) == (one_group and Hkv % 8 == 0), kern
    log = log.view(B, Hq, nqt, 4).cpu().numpy()
    for b in range(B):
        for h in range(Hq):
            ref = visited_tiles_masked(Nq, Nk, causal, left, right, bm[b, h if per_head else 0], bq, bk)
            for t in range(nqt):
                first, count, edge, end = log[b, h, t]
                assert count == len(ref[t]), (b, h, t, count, ref[t])
                assert 0 <= edge <= count
                if ref[t]:
                    assert first == ref[t][0] and end == ref[t][-1] + 1
                else:
                    assert first == -1 and end == -1
    print(f"block sparse {c}: max|dO|={eo:.2e} max|dLSE|={el:.2e}")


def test_block_mask_rows_with_nothing():
    # query blocks whose whole mask row is off give O = 0 and LSE = -inf
    import torch
    bm = np.ones((1, 1, 4, 4), np.uint8)
    bm[0, 0, 1, :] = 0
    _, _, O, L = case(1, 2, 2, 256, 256, 128, "bf16", 61, bmask=bm, bq=64, bk=64)
    assert torch.all(O[:, :, 64:128] == 0) and torch.all(torch.isneginf(L[:, :, 64:128]))


def test_all_modifiers_with_block_mask_both_layouts():
    # every feature at once, with a small grid (two key-split wave groups) and a large
    # one (one group per workgroup)
    for Hq, groups in ((2, 2), (160, 1)):
        rng = np.random.default_rng(Hq)
        bm = (rng.random((1, Hq, 16, 16)) < 0.6).astype(np.uint8)
        bm[..., 0] = 1
        slopes = np.linspace(0.01, 0.2, Hq)
        bias = rng.standard_normal((Hq, 1024))
        case(1, Hq, 2, 512, 1024, 128, "f16", 70 + Hq, True, softcap=15.0, slopes=slopes, bias=bias,
             bmask=bm, bq=32, bk=64)
        assert f"groups={groups}" in ea.mfa_last_dispatch()["kernel"]


def test_large_sparse_sampled():
    # a long causal sequence with a 128 x 128 block mask of about 30% density, sampled rows
    import torch
    B, H, N, D = 1, 8, 8192, 128
    x = A.dense_inputs(B, H, H, N, N, D, "bf16", 77)
    rng = np.random.default_rng(77)
    bm = (rng.random((1, H, 64, 64)) < 0.3).astype(np.uint8)
    bm[:, :, np.arange(64), np.arange(64)] = 1
    q, k, v = (to_dev(t, "bf16") for t in (x.q, x.k, x.v))
    print("mfa_fwd_ext large sparse", flush=True)
    O, L = ea.mfa_fwd_ext(q, k, v, scale=1 / math.sqrt(D), causal=True, softcap=30.0,
                          block_mask=dev_u8(bm), block_q=128, block_k=128)
    torch.cuda.synchronize()
    rows = sorted({(0, h, i) for h in (0, 3, 7) for i in (0, 1, 127, 128, 4095, 4096, 8191)} |
                  {(0, int(rng.integers(H)), int(rng.integers(N))) for _ in range(60)})
    qf, kf, vf = (oracle.widen(t, "bf16") for t in (x.q, x.k, x.v))
    Or, Lr = oracle.attention_ext(qf, kf, vf, 1 / math.sqrt(D), True, softcap=30.0, block_mask=bm,
                                  block_q=128, block_k=128, rows=rows)
    idx = tuple(np.array(rows).T)
    assert_close_o(to_f64(O, "bf16")[idx], Or, "bf16", "large sparse")
    assert_close_lse(L.cpu().numpy()[idx], Lr, "large sparse")
