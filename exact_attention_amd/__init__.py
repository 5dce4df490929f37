"""exact_attention_amd — MI355X (gfx950) fused exact attention.

A thin ctypes binding over ``libmfa.so`` (C ABI in ``include/mfa.h``).  The functions
keep the C names; they only marshal arguments: check tensor placement, dtype, shape and
contiguity, allocate outputs with torch when the caller passes none, pass raw device
pointers and the current HIP stream, and raise ``MfaError`` on a negative status.
Every step of the computation runs in the library's HIP kernels; there is no other
code path.  If the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmfa.so")

MFA_F16 = 0
MFA_BF16 = 1

STATUS = {
    0: "MFA_OK", -1: "MFA_ERR_NULL", -2: "MFA_ERR_SHAPE", -3: "MFA_ERR_GQA",
    -4: "MFA_ERR_HEAD_DIM", -5: "MFA_ERR_DTYPE", -6: "MFA_ERR_WINDOW", -7: "MFA_ERR_SCALE",
    -8: "MFA_ERR_WORKSPACE", -9: "MFA_ERR_PAGED", -10: "MFA_ERR_OVERFLOW", -11: "MFA_ERR_HIP",
    -12: "MFA_ERR_ALIGN", -13: "MFA_ERR_ARG",
}


class MfaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({mfa_status_string(status)})")


class mfa_plan(ctypes.Structure):
    _fields_ = [("BM", ctypes.c_int), ("BN", ctypes.c_int), ("waves", ctypes.c_int),
                ("n_q_tiles", ctypes.c_int), ("n_k_tiles", ctypes.c_int),
                ("visited", ctypes.c_longlong), ("edge", ctypes.c_longlong)]


class mfa_dispatch_info(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 96), ("op", ctypes.c_int), ("BM", ctypes.c_int),
                ("BN", ctypes.c_int), ("waves", ctypes.c_int), ("grid", ctypes.c_int * 3),
                ("block", ctypes.c_int), ("num_splits", ctypes.c_int),
                ("chunk_tokens", ctypes.c_int), ("planned", ctypes.c_longlong),
                ("n_launches", ctypes.c_int)]


class mfa_fwd_ext_args(ctypes.Structure):
    _fields_ = [("softcap", ctypes.c_float), ("alibi_slopes", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("bias_stride_b", ctypes.c_longlong),
                ("bias_stride_h", ctypes.c_longlong), ("block_mask", ctypes.c_void_p),
                ("mask_stride_b", ctypes.c_longlong), ("mask_stride_h", ctypes.c_longlong),
                ("mask_q_blocks", ctypes.c_int), ("mask_k_blocks", ctypes.c_int),
                ("block_q", ctypes.c_int), ("block_k", ctypes.c_int),
                ("tile_log", ctypes.c_void_p)]


_LIB = None

_VP = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SIGS = {
    "mfa_plan_fwd": (_I, [_I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(mfa_plan), _VP, ctypes.c_longlong]),
    "mfa_fwd": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I, _VP]),
    "mfa_fwd_tilelog": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I,
                             _VP, _VP]),
    "mfa_fwd_ext": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I,
                         ctypes.POINTER(mfa_fwd_ext_args), _I, _VP]),
    "mfa_fwd_varlen": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                            _I, _I, _I, _I, _VP]),
    "mfa_fwd_varlen_tilelog": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I,
                                    _I, _F, _I, _I, _I, _I, _VP, _VP]),
    "mfa_fwd_varlen_paged": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I,
                                  _I, _I, _I, _I, _F, _I, _I, _I, _I, _VP]),
    "mfa_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I]),
    "mfa_bwd": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _I, _I, _I,
                     _I, _I, _I, _F, _I, _I, _I, _I, _VP]),
    "mfa_decode_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I]),
    "mfa_decode_multi_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I, _I]),
    "mfa_decode_paged_multi": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I,
                                    _I, _F, _I, _VP, ctypes.c_size_t, _I, _VP]),
    "mfa_decode_num_splits": (_I, [_I, _I, _I]),
    "mfa_decode_paged_noalloc": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I,
                                      _I, _F, _I, _I, _VP]),
    "mfa_decode_paged": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _F,
                              _I, _VP, ctypes.c_size_t, _I, _VP]),
    "mfa_last_dispatch": (_I, [ctypes.POINTER(mfa_dispatch_info)]),
    "mfa_status_string": (ctypes.c_char_p, [_I]),
    "mfa_version": (_I, []),
}

EXPORTS = tuple(_SIGS)


def lib():
    """Load libmfa.so (built in-tree by ``exact_attention_amd.build``); raise if absent."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m exact_attention_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def mfa_status_string(status: int) -> str:
    return lib().mfa_status_string(int(status)).decode()


def mfa_version() -> int:
    return int(lib().mfa_version())


def _check(st: int, where: str):
    if st != 0:
        raise MfaError(st, where)


_RECORD = None   # list collecting (name, args) of library calls while prepare() runs
_HELD = None     # list collecting the tensors behind those calls' pointers


def _call(name: str, *args):
    """Call library entry point ``name`` with marshalled ``args``; raise on a negative status."""
    st = getattr(lib(), name)(*args)
    if _RECORD is not None:
        _RECORD.append((name, args))
    _check(st, name)
    return st


def prepare(fn, *args, **kw):
    """Run binding function ``fn(*args, **kw)`` once and return a callable that repeats its
    library call with the same marshalled arguments (the same tensors, outputs and stream),
    skipping the Python-side checks: for timing loops, where per-call marshalling would
    otherwise set the pace.  The callable holds references to every argument, so the
    device memory its pointers name stays allocated while it exists."""
    global _RECORD, _HELD
    _RECORD, _HELD = [], []
    try:
        fn(*args, **kw)
        calls, held = _RECORD, _HELD
    finally:
        _RECORD, _HELD = None, None
    if len(calls) != 1:
        raise RuntimeError(f"expected one library call, got {len(calls)}")
    name, cargs = calls[0]
    cfn = getattr(lib(), name)

    def again():
        st = cfn(*cargs)
        if st != 0:
            raise MfaError(st, name)

    again.keep = (args, kw, held)   # the tensors behind the raw pointers in cargs
    return again


def _scale(scale) -> float:
    """The softmax scale is an explicit argument with no default (the pages give it as the
    scalar that multiplies Q K^T before masking); the C ABI checks that it is finite."""
    if scale is None or isinstance(scale, bool):
        raise ValueError("scale is required (it multiplies Q K^T; no default is applied)")
    return float(scale)


def mfa_plan_fwd(Nq: int, Nk: int, D: int, dtype: int = MFA_F16, causal: bool = False,
                 win_left: int = -1, win_right: int = -1, with_ranges: bool = True):
    """Host-only tile plan.  Returns (plan dict, list of (kt_lo, kt_hi) per query tile)."""
    plan = mfa_plan()
    probe = lib().mfa_plan_fwd(Nq, Nk, D, dtype, int(causal), win_left, win_right,
                               ctypes.byref(plan), None, 0)
    _check(probe, "mfa_plan_fwd")
    ranges = None
    if with_ranges:
        buf = (ctypes.c_int32 * (2 * plan.n_q_tiles))()
        _check(lib().mfa_plan_fwd(Nq, Nk, D, dtype, int(causal), win_left, win_right,
                                  ctypes.byref(plan), ctypes.cast(buf, _VP), 2 * plan.n_q_tiles),
               "mfa_plan_fwd")
        ranges = [(buf[2 * t], buf[2 * t + 1]) for t in range(plan.n_q_tiles)]
    d = {f: getattr(plan, f) for f, _ in mfa_plan._fields_}
    return d, ranges


def mfa_last_dispatch() -> dict:
    info = mfa_dispatch_info()
    _check(lib().mfa_last_dispatch(ctypes.byref(info)), "mfa_last_dispatch")
    d = {f: getattr(info, f) for f, _ in mfa_dispatch_info._fields_}
    d["kernel"] = info.kernel.decode()
    d["grid"] = list(info.grid)
    return d


def mfa_decode_workspace_bytes(B: int, Hq: int, D: int, page_size: int, max_pages_per_seq: int,
                               num_splits: int = 0) -> int:
    return int(lib().mfa_decode_workspace_bytes(B, Hq, D, page_size, max_pages_per_seq, num_splits))


def mfa_decode_num_splits(page_size: int, max_pages_per_seq: int, num_splits: int = 0) -> int:
    st = int(lib().mfa_decode_num_splits(page_size, max_pages_per_seq, num_splits))
    if st < 0:
        raise MfaError(st, "mfa_decode_num_splits")
    return st


# ------------------------------------------------------------------ torch marshalling

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return MFA_F16
    if t.dtype == torch.bfloat16:
        return MFA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float16 / bfloat16)")


def _hold(t):
    """Note a tensor whose pointer is passed to the library (kept alive by prepare())."""
    if _HELD is not None:
        _HELD.append(t)
    return t


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _hold(t).data_ptr()


def _need(t, shape, dtype, name):
    """Shape and dtype of a tensor the caller passes in: the C ABI sees only pointers and the
    sizes given here, so every buffer must hold exactly what those sizes say."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)} "
                         f"(got {t.dtype} {tuple(t.shape)})")


def _need_tile_log(tile_log, B, Hq, Nq, D, dtype):
    """tile_log holds B * Hq * n_q_tiles * 4 int32 (n_q_tiles from the host plan)."""
    torch = _torch()
    if tile_log.dtype != torch.int32:
        raise TypeError("tile_log must be int32")
    plan, _ = mfa_plan_fwd(Nq, Nq, D, dtype, with_ranges=False)
    need = B * Hq * plan["n_q_tiles"] * 4
    if tile_log.numel() < need:
        raise ValueError(f"tile_log must hold at least {need} int32 (B * Hq * n_q_tiles * 4)")


def _stream(t):
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def mfa_fwd(q, k, v, scale: float, causal: bool = False, win_left: int = -1,
            win_right: int = -1, out=None, lse=None, return_lse: bool = True, tile_log=None):
    """Forward pass on torch tensors q [B,Hq,Nq,D], k/v [B,Hkv,Nk,D] (fp16 or bf16).

    ``scale`` multiplies Q K^T and has no default.  Returns
    ``(out, lse)``; ``lse`` is None when ``return_lse`` is False and none is given.
    ``tile_log`` (int32 device tensor) selects ``mfa_fwd_tilelog``.
    """
    scale = _scale(scale)
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, D]")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D:
        raise ValueError("shape mismatch between q, k and v")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq)):
        raise ValueError("lse must be float32 [B, Hq, Nq]")
    if out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must match q")
    if tile_log is not None:
        _need_tile_log(tile_log, B, Hq, Nq, D, dt)
    args = [_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
            _dev(lse, "lse") if lse is not None else None,
            B, Hq, Hkv, Nq, Nk, D, float(scale), int(bool(causal)), int(win_left),
            int(win_right), dt, _stream(q)]
    if tile_log is None:
        _call("mfa_fwd", *args)
    else:
        _call("mfa_fwd_tilelog", *args, _dev(tile_log, "tile_log"))
    return out, lse


def mfa_fwd_tilelog(q, k, v, tile_log, **kw):
    return mfa_fwd(q, k, v, tile_log=tile_log, **kw)


def mfa_bwd(q, k, v, out, dout, lse, scale: float, causal: bool = False,
            win_left: int = -1, win_right: int = -1, dq=None, dk=None, dv=None, workspace=None):
    """Backward pass on torch tensors: the gradients (dq, dk, dv) of ``mfa_fwd``'s output
    for upstream gradient ``dout``.  ``out`` and ``lse`` are the forward's results for the
    same q, k, v, scale and mask arguments.  ``workspace`` is allocated here when absent.
    """
    scale = _scale(scale)
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q, k, v must be 4-D [B, H, N, D]")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("shape mismatch between q, k and v")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    for t, n in ((out, "out"), (dout, "dout")):
        if tuple(t.shape) != tuple(q.shape) or t.dtype != q.dtype:
            raise ValueError(f"{n} must match q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("lse must be float32 [B, Hq, Nq]")
    dt = _dtype_code(q)
    for t, like, n in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if t is not None:
            _need(t, like.shape, like.dtype, n)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = int(lib().mfa_bwd_workspace_bytes(B, Hq, Nq))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    _call("mfa_bwd", _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                         _dev(dout, "dout"), _dev(lse, "lse"), _dev(dq, "dq"), _dev(dk, "dk"),
                         _dev(dv, "dv"), _dev(workspace, "workspace"), wbytes, B, Hq, Hkv, Nq, Nk,
                         D, float(scale), int(bool(causal)), int(win_left), int(win_right), dt,
                         _stream(q))
    return dq, dk, dv


def mfa_fwd_ext(q, k, v, scale: float, causal: bool = False, win_left: int = -1,
                win_right: int = -1, softcap: float = 0.0, alibi_slopes=None, bias=None,
                block_mask=None, block_q: int = 0, block_k: int = 0, out=None, lse=None,
                return_lse: bool = True, tile_log=None):
    """Dense forward with score modifiers and a block-sparse mask on torch tensors.

    q [B,Hq,Nq,D], k/v [B,Hkv,Nk,D].  ``alibi_slopes``: float32 [Hq].  ``bias``: float32
    with the keys as its last, contiguous dimension, broadcastable to [B, Hq, Nk] through
    its strides (e.g. [Nk], [Hq, Nk] or [B, Hq, Nk] views).  ``block_mask``: uint8/bool
    [B?, H?, nqb, nkb] (leading dims broadcast through strides) with blocks of
    ``block_q`` x ``block_k`` (multiples of 32).  Returns ``(out, lse)``.
    """
    scale = _scale(scale)
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q, k, v must be 4-D [B, H, N, D]")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("shape mismatch between q, k and v")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    dt = _dtype_code(q)
    if out is not None:
        _need(out, q.shape, q.dtype, "out")
    if lse is not None:
        _need(lse, (B, Hq, Nq), torch.float32, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    ext = mfa_fwd_ext_args()
    ext.softcap = float(softcap)
    keep = []
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or tuple(alibi_slopes.shape) != (Hq,):
            raise ValueError("alibi_slopes must be float32 [Hq]")
        ext.alibi_slopes = _dev(alibi_slopes, "alibi_slopes")
    if bias is not None:
        if bias.dtype != torch.float32 or bias.shape[-1] != Nk or bias.stride(-1) != 1:
            raise ValueError("bias must be float32 with a contiguous last dimension of Nk")
        b3 = bias.expand(B, Hq, Nk) if bias.dim() <= 3 else None
        if b3 is None:
            raise ValueError("bias must broadcast to [B, Hq, Nk]")
        if not bias.is_cuda:
            raise ValueError("bias must be a device tensor")
        ext.bias = _hold(bias).data_ptr()
        ext.bias_stride_b, ext.bias_stride_h = b3.stride(0), b3.stride(1)
        keep.append(bias)
    if block_mask is not None:
        bm = block_mask if block_mask.dtype == torch.uint8 else block_mask.to(torch.uint8)
        if bm.dim() != 4 or bm.stride(-1) != 1 or not bm.is_cuda:
            raise ValueError("block_mask must be a 4-D device tensor [B?, H?, nqb, nkb]")
        b4 = bm.expand(B, Hq, bm.shape[2], bm.shape[3])
        if b4.stride(2) != bm.shape[3]:
            raise ValueError("block_mask rows must be contiguous")
        ext.block_mask = _hold(bm).data_ptr()
        ext.mask_stride_b, ext.mask_stride_h = b4.stride(0), b4.stride(1)
        ext.mask_q_blocks, ext.mask_k_blocks = bm.shape[2], bm.shape[3]
        ext.block_q, ext.block_k = int(block_q), int(block_k)
        keep.append(bm)
    if tile_log is not None:
        _need_tile_log(tile_log, B, Hq, Nq, D, dt)
        ext.tile_log = _dev(tile_log, "tile_log")
    _call("mfa_fwd_ext", _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                             _dev(lse, "lse") if lse is not None else None, B, Hq, Hkv, Nq, Nk, D,
                             float(scale), int(bool(causal)), int(win_left), int(win_right),
                             ctypes.byref(ext), dt, _stream(q))
    return out, lse


def mfa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                   scale: float, causal: bool = False, win_left: int = -1,
                   win_right: int = -1, out=None, lse=None, return_lse: bool = True,
                   tile_log=None):
    """Packed variable-length forward on torch tensors.

    q [total_q, Hq, D], k/v [total_k, Hkv, D] (fp16 or bf16, token-major); cu_seqlens_q /
    cu_seqlens_k int32 [B + 1] device tensors; max_seqlen_q / max_seqlen_k host ints
    bounding every sequence's lengths.  Returns ``(out, lse)`` with lse [Hq, total_q].
    ``tile_log`` selects ``mfa_fwd_varlen_tilelog``.
    """
    scale = _scale(scale)
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q must be [total_q, Hq, D] and k, v [total_k, Hkv, D]")
    total_q, Hq, D = q.shape
    total_k, Hkv, Dk = k.shape
    if Dk != D:
        raise ValueError("head dimension mismatch")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B + 1]")
    B = cu_seqlens_q.numel() - 1
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, total_q)):
        raise ValueError("lse must be float32 [Hq, total_q]")
    if out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must match q")
    if tile_log is not None:
        _need_tile_log(tile_log, B, Hq, max(1, int(max_seqlen_q)), D, dt)
    args = [_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
            _dev(lse, "lse") if lse is not None else None,
            _dev(cu_seqlens_q, "cu_seqlens_q"), _dev(cu_seqlens_k, "cu_seqlens_k"),
            B, Hq, Hkv, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), D, float(scale),
            int(bool(causal)), int(win_left), int(win_right), dt, _stream(q)]
    if tile_log is None:
        _call("mfa_fwd_varlen", *args)
    else:
        _call("mfa_fwd_varlen_tilelog", *args, _dev(tile_log, "tile_log"))
    return out, lse


def mfa_fwd_varlen_paged(q, k_pages, v_pages, block_table, seq_lens_k, cu_seqlens_q,
                         max_seqlen_q: int, max_seqlen_k: int, scale: float,
                         causal: bool = False,
                         win_left: int = -1, win_right: int = -1, out=None, lse=None,
                         return_lse: bool = True):
    """Packed queries over a paged KV cache (chunked prefill) on torch tensors.

    q [total_q, Hq, D]; k_pages/v_pages [num_pages, page_size, Hkv, D]; block_table int32
    [B, max_pages_per_seq]; seq_lens_k int32 [B] (cached keys, the new tokens' included);
    cu_seqlens_q int32 [B + 1]; all on the device; max_seqlen_q / max_seqlen_k host bounds
    of every sequence's query and key counts.  Returns ``(out, lse)``, lse [Hq, total_q].
    """
    scale = _scale(scale)
    torch = _torch()
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("q must be [total_q, Hq, D] and the page pools [P, page, Hkv, D]")
    total_q, Hq, D = q.shape
    P, page_size, Hkv, Dk = k_pages.shape
    if Dk != D:
        raise ValueError("head dimension mismatch")
    if k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("q and the page pools must share one dtype")
    for t, n in ((block_table, "block_table"), (seq_lens_k, "seq_lens_k"), (cu_seqlens_q, "cu_seqlens_q")):
        if t.dtype != torch.int32:
            raise TypeError(f"{n} must be int32")
    B = block_table.shape[0]
    if block_table.dim() != 2 or tuple(seq_lens_k.shape) != (B,) or tuple(cu_seqlens_q.shape) != (B + 1,):
        raise ValueError("block_table must be [B, max_pages], seq_lens_k [B], cu_seqlens_q [B + 1]")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, total_q)):
        raise ValueError("lse must be float32 [Hq, total_q]")
    if out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must match q")
    _call("mfa_fwd_varlen_paged", 
        _dev(q, "q"), _dev(k_pages, "k_pages"), _dev(v_pages, "v_pages"),
        _dev(block_table, "block_table"), _dev(seq_lens_k, "seq_lens_k"),
        _dev(cu_seqlens_q, "cu_seqlens_q"), _dev(out, "out"),
        _dev(lse, "lse") if lse is not None else None, B, Hq, Hkv, total_q, int(max_seqlen_q),
        int(max_seqlen_k), D,
        page_size, P, block_table.shape[1], float(scale), int(bool(causal)), int(win_left),
        int(win_right), dt, _stream(q))
    return out, lse


def mfa_decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale: float,
                     num_splits: int = 0, out=None, lse=None, return_lse: bool = True,
                     workspace=None):
    """Paged split-KV decode on torch tensors.

    q [B,Hq,D]; k_pages/v_pages [num_pages, page_size, Hkv, D]; block_table int32
    [B, max_pages_per_seq]; seq_lens int32 [B] (device).  Returns ``(out, lse)``.
    ``workspace`` (any device tensor of enough bytes) is allocated here when absent.
    """
    scale = _scale(scale)
    torch = _torch()
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("q must be [B, Hq, D] and the page pools [P, page, Hkv, D]")
    B, Hq, D = q.shape
    P, page_size, Hkv, Dk = k_pages.shape
    if Dk != D:
        raise ValueError("head dimension mismatch")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    if k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("q and the page pools must share one dtype")
    dt = _dtype_code(q)
    max_pages = block_table.shape[1]
    if out is not None:
        _need(out, q.shape, q.dtype, "out")
    if lse is not None:
        _need(lse, (B, Hq), torch.float32, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = mfa_decode_workspace_bytes(B, Hq, D, page_size, max_pages, num_splits)
    if need == 0:
        raise MfaError(-13, "mfa_decode_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    _call("mfa_decode_paged", 
        _dev(q, "q"), _dev(k_pages, "k_pages"), _dev(v_pages, "v_pages"),
        _dev(block_table, "block_table"), _dev(seq_lens, "seq_lens"), _dev(out, "out"),
        _dev(lse, "lse") if lse is not None else None,
        B, Hq, Hkv, D, page_size, P, max_pages, float(scale), int(num_splits),
        _dev(workspace, "workspace"), wbytes, dt, _stream(q))
    return out, lse


def mfa_decode_paged_noalloc(q, k_pages, v_pages, block_table, seq_lens, scale: float, out,
                             lse=None, num_splits: int = 0):
    """``mfa_decode_paged`` with the split partials in the library's fixed per-GPU scratch
    (no workspace, nothing allocated by the call): ``out`` [B, Hq, D] and the optional
    ``lse`` [B, Hq] float32 must be given.  Calls overlapping on one GPU race."""
    scale = _scale(scale)
    torch = _torch()
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("q must be [B, Hq, D] and the page pools [P, page, Hkv, D]")
    B, Hq, D = q.shape
    P, page_size, Hkv, Dk = k_pages.shape
    if Dk != D:
        raise ValueError("head dimension mismatch")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    if k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("q and the page pools must share one dtype")
    _need(out, q.shape, q.dtype, "out")
    if lse is not None:
        _need(lse, (B, Hq), torch.float32, "lse")
    _call("mfa_decode_paged_noalloc", 
        _dev(q, "q"), _dev(k_pages, "k_pages"), _dev(v_pages, "v_pages"),
        _dev(block_table, "block_table"), _dev(seq_lens, "seq_lens"), _dev(out, "out"),
        _dev(lse, "lse") if lse is not None else None,
        B, Hq, Hkv, D, page_size, P, block_table.shape[1], float(scale), int(num_splits),
        _dtype_code(q), _stream(q))
    return out, lse


def mfa_decode_multi_workspace_bytes(B: int, Nq: int, Hq: int, D: int, page_size: int,
                                     max_pages_per_seq: int, num_splits: int = 0) -> int:
    return int(lib().mfa_decode_multi_workspace_bytes(B, Nq, Hq, D, page_size, max_pages_per_seq,
                                                      num_splits))


def mfa_decode_paged_multi(q, k_pages, v_pages, block_table, seq_lens, scale: float,
                           num_splits: int = 0, out=None, lse=None, return_lse: bool = True,
                           workspace=None):
    """Paged split-KV decode of Nq <= 4 new tokens per sequence on torch tensors.

    q [B, Nq, Hq, D]; k_pages/v_pages [num_pages, page_size, Hkv, D]; block_table int32
    [B, max_pages_per_seq]; seq_lens int32 [B] (the new tokens included).  Returns
    ``(out [B, Nq, Hq, D], lse [B, Nq, Hq])``.
    """
    scale = _scale(scale)
    torch = _torch()
    if q.dim() != 4 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("q must be [B, Nq, Hq, D] and the page pools [P, page, Hkv, D]")
    B, Nq, Hq, D = q.shape
    P, page_size, Hkv, Dk = k_pages.shape
    if Dk != D:
        raise ValueError("head dimension mismatch")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    if k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("q and the page pools must share one dtype")
    dt = _dtype_code(q)
    max_pages = block_table.shape[1]
    if out is not None:
        _need(out, q.shape, q.dtype, "out")
    if lse is not None:
        _need(lse, (B, Nq, Hq), torch.float32, "lse")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=q.device)
    need = mfa_decode_multi_workspace_bytes(B, Nq, Hq, D, page_size, max_pages, num_splits)
    if need == 0:
        raise MfaError(-2, "mfa_decode_multi_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    _call("mfa_decode_paged_multi", 
        _dev(q, "q"), _dev(k_pages, "k_pages"), _dev(v_pages, "v_pages"),
        _dev(block_table, "block_table"), _dev(seq_lens, "seq_lens"), _dev(out, "out"),
        _dev(lse, "lse") if lse is not None else None,
        B, Nq, Hq, Hkv, D, page_size, P, max_pages, float(scale), int(num_splits),
        _dev(workspace, "workspace"), wbytes, dt, _stream(q))
    return out, lse


__all__ = ["MFA_F16", "MFA_BF16", "MfaError", "EXPORTS", "lib", "mfa_fwd", "mfa_fwd_tilelog",
           "mfa_fwd_ext", "mfa_fwd_ext_args", "mfa_bwd", "mfa_fwd_varlen", "mfa_fwd_varlen_paged",
           "mfa_decode_paged_multi",
           "mfa_decode_multi_workspace_bytes",
           "mfa_decode_paged", "mfa_decode_workspace_bytes", "mfa_decode_num_splits",
           "mfa_decode_paged_noalloc",
           "mfa_plan_fwd", "mfa_last_dispatch", "mfa_status_string", "mfa_version", "prepare"]
