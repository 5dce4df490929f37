"""Helpers shared by the GPU tests (no attention arithmetic here)."""
import numpy as np

TOL_O = {"f16": 2e-3, "bf16": 1.5e-2}   # max-abs on O (fp32 accumulation)
TOL_LSE = 1e-3                          # absolute, on LSE
U_GRAD = {"f16": 2.0 ** -12, "bf16": 2.0 ** -9}   # unit roundoff of the gradient type


def torch_dtype(dtype):
    import torch
    return torch.float16 if dtype == "f16" else torch.bfloat16


def to_dev(bits: np.ndarray, dtype: str):
    """uint16 bit patterns -> device tensor of the 16-bit float type (bit-identical)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")
    return t.view(torch_dtype(dtype))


def to_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t, dtype) -> np.ndarray:
    import oracle
    return oracle.widen(to_bits(t), dtype)


MANT_BITS = {"f16": 11, "bf16": 8}   # significant bits of the output type


def output_step(dtype: str, ref: np.ndarray) -> np.ndarray:
    """One step (ulp) of the output type at |ref| (normal range)."""
    a = np.maximum(np.abs(ref), 2.0 ** -14)
    return np.exp2(np.floor(np.log2(a)) - (MANT_BITS[dtype] - 1))


UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}   # relative error of one RNE rounding


def assert_close_o(got: np.ndarray, ref: np.ndarray, dtype: str, what="", ref_pabs=None):
    """max |got - ref| <= the O tolerance of the type.

    With ref_pabs (the oracle's attention applied to |V|, i.e. sum_j P_ij |V_jd|), an
    element's bound is the larger of that tolerance and what the rounding of the
    arithmetic allows there: P rounded to the input type before P V (relative error u on
    each term; for f16 the row sum adds the rounded P as well) and O rounded once:
        u (sum_j P_ij |V_jd| + |O_id|) + step(O_id) / 2 + 1e-6.
    For outputs of about unit scale this is below the tolerance; it exceeds it where the
    softmax is peaked and |O| is 2 or more (one bf16 step there is 2^-6)."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if not got.size:
        return 0.0
    d = np.abs(got - ref)
    err = float(np.max(d))
    if ref_pabs is not None:
        assert ref_pabs.shape == ref.shape
        u = UNIT_ROUNDOFF[dtype]
        bound = np.maximum(TOL_O[dtype], u * (ref_pabs + np.abs(ref)) + output_step(dtype, ref) / 2 + 1e-6)
        j = int(np.argmax(d - bound))
        assert d.flat[j] <= bound.flat[j], (f"{what}: |dO| = {d.flat[j]:.3e} > {bound.flat[j]:.3e} "
                                             f"at |O| = {abs(ref.flat[j]):.3f}")
    else:
        assert err <= TOL_O[dtype], f"{what}: max |dO| = {err:.3e} > {TOL_O[dtype]}"
    return err


def assert_close_lse(got: np.ndarray, ref: np.ndarray, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(got[fin]))
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    assert err <= TOL_LSE, f"{what}: max |dLSE| = {err:.3e} > {TOL_LSE}"
    return err


def assert_close_grads(names, gots, refs, dtype):
    """Gradients: max |got - ref| <= 8 u times the largest reference magnitude of the
    group (dQ, dK and dV all scale with |dO|; one of them can be exactly zero, e.g. dQ
    with a single key)."""
    M = max(float(np.max(np.abs(r))) if r.size else 0.0 for r in refs)
    tol = 8 * U_GRAD[dtype] * max(M, 1e-6)
    bad = []
    for name, got, ref in zip(names, gots, refs):
        assert np.all(np.isfinite(got)), f"{name}: non-finite"
        err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
        m = float(np.max(np.abs(ref))) if ref.size else 0.0
        print(f"  {name}: max|d|={err:.3e}  max|ref|={m:.3e}  tol={tol:.3e}")
        if err > tol:
            bad.append(f"{name}: max |d| = {err:.3e} > {tol:.3e}")
    assert not bad, "; ".join(bad)


def oracle_heads(qf, kf, vf, scale, causal, left, right, heads, workers=None):
    """``oracle.attention`` over whole heads, several at once.

    ``heads`` lists (b, h) pairs; query head h reads KV head h // (Hq / Hkv) (consecutive
    grouping), passed to the oracle as a one-head problem.  Threads run the heads side by
    side (numpy releases the GIL inside its array arithmetic) with BLAS limited to one
    thread each.  Returns {(b, h): (O [Nq, D], LSE [Nq])}."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from threadpoolctl import threadpool_limits

    g = qf.shape[1] // kf.shape[1]

    def one(bh):
        b, h = bh
        kv = h // g
        O, L = oracle.attention(qf[b:b + 1, h:h + 1], kf[b:b + 1, kv:kv + 1],
                                vf[b:b + 1, kv:kv + 1], scale, causal, left, right)
        return O[0, 0], L[0, 0]

    n = workers or max(1, min(16, os.cpu_count() or 1, len(heads)))
    with threadpool_limits(1), ThreadPoolExecutor(n) as ex:
        return dict(zip(heads, ex.map(one, heads)))
