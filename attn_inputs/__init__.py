"""Seeded synthetic inputs for exact attention, shared by the oracle and the HIP path.

This module only *draws* data: it holds none of the attention arithmetic.  Both the
CPU oracle (``oracle/``) and the GPU side (tests, ``bench.py``) take their inputs from
here, so the two sides see bit-identical operands.

Recipe (the workloads of the paged-decode and prefill benchmarks described on the
mlx-mfa pages, "Performance" table, and the MXFlashAttn paged Split-KV decode page):

* ``numpy.random.default_rng(seed)`` (PCG64).
* Dense prefill: draw Q, K, V in that order as ``standard_normal(shape, float32)``
  with Q ``[B, Hq, Nq, D]`` and K, V ``[B, Hkv, Nk, D]`` (the ``[B, H, N, D]``
  row-major layout of the mlx-mfa "Supported Configurations" table).
* Rounding to the storage type: fp16 by numpy's cast (round to nearest even);
  bf16 by round-to-nearest-even on the float32 bit pattern.  Arrays are returned as
  ``uint16`` bit patterns so that no later cast can perturb them.
* Paged decode: draw order is ``seq_lens`` (uniform integers in ``[len_lo, len_hi]``),
  then a permutation of the page pool, then q ``[B, Hq, D]``, then the K tokens and
  the V tokens of every sequence in order (``[sum(L_b), Hkv, D]`` each).  The pool
  holds ``P = sum(ceil(L_b / page_size))`` pages plus ``extra_pages`` unused ones;
  the permutation is dealt to the sequences in order, so page ``j`` of sequence
  ``b`` is ``block_table[b, j]``.  Token ``t`` of sequence ``b`` is stored at
  ``(block_table[b, t // page_size], t % page_size)`` of the pool
  ``[num_pages, page_size, Hkv, D]``.  Unused block-table entries are -1; tail slots
  of each sequence's last page and every unused page hold NaN, so that a kernel
  which reads them is caught.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F16 = "f16"
BF16 = "bf16"

NAN_BITS = {F16: np.uint16(0x7E00), BF16: np.uint16(0x7FC0)}


def round_f32_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 array to fp16 or bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = x.view(np.uint32)
        # round-to-nearest-even on the upper 16 bits; NaNs are kept quiet NaNs
        rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            out[nan] = NAN_BITS[BF16]
        return out
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal_bits(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return round_f32_to_bits(rng.standard_normal(shape, dtype=np.float32), dtype)


@dataclass
class DenseInputs:
    q: np.ndarray  # uint16 bits [B, Hq, Nq, D]
    k: np.ndarray  # uint16 bits [B, Hkv, Nk, D]
    v: np.ndarray  # uint16 bits [B, Hkv, Nk, D]
    dtype: str


def dense_inputs(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, D: int, dtype: str,
                 seed: int) -> DenseInputs:
    rng = np.random.default_rng(seed)
    q = _normal_bits(rng, (B, Hq, Nq, D), dtype)
    k = _normal_bits(rng, (B, Hkv, Nk, D), dtype)
    v = _normal_bits(rng, (B, Hkv, Nk, D), dtype)
    return DenseInputs(q, k, v, dtype)


def grad_inputs(B: int, Hq: int, Nq: int, D: int, dtype: str, seed: int) -> np.ndarray:
    """Upstream gradient dO: standard normal, rounded to `dtype`; uint16 bits [B, Hq, Nq, D]."""
    rng = np.random.default_rng(seed)
    return _normal_bits(rng, (B, Hq, Nq, D), dtype)


@dataclass
class PagedInputs:
    q: np.ndarray            # uint16 bits [B, Hq, D]
    k_pages: np.ndarray      # uint16 bits [num_pages, page_size, Hkv, D]
    v_pages: np.ndarray      # uint16 bits [num_pages, page_size, Hkv, D]
    block_table: np.ndarray  # int32 [B, max_pages_per_seq], -1 where unused
    seq_lens: np.ndarray     # int32 [B]
    page_size: int
    dtype: str
    pages_used: int = field(default=0)


def paged_inputs(B: int, Hq: int, Hkv: int, D: int, dtype: str, seed: int, *,
                 len_lo: int, len_hi: int, page_size: int = 16,
                 max_pages_per_seq: int | None = None, extra_pages: int = 0,
                 seq_lens=None) -> PagedInputs:
    """Paged KV pool with a seeded random page permutation (see module docstring).

    ``seq_lens`` may be given explicitly (still consuming no random draws for them).
    """
    rng = np.random.default_rng(seed)
    if seq_lens is None:
        seq_lens = rng.integers(len_lo, len_hi, endpoint=True, size=B)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    assert seq_lens.shape == (B,)
    pages_per_seq = [int(math.ceil(int(L) / page_size)) for L in seq_lens]
    used = int(sum(pages_per_seq))
    num_pages = used + int(extra_pages)
    if max_pages_per_seq is None:
        max_pages_per_seq = max(1, int(math.ceil(len_hi / page_size)))
    if max(pages_per_seq, default=0) > max_pages_per_seq:
        raise ValueError("max_pages_per_seq too small for the drawn sequence lengths")
    perm = rng.permutation(num_pages).astype(np.int64)
    q = _normal_bits(rng, (B, Hq, D), dtype)
    total = int(seq_lens.sum())
    k_tok = _normal_bits(rng, (total, Hkv, D), dtype)
    v_tok = _normal_bits(rng, (total, Hkv, D), dtype)

    block_table, k_pages, v_pages = _scatter_pages(k_tok, v_tok, seq_lens, perm, num_pages,
                                                   page_size, max_pages_per_seq, dtype)
    return PagedInputs(q, k_pages, v_pages, block_table, seq_lens.astype(np.int32),
                       page_size, dtype, used)


def _scatter_pages(k_tok, v_tok, seq_lens, perm, num_pages, page_size, max_pages_per_seq, dtype):
    """Deal the permuted pages to the sequences in order and copy each sequence's tokens
    (consecutive in ``k_tok`` / ``v_tok``) into them; everything else holds NaN."""
    B = len(seq_lens)
    Hkv, D = k_tok.shape[1:]
    block_table = np.full((B, max_pages_per_seq), -1, dtype=np.int32)
    k_pages = np.full((num_pages, page_size, Hkv, D), NAN_BITS[dtype], dtype=np.uint16)
    v_pages = np.full((num_pages, page_size, Hkv, D), NAN_BITS[dtype], dtype=np.uint16)
    cursor = 0
    tok0 = 0
    for b in range(B):
        L = int(seq_lens[b])
        n = int(math.ceil(L / page_size))
        pages = perm[cursor:cursor + n]
        cursor += n
        block_table[b, :n] = pages
        for j in range(n):
            t0 = j * page_size
            t1 = min(L, t0 + page_size)
            k_pages[pages[j], : t1 - t0] = k_tok[tok0 + t0: tok0 + t1]
            v_pages[pages[j], : t1 - t0] = v_tok[tok0 + t0: tok0 + t1]
        tok0 += L
    return block_table, k_pages, v_pages


def paged_multi_inputs(B: int, Nq: int, Hq: int, Hkv: int, D: int, dtype: str, seed: int, *,
                       len_lo: int, len_hi: int, page_size: int = 16,
                       max_pages_per_seq: int | None = None, extra_pages: int = 0,
                       seq_lens=None) -> PagedInputs:
    """``paged_inputs`` with ``Nq`` query tokens per sequence: q is ``[B, Nq, Hq, D]``
    (same draw order; the q draw has the extra token axis)."""
    rng = np.random.default_rng(seed)
    if seq_lens is None:
        seq_lens = rng.integers(len_lo, len_hi, endpoint=True, size=B)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    pages_per_seq = [int(math.ceil(int(L) / page_size)) for L in seq_lens]
    used = int(sum(pages_per_seq))
    num_pages = max(1, used + int(extra_pages))
    if max_pages_per_seq is None:
        max_pages_per_seq = max(1, int(math.ceil(len_hi / page_size)))
    if max(pages_per_seq, default=0) > max_pages_per_seq:
        raise ValueError("max_pages_per_seq too small for the drawn sequence lengths")
    perm = rng.permutation(num_pages).astype(np.int64)
    q = _normal_bits(rng, (B, Nq, Hq, D), dtype)
    total = int(seq_lens.sum())
    k_tok = _normal_bits(rng, (total, Hkv, D), dtype)
    v_tok = _normal_bits(rng, (total, Hkv, D), dtype)
    block_table, k_pages, v_pages = _scatter_pages(k_tok, v_tok, seq_lens, perm, num_pages,
                                                   page_size, max_pages_per_seq, dtype)
    return PagedInputs(q, k_pages, v_pages, block_table, seq_lens.astype(np.int32),
                       page_size, dtype, used)


@dataclass
class PagedVarlenInputs:
    q: np.ndarray             # uint16 bits [total_q, Hq, D]
    k_pages: np.ndarray       # uint16 bits [num_pages, page_size, Hkv, D]
    v_pages: np.ndarray
    block_table: np.ndarray   # int32 [B, max_pages_per_seq], -1 where unused
    seq_lens_k: np.ndarray    # int32 [B]: cached tokens, the new ones included
    cu_seqlens_q: np.ndarray  # int32 [B + 1]
    page_size: int
    dtype: str


def paged_varlen_inputs(Hq: int, Hkv: int, D: int, dtype: str, seed: int, *,
                        B: int | None = None, new_lo: int | None = None, new_hi: int | None = None,
                        ctx_lo: int | None = None, ctx_hi: int | None = None, seqlens_q=None,
                        ctx_lens=None, page_size: int = 16, max_pages_per_seq: int | None = None,
                        extra_pages: int = 0) -> PagedVarlenInputs:
    """Chunked prefill over a paged KV cache: each sequence has ``ctx_b`` earlier tokens
    cached and ``Lq_b`` new ones whose K/V are already appended, so ``Lk_b = ctx_b + Lq_b``
    and the queries are the last ``Lq_b`` positions (bottom-right alignment).

    Draw order: new-token counts (uniform in ``[new_lo, new_hi]`` unless ``seqlens_q``
    is given), context lengths (uniform in ``[ctx_lo, ctx_hi]`` unless ``ctx_lens``),
    the page permutation, Q ``[total_q, Hq, D]``, then the K tokens and the V tokens of
    every sequence in order.  Pages are dealt and filled as in ``paged_inputs``.
    """
    rng = np.random.default_rng(seed)
    if seqlens_q is None:
        seqlens_q = rng.integers(new_lo, new_hi, endpoint=True, size=B)
    seqlens_q = np.asarray(seqlens_q, dtype=np.int64)
    B = len(seqlens_q)
    if ctx_lens is None:
        ctx_lens = rng.integers(ctx_lo, ctx_hi, endpoint=True, size=B)
    lk = np.asarray(ctx_lens, dtype=np.int64) + seqlens_q
    pages_per_seq = [int(math.ceil(int(L) / page_size)) for L in lk]
    used = int(sum(pages_per_seq))
    num_pages = max(1, used + int(extra_pages))
    if max_pages_per_seq is None:
        max_pages_per_seq = max(1, max(pages_per_seq))
    if max(pages_per_seq) > max_pages_per_seq:
        raise ValueError("max_pages_per_seq too small for the drawn lengths")
    perm = rng.permutation(num_pages).astype(np.int64)
    cu_q = np.concatenate([[0], np.cumsum(seqlens_q)]).astype(np.int32)
    q = _normal_bits(rng, (int(cu_q[-1]), Hq, D), dtype)
    total_k = int(lk.sum())
    k_tok = _normal_bits(rng, (total_k, Hkv, D), dtype)
    v_tok = _normal_bits(rng, (total_k, Hkv, D), dtype)
    bt, kp, vp = _scatter_pages(k_tok, v_tok, lk, perm, num_pages, page_size, max_pages_per_seq,
                                dtype)
    return PagedVarlenInputs(q, kp, vp, bt, lk.astype(np.int32), cu_q, page_size, dtype)


@dataclass
class VarlenInputs:
    q: np.ndarray             # uint16 bits [total_q, Hq, D]
    k: np.ndarray             # uint16 bits [total_k, Hkv, D]
    v: np.ndarray             # uint16 bits [total_k, Hkv, D]
    cu_seqlens_q: np.ndarray  # int32 [B + 1]
    cu_seqlens_k: np.ndarray  # int32 [B + 1]
    dtype: str


def varlen_inputs(Hq: int, Hkv: int, D: int, dtype: str, seed: int, *, B: int | None = None,
                  len_lo: int | None = None, len_hi: int | None = None, seqlens_q=None,
                  seqlens_k=None, pad_q: int = 0, pad_k: int = 0) -> VarlenInputs:
    """Packed variable-length sequences (token-major ``[total, H, D]``).

    Draw order: the query lengths (uniform integers in ``[len_lo, len_hi]``, unless
    ``seqlens_q`` is given), then Q, K, V.  ``seqlens_k`` defaults to the query lengths
    (self-attention packing); giving longer key lengths models chunked prefill, where each
    sequence's new queries follow ``Lk_b - Lq_b`` earlier keys.  ``pad_q`` / ``pad_k`` extra
    tokens after the last sequence belong to no sequence and hold NaN.
    """
    rng = np.random.default_rng(seed)
    if seqlens_q is None:
        seqlens_q = rng.integers(len_lo, len_hi, endpoint=True, size=B)
    seqlens_q = np.asarray(seqlens_q, dtype=np.int64)
    seqlens_k = seqlens_q if seqlens_k is None else np.asarray(seqlens_k, dtype=np.int64)
    if seqlens_k.shape != seqlens_q.shape:
        raise ValueError("seqlens_q and seqlens_k differ in length")
    cu_q = np.concatenate([[0], np.cumsum(seqlens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(seqlens_k)]).astype(np.int32)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = _normal_bits(rng, (tq, Hq, D), dtype)
    k = _normal_bits(rng, (tk, Hkv, D), dtype)
    v = _normal_bits(rng, (tk, Hkv, D), dtype)
    if pad_q:
        q = np.concatenate([q, np.full((pad_q, Hq, D), NAN_BITS[dtype], np.uint16)])
    if pad_k:
        k = np.concatenate([k, np.full((pad_k, Hkv, D), NAN_BITS[dtype], np.uint16)])
        v = np.concatenate([v, np.full((pad_k, Hkv, D), NAN_BITS[dtype], np.uint16)])
    return VarlenInputs(q, k, v, cu_q, cu_k, dtype)


def block_mask_inputs(B: int, H: int, Nq: int, Nk: int, block_q: int, block_k: int,
                      density: float, seed: int, diagonal: bool = True) -> np.ndarray:
    """A seeded random block mask ``[B, H, ceil(Nq/block_q), ceil(Nk/block_k)]`` (uint8):
    each block is on with probability ``density`` (uniform draws in one call, after which
    the diagonal blocks are set when ``diagonal``)."""
    rng = np.random.default_rng(seed)
    nqb, nkb = -(-Nq // block_q), -(-Nk // block_k)
    bm = (rng.random((B, H, nqb, nkb)) < density).astype(np.uint8)
    if diagonal:
        d = np.arange(min(nqb, nkb))
        bm[:, :, d, d] = 1
    return bm


# The benchmark workloads, by name.  Shapes follow the mlx-mfa "Performance" table
# (B=2, H=8, f16, D=128, causal / window 512), its GQA statement (Hq a multiple of
# Hkv), and the MXFlashAttn paged split-KV decode setting (pages of 16 tokens,
# Hq=32, Hkv=8, D=128).
WORKLOADS = {
    "tiny_dense": dict(B=1, Hq=2, Hkv=2, Nq=128, Nk=128, D=64, dtype=F16, causal=False, left=-1,
                       right=-1, seed=101),
    "dense_causal_prefill": dict(B=2, Hq=8, Hkv=8, Nq=4096, Nk=4096, D=128, dtype=F16, causal=True,
                                 left=-1, right=-1, seed=102),
    "gqa_causal_long_prefill": dict(B=1, Hq=32, Hkv=8, Nq=16384, Nk=16384, D=128, dtype=BF16,
                                    causal=True, left=-1, right=-1, seed=103),
    "sliding_window_causal": dict(B=2, Hq=8, Hkv=8, Nq=8192, Nk=8192, D=128, dtype=F16, causal=True,
                                  left=512, right=0, seed=104),
    "paged_splitkv_decode": dict(B=16, Hq=32, Hkv=8, D=128, dtype=BF16, page_size=16, len_lo=1024,
                                 len_hi=32768, seed=105),
    # packed variable-length causal prefill (mlx-mfa "Variable-length" feature): a
    # serving-style mix of prompt lengths, GQA heads of the long-context workload
    "packed_varlen_causal_prefill": dict(B=16, Hq=32, Hkv=8, D=128, dtype=BF16, causal=True, left=-1,
                                         right=-1, len_lo=256, len_hi=4096, seed=106),
    # chunked prefill over the paged cache (the mlx-mfa 2.5.2 capability table: packed queries over paged keys):
    # new chunks of 512..2048 tokens after 1024..16384 cached ones, pages of 16
    "paged_chunked_prefill": dict(B=8, Hq=32, Hkv=8, D=128, dtype=BF16, causal=True, left=-1,
                                  right=-1, page_size=16, new_lo=512, new_hi=2048, ctx_lo=1024,
                                  ctx_hi=16384, seed=107),
    # speculative verification: 4 new tokens per sequence over the decode workload's cache
    "paged_multi_query_decode": dict(B=16, Nq=4, Hq=32, Hkv=8, D=128, dtype=BF16, page_size=16,
                                     len_lo=1024, len_hi=32768, seed=108),
    # block-sparse causal prefill (mlx-mfa "Block-sparse attention"): 128 x 128 blocks
    # on with probability 1/4, plus the diagonal
    "block_sparse_causal_prefill": dict(B=1, Hq=16, Hkv=16, Nq=16384, Nk=16384, D=128, dtype=F16,
                                        causal=True, left=-1, right=-1, block_q=128, block_k=128,
                                        density=0.25, seed=109),
    # training step after the prefill: the backward over the dense causal prefill shape,
    # in bf16 (the mlx-bun page's backward; upstream gradient from grad_inputs)
    "dense_causal_backward": dict(B=2, Hq=8, Hkv=8, Nq=4096, Nk=4096, D=128, dtype=BF16,
                                  causal=True, left=-1, right=-1, seed=110),
}


def workload(name: str) -> dict:
    """The named workload's parameters (a copy), with name and scale = 1 / sqrt(D)."""
    c = dict(WORKLOADS[name])
    c["name"] = name
    c["scale"] = 1.0 / math.sqrt(c["D"])
    return c


def workload_inputs(name: str):
    """The named workload's seeded inputs (the generator its layout calls for)."""
    c = workload(name)
    if name == "paged_multi_query_decode":
        return paged_multi_inputs(c["B"], c["Nq"], c["Hq"], c["Hkv"], c["D"], c["dtype"], c["seed"],
                                  len_lo=c["len_lo"], len_hi=c["len_hi"], page_size=c["page_size"])
    if name == "paged_chunked_prefill":
        return paged_varlen_inputs(c["Hq"], c["Hkv"], c["D"], c["dtype"], c["seed"], B=c["B"],
                                   new_lo=c["new_lo"], new_hi=c["new_hi"], ctx_lo=c["ctx_lo"],
                                   ctx_hi=c["ctx_hi"], page_size=c["page_size"])
    if name == "packed_varlen_causal_prefill":
        return varlen_inputs(c["Hq"], c["Hkv"], c["D"], c["dtype"], c["seed"], B=c["B"],
                             len_lo=c["len_lo"], len_hi=c["len_hi"])
    if name in ("paged_splitkv_decode",):
        return paged_inputs(c["B"], c["Hq"], c["Hkv"], c["D"], c["dtype"], c["seed"],
                            len_lo=c["len_lo"], len_hi=c["len_hi"],
                            page_size=c["page_size"])
    return dense_inputs(c["B"], c["Hq"], c["Hkv"], c["Nq"], c["Nk"], c["D"], c["dtype"],
                        c["seed"])
