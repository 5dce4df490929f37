"""CPU oracle for exact attention — TEST INFRASTRUCTURE, not part of the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The HIP library never calls it,
and the oracle imports nothing from the HIP path (the two share no code; only the
seeded generators of ``attn_inputs`` serve both).

It computes, in float64 and by the plain definition, what the fused kernels compute
tile by tile:

* ``attention``: softmax(scale * Q K^T + mask) V and the row log-sum-exp, with
  causal and (left, right) window visibility and grouped-query head mapping.  This
  is the materialised form of the forward pass (mlx-bun ``flash-attention.ts``:
  the ``manualSdpa`` reference and the forward shader's online softmax, which
  reaches the same result up to rounding).
* ``attention_backward``: the gradients dQ, dK, dV of ``attention`` for an upstream
  gradient dO (mlx-bun backward: D-vector, dK/dV and dQ passes).
* ``attention_ext``: the same with softcap, ALiBi, an additive per-key bias and a
  block-sparse mask (mlx-mfa "Softcap", "ALiBi", "Block-sparse attention", "attn_bias").
* ``attention_varlen``: the same for sequences of different lengths packed along the
  token axis and delimited by ``cu_seqlens`` (mlx-mfa "Variable-length" feature),
  each sequence on its own with bottom-right alignment.
* ``attention_varlen_paged``: packed queries whose keys come from a paged KV cache
  (chunked prefill; mlx-mfa 2.5.2 capability table, packed queries over paged keys).
* ``decode_paged``: single-query attention over a paged KV cache, gathered through
  the block table with its own loop (MXFlashAttn paged Split-KV decode; mlx-mfa
  "Paged KV" feature).
* ``decode_paged_multi``: decode of up to a few new tokens per sequence (speculative
  verification), causal among the new tokens (mlx-mfa 2.5.2 "Flash Decode" feature, up to four
  new tokens).
* ``lse_merge``: the combination of partial (O, LSE) pairs that a split-KV decode's
  second pass performs (mlx-mfa 2.5.2 "Flash Decode" feature: split-KV in two phases).
* ``visited_tiles``: the brute-force set of key tiles holding at least one visible
  (query, key) pair for each query tile (mlx-mfa "Causal tile-skip" and "Sliding
  window" features).

Every function is pinned by tests in ``tests/test_oracle_*.py`` against closed
forms, invariants, a pure-Python scalar implementation (``oracle.scalar``) and
PyTorch's float64 CPU attention routine.  No function here is "parity unpinned".
"""
from .reference import (attention, attention_backward, attention_ext, attention_probs,
                        attention_varlen,
                        attention_varlen_paged,
                        decode_paged, decode_paged_multi, gather_paged, lse_merge, visible,
                        visited_tiles, widen, window_bounds)

__all__ = ["attention", "attention_backward", "attention_ext", "attention_probs", "attention_varlen", "attention_varlen_paged",
           "decode_paged", "decode_paged_multi", "gather_paged", "lse_merge", "visible",
           "visited_tiles", "widen", "window_bounds"]
