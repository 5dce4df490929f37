/*
 * mfa.h — C ABI of the MI355X (gfx950) fused exact-attention library, libmfa.so.
 *
 * Exact attention O = softmax(scale * Q K^T + mask) V with an fp32 online softmax that
 * never materialises the score matrix:
 *
 *   mfa_fwd           tiled forward (prefill) with causal / sliding-window key-tile
 *                     skipping and grouped-query head mapping; writes O and the row
 *                     log-sum-exp.  Defined by the FlashAttention-2 forward shader of
 *                     the mlx-bun flash-attention.ts page (online softmax with running
 *                     max m and sum l in fp32, O = o / l, LSE = m + log l) and the
 *                     mlx-mfa 2.5.2 page's feature list ("Causal tile-skip",
 *                     "Sliding window", "Native GQA").
 *   mfa_fwd_ext       the same with softcap, ALiBi, an additive key bias and a
 *                     block-sparse mask (mlx-mfa "Softcap", "ALiBi", "Block-sparse").
 *   mfa_bwd           the backward pass of mfa_fwd (dQ, dK, dV from the saved LSE).
 *   mfa_fwd_varlen    the same forward over packed sequences of different lengths
 *                     delimited by cu_seqlens (mlx-mfa "Variable-length"), each
 *                     sequence masked on its own lengths.
 *   mfa_fwd_varlen_paged  packed queries whose keys sit in a paged KV cache (chunked
 *                     prefill; mlx-mfa 2.5.2 capability table, packed queries over paged keys).
 *   mfa_decode_paged_multi  the same for Nq <= 4 new tokens per sequence (speculative
 *                     verification), with the query rows of a KV head packed together.
 *   mfa_decode_paged  single-query decode over a paged KV cache, split across
 *                     workgroups along the keys, with partial (O, LSE) pairs merged in
 *                     a second pass.  Defined by the mlx-mfa 2.5.2 page (the "Flash Decode"
 *                     feature, a split-KV decode in two phases, and the "Paged KV"
 *                     feature, a pool of pages addressed through a block table) and
 *                     the MXFlashAttn 1.5.0 page (M1 paged Split-KV
 *                     decode; the per-split (m, l) slot race section).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensors are caller-owned, contiguous, 16-byte aligned device memory.  The
 *   library allocates no device memory; the decode and backward workspaces are passed in.
 * - Element type: 16-bit storage, MFA_F16 (IEEE half) or MFA_BF16 (bfloat16), the
 *   same for Q, K, V and O.  LSE is float32.  All arithmetic accumulates in fp32.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 *   call returns without synchronising.  A call issues kernel launches only (no
 *   allocation, memset or synchronisation), so it may be captured in a HIP graph; a
 *   replay reads whatever the captured buffers hold at that time.
 * - Arguments are validated before anything is launched; on failure a negative
 *   mfa_status is returned and nothing is written.  There is no fallback path.
 * - Visibility (mlx-mfa "Sliding window" feature, window_size=(left, right), -1 =
 *   unbounded; causal mask of the mlx-bun forward shader), with off = Nk - Nq
 *   (bottom-right alignment) and both window ends inclusive: key j is visible to
 *   query i iff
 *       (!causal || j <= i + off) && (left < 0 || j >= i + off - left)
 *                                 && (right < 0 || j <= i + off + right).
 *   A row with no visible key gets O = 0 and LSE = -inf.
 * - Grouped-query attention: query head h reads KV head h / (Hq / Hkv) (mlx-bun
 *   forward shader head mapping); Hq must be a multiple of Hkv.
 * - Thread safety: calls may be made from several host threads; the dispatch record
 *   returned by mfa_last_dispatch is per host thread.
 */
#ifndef MFA_H
#define MFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MFA_F16 = 0, MFA_BF16 = 1 } mfa_dtype;

typedef enum {
    MFA_OK = 0,
    MFA_ERR_NULL = -1,      /* a required pointer is NULL */
    MFA_ERR_SHAPE = -2,     /* a size is < 1 (or inconsistent) */
    MFA_ERR_GQA = -3,       /* Hq is not a multiple of Hkv */
    MFA_ERR_HEAD_DIM = -4,  /* D not in {64, 128} */
    MFA_ERR_DTYPE = -5,     /* dtype not MFA_F16 / MFA_BF16 */
    MFA_ERR_WINDOW = -6,    /* win_left or win_right < -1 */
    MFA_ERR_SCALE = -7,     /* scale is not finite */
    MFA_ERR_WORKSPACE = -8, /* decode workspace NULL or too small */
    MFA_ERR_PAGED = -9,     /* page_size != 16, num_pages or max_pages_per_seq < 1 */
    MFA_ERR_OVERFLOW = -10, /* sizes exceed the 64-bit element / launch-grid limits */
    MFA_ERR_HIP = -11,      /* the HIP runtime reported an error at launch */
    MFA_ERR_ALIGN = -12,    /* a tensor pointer is not 16-byte aligned */
    MFA_ERR_ARG = -13       /* other invalid argument (e.g. num_splits < 0) */
} mfa_status;

/* Tile plan of the forward kernel for one (batch, head): host-only, launches nothing.
 * Defined by the causal tile-skip and sliding-window features of the mlx-mfa 2.5.2
 * page: only key tiles holding at least one visible (query, key) pair are visited,
 * and only tiles crossing the mask boundary are masked element-wise. */
typedef struct {
    int BM;               /* query rows per workgroup (one query tile) */
    int BN;               /* keys per key tile */
    int waves;            /* wavefronts (64 lanes) per wave group: one group covers the
                             BM query rows of a tile.  mfa_fwd runs one or two groups per
                             workgroup, chosen at launch from the grid size (with two, the
                             groups split the tile's key range, or on large dense GQA
                             grids take the same tile of two query heads that share a KV
                             head); mfa_last_dispatch reports the workgroup actually
                             launched */
    int n_q_tiles;        /* ceil(Nq / BM) */
    int n_k_tiles;        /* ceil(Nk / BN) */
    long long visited;    /* key tiles visited, summed over the query tiles */
    long long edge;       /* of which are masked element-wise */
} mfa_plan;

/* Fill *plan for the given problem.  If kt_range is not NULL it must hold
 * 2 * n_q_tiles ints (pass its capacity in kt_range_len); on return kt_range[2t] and
 * kt_range[2t+1] are the half-open key-tile range [lo, hi) visited by query tile t
 * (lo == hi when the tile sees no key).  Returns MFA_OK or a validation error; if
 * kt_range_len is too small, MFA_ERR_ARG with *plan still filled. */
int mfa_plan_fwd(int Nq, int Nk, int D, int dtype, int causal, int win_left, int win_right,
                 mfa_plan* plan, int32_t* kt_range, long long kt_range_len);

/* Forward pass.
 *   q    [B, Hq,  Nq, D]  dtype          k, v  [B, Hkv, Nk, D]  dtype
 *   out  [B, Hq,  Nq, D]  dtype (written, rounded to nearest even from fp32)
 *   lse  [B, Hq,  Nq]     float32, natural log of the sum of exp of the scaled
 *                         visible scores; may be NULL
 *   scale multiplies Q K^T before masking (finite; no default is applied)
 *   causal (0/1), win_left / win_right >= -1 (-1 = unbounded)
 * Errors: MFA_ERR_NULL, _DTYPE, _HEAD_DIM, _SHAPE, _GQA, _WINDOW, _SCALE, _ALIGN,
 * _OVERFLOW, _HIP. */
int mfa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
            int B, int Hq, int Hkv, int Nq, int Nk, int D, float scale,
            int causal, int win_left, int win_right, int dtype, void* stream);

/* Same as mfa_fwd, and additionally records, for every (b, h, query tile), four int32
 * values in tile_log[((b * Hq + h) * n_q_tiles + t) * 4 + {0,1,2,3}]:
 *   first key tile visited (or -1), number of key tiles visited, number of those
 *   masked element-wise, one past the last key tile visited (or -1).
 * tile_log is device memory of B * Hq * n_q_tiles * 4 int32 (n_q_tiles from
 * mfa_plan_fwd).  Used to check that the kernel visits exactly the planned tiles. */
int mfa_fwd_tilelog(const void* q, const void* k, const void* v, void* out, float* lse,
                    int B, int Hq, int Hkv, int Nq, int Nk, int D, float scale,
                    int causal, int win_left, int win_right, int dtype, void* stream,
                    int32_t* tile_log);

/* Score modifiers and block-sparse mask for mfa_fwd_ext (mlx-mfa 2.5.2 feature list:
 * the "Softcap", "ALiBi" and "Block-sparse attention" features, i.e. a tanh cap on the
 * scores inside the kernel, a linear distance penalty per head, and a mask of blocks whose
 * tiles are skipped; mlx-mfa 2.61.0 "Native attn_bias" feature, an additive bias on the
 * logits, per key and per head per key).  With
 * off = Nk - Nq the score of query i and key j of head h in batch b is, in this order:
 *   s = scale * q_i . k_j
 *   s = softcap * tanh(s / softcap)                         if softcap > 0
 *   s = s - alibi_slopes[h] * |i + off - j|                 if alibi_slopes != NULL
 *   s = s + bias[b * bias_stride_b + h * bias_stride_h + j]  if bias != NULL
 * then keys outside the causal / window rule, and keys in a block with
 *   block_mask[b * mask_stride_b + h * mask_stride_h + (i / block_q) * mask_k_blocks
 *              + j / block_k] == 0
 * are removed before the softmax; whole key tiles with no computed block are skipped.
 * All pointers are device memory (NULL = feature off); strides are in elements (0
 * broadcasts over batch or head). */
typedef struct {
    float softcap;                 /* 0 = off, else > 0 and finite */
    const float* alibi_slopes;     /* [Hq] float32 or NULL */
    const float* bias;             /* float32, keys contiguous, or NULL */
    long long bias_stride_b, bias_stride_h;
    const uint8_t* block_mask;     /* uint8 (0 = skip) or NULL */
    long long mask_stride_b, mask_stride_h;
    int mask_q_blocks;             /* >= ceil(Nq / block_q) rows of key blocks per (b, h) */
    int mask_k_blocks;             /* >= ceil(Nk / block_k) key blocks per row */
    int block_q, block_k;          /* positive multiples of 32 */
    int32_t* tile_log;             /* optional per-tile record, as for mfa_fwd_tilelog */
} mfa_fwd_ext_args;

/* Dense forward (layouts and conventions of mfa_fwd) with the modifiers of *ext.  The
 * tile record (ext->tile_log) lists, per (b, h, query tile), the first visited key tile,
 * the number visited, how many were masked element-wise and one past the last visited.
 * With a block mask, Nk must be at most 131072 (2048 key tiles per query tile) and
 * mfa_last_dispatch reports planned = -1.
 * Errors: those of mfa_fwd, plus MFA_ERR_NULL (ext NULL), MFA_ERR_ARG (softcap < 0 or
 * not finite, block sizes not positive multiples of 32, mask dimensions too small,
 * negative strides), MFA_ERR_OVERFLOW (Nk too large for a block mask). */
int mfa_fwd_ext(const void* q, const void* k, const void* v, void* out, float* lse,
                int B, int Hq, int Hkv, int Nq, int Nk, int D, float scale,
                int causal, int win_left, int win_right, const mfa_fwd_ext_args* ext,
                int dtype, void* stream);

/* Forward pass over packed variable-length sequences (mlx-mfa 2.5.2 feature list:
 * "Variable-length", packed sequences delimited by cu_seqlens; the page's note that
 * the causal varlen output for N_q < N_k was corrected).  Each sequence is attended on
 * its own, with the visibility rule above applied to its own lengths: for sequence b,
 * Nq = Lq_b, Nk = Lk_b and off = Lk_b - Lq_b (bottom-right), so a chunk of Lq_b new
 * queries after Lk_b - Lq_b earlier keys (chunked prefill) sees all of them.
 *   q    [total_q, Hq,  D]  dtype   token-major: sequence b owns tokens
 *                                   cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1
 *   k, v [total_k, Hkv, D]  dtype   sequence b owns cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1
 *   out  [total_q, Hq,  D]  dtype   rows of tokens outside every sequence are not written
 *   lse  [Hq, total_q]      float32 or NULL (natural log, as for mfa_fwd)
 *   cu_seqlens_q, cu_seqlens_k: int32 [B + 1] device memory, read by the kernel
 *   max_seqlen_q, max_seqlen_k: host upper bounds of Lq_b and Lk_b (they size the grid)
 * Device-side contract (the offsets stay on the device and are not checked on the
 * host): both arrays are non-decreasing, start at >= 0 and end at <= total_q / total_k,
 * and Lq_b <= max_seqlen_q, Lk_b <= max_seqlen_k.  Out of contract the kernel stays in
 * bounds (offsets are clamped into the tensors and lengths to the maxima) but the result
 * is unspecified.  Lq_b = 0 writes nothing; Lq_b > 0 with Lk_b = 0 gives O = 0 and
 * LSE = -inf on those rows.  mfa_last_dispatch reports planned = -1 (lengths unknown
 * on the host).
 * Errors: MFA_ERR_NULL, _DTYPE, _HEAD_DIM, _SHAPE, _GQA, _WINDOW, _SCALE, _ALIGN, _ARG,
 * _OVERFLOW, _HIP. */
int mfa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                   int B, int Hq, int Hkv, int total_q, int total_k,
                   int max_seqlen_q, int max_seqlen_k, int D, float scale,
                   int causal, int win_left, int win_right, int dtype, void* stream);

/* mfa_fwd_varlen plus the per-tile visit record of mfa_fwd_tilelog, indexed by
 * (b, h, query tile t) with n_q_tiles = ceil(max_seqlen_q / BM); tiles past a
 * sequence's end record (-1, 0, 0, -1). */
int mfa_fwd_varlen_tilelog(const void* q, const void* k, const void* v, void* out, float* lse,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int B, int Hq, int Hkv, int total_q, int total_k,
                           int max_seqlen_q, int max_seqlen_k, int D, float scale,
                           int causal, int win_left, int win_right, int dtype, void* stream,
                           int32_t* tile_log);

/* Packed queries over a paged KV cache: chunked prefill and speculative or
 * multi-token verification (mlx-mfa 2.5.2 capability table, packed variable-length
 * queries over paged keys; the paged-cache addressing of mfa_decode_paged).  Sequence b has
 * Lq_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] new query tokens and Lk_b = seq_lens_k[b]
 * cached keys, which include the new tokens' own keys (appended before the call); the
 * visibility rule applies with Nq = Lq_b, Nk = Lk_b, off = Lk_b - Lq_b, so the queries
 * are the last Lq_b positions of the sequence.
 *   q            [total_q, Hq, D]                    dtype (token-major, as mfa_fwd_varlen)
 *   k_pages      [num_pages, page_size, Hkv, D]      dtype
 *   v_pages      [num_pages, page_size, Hkv, D]      dtype
 *   block_table  [B, max_pages_per_seq] int32 (device): token t of sequence b lives in
 *                page block_table[b, t / page_size], slot t % page_size
 *   seq_lens_k   [B] int32 (device)
 *   cu_seqlens_q [B + 1] int32 (device)
 *   out          [total_q, Hq, D] dtype;  lse [Hq, total_q] float32 or NULL
 *   max_seqlen_q, max_seqlen_k: host upper bounds of Lq_b and Lk_b (they size the grid)
 *   page_size must be 16.
 * Device-side contract: cu_seqlens_q as for mfa_fwd_varlen (Lq_b <= max_seqlen_q);
 * 0 <= seq_lens_k[b] <= min(max_seqlen_k, max_pages_per_seq * page_size); the first
 * ceil(seq_lens_k[b] / page_size) entries of row b of block_table are valid page
 * indices.  Out of contract the kernel stays in bounds (offsets and lengths are clamped,
 * pages outside [0, num_pages) read as zeros) but the result is unspecified.  Slots
 * past seq_lens_k[b] are never used, whatever they hold.
 * Errors: MFA_ERR_NULL, _DTYPE, _HEAD_DIM, _SHAPE, _GQA, _WINDOW, _SCALE, _PAGED, _ALIGN,
 * _ARG, _OVERFLOW, _HIP. */
int mfa_fwd_varlen_paged(const void* q, const void* k_pages, const void* v_pages,
                         const int32_t* block_table, const int32_t* seq_lens_k,
                         const int32_t* cu_seqlens_q, void* out, float* lse,
                         int B, int Hq, int Hkv, int total_q, int max_seqlen_q,
                         int max_seqlen_k, int D, int page_size, int num_pages,
                         int max_pages_per_seq, float scale,
                         int causal, int win_left, int win_right, int dtype, void* stream);

/* Bytes of workspace mfa_bwd needs (0 if an argument is < 1). */
size_t mfa_bwd_workspace_bytes(int B, int Hq, int Nq);

/* Backward pass of mfa_fwd: the gradients of O with respect to Q, K and V for an
 * upstream gradient dO (the FlashAttention-2 backward of the mlx-bun flash-attention.ts
 * page: D-vector, dK/dV and dQ passes recomputing P from the saved LSE; here the D-vector
 * is formed inside the dQ pass, which runs first).  With P the
 * forward's probabilities (masked keys have P = 0):
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_d dO_id O_id,  dS = P * (dP - D),
 *   dQ = scale dS K,  dK = scale dS^T Q,
 * and with grouped query heads dK, dV of a KV head sum over its Hq / Hkv query heads.
 *   q, out, dout, dq  [B, Hq, Nq, D] dtype     k, v, dk, dv  [B, Hkv, Nk, D] dtype
 *   lse               [B, Hq, Nq] float32 as written by mfa_fwd for the same arguments
 *   scale, causal, win_left, win_right: as passed to mfa_fwd
 *   workspace         at least mfa_bwd_workspace_bytes(B, Hq, Nq) bytes of device memory
 *                     (contents on entry do not matter)
 * dq, dk, dv are written in full (zeros where no visible pair contributes), rounded to
 * nearest even from fp32 accumulation.  The result is deterministic: no atomics.
 * Errors: those of mfa_fwd, plus MFA_ERR_WORKSPACE. */
int mfa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
            const float* lse, void* dq, void* dk, void* dv, void* workspace,
            size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int D, float scale,
            int causal, int win_left, int win_right, int dtype, void* stream);

/* Bytes of workspace mfa_decode_paged needs for these sizes (num_splits 0 = auto).
 * The workspace holds the per-split partial results of the split-KV decode: one slot per
 * (sequence, query head, split), each D fp32 partial outputs plus one fp32 log-sum-exp,
 * i.e. B * Hq * S * (D + 1) * 4 bytes with S = mfa_decode_num_splits(...).  This follows
 * the MXFlashAttn 1.5.0 page: its split-KV decode keeps one (m, l) slot per split and
 * merges them in a second pass (section on the non-deterministic out-of-bounds write in
 * the split-KV scratch slots), and its roadmap names the scratch lifetime under graph
 * capture as an open problem, which is why the caller owns this memory here.
 * Returns 0 if the arguments are invalid (B, Hq < 1, D not 64 / 128, page_size != 16,
 * max_pages_per_seq < 1 or num_splits < 0); never allocates. */
size_t mfa_decode_workspace_bytes(int B, int Hq, int D, int page_size, int max_pages_per_seq,
                                  int num_splits);

/* Number of key splits mfa_decode_paged will use (num_splits 0 = auto), or a negative
 * status if the arguments are invalid. */
int mfa_decode_num_splits(int page_size, int max_pages_per_seq, int num_splits);

/* Paged split-KV decode: one new query token per sequence.
 *   q            [B, Hq, D]                          dtype
 *   k_pages      [num_pages, page_size, Hkv, D]      dtype   (pool of KV pages)
 *   v_pages      [num_pages, page_size, Hkv, D]      dtype
 *   block_table  [B, max_pages_per_seq] int32: token t of sequence b lives in page
 *                block_table[b, t / page_size], slot t % page_size
 *   seq_lens     [B] int32, device memory: cached tokens of each sequence, all visible
 *   out          [B, Hq, D] dtype;  lse [B, Hq] float32 or NULL
 *   page_size must be 16.  num_splits: 0 = auto, else an upper bound on the number of
 *   key splits; splits are contiguous ranges of logical token positions, so the result
 *   does not depend on where the pages sit in the pool.
 *   workspace: device memory of at least mfa_decode_workspace_bytes(...) bytes, holding
 *   the per-split partial (O, LSE); its contents on entry do not matter.
 * Device-side contract (seq_lens stays on the device and is not checked on the host):
 *   0 <= seq_lens[b] <= max_pages_per_seq * page_size and the first
 *   ceil(seq_lens[b] / page_size) entries of row b of block_table are valid page
 *   indices.  Out of contract, the kernels stay in bounds (lengths are clamped to the
 *   capacity and invalid page indices are skipped) but the result is unspecified.
 *   Tokens past seq_lens[b] are never used, whatever they hold.  seq_lens[b] == 0
 *   gives O = 0 and LSE = -inf.
 * Errors: MFA_ERR_NULL, _DTYPE, _HEAD_DIM, _SHAPE, _GQA, _PAGED, _SCALE, _ALIGN,
 * _WORKSPACE, _ARG, _OVERFLOW, _HIP. */
int mfa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                     const int32_t* block_table, const int32_t* seq_lens,
                     void* out, float* lse,
                     int B, int Hq, int Hkv, int D, int page_size, int num_pages,
                     int max_pages_per_seq, float scale, int num_splits,
                     void* workspace, size_t workspace_bytes, int dtype, void* stream);

/* mfa_decode_paged without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The split partials live in a fixed scratch array inside the library, one
 * per GPU, 32 MiB (33,554,432 bytes), held until the process ends; the call itself
 * allocates nothing.  Arguments, layouts, device-side contract and results are those of
 * mfa_decode_paged with the same num_splits (the same kernels run).
 * Limit: the partials take mfa_decode_workspace_bytes(B, Hq, D, page_size,
 * max_pages_per_seq, num_splits) bytes; above 32 MiB the call returns MFA_ERR_WORKSPACE
 * (pass a smaller num_splits, or use mfa_decode_paged with a workspace of that size).
 * Every call on one GPU uses that GPU's one scratch array: calls that overlap in time on
 * the same GPU (concurrent streams or host threads) race and must be serialised by the
 * caller.  Nothing in the scratch needs clearing between calls.
 * Errors: those of mfa_decode_paged; MFA_ERR_HIP also if the scratch address cannot be
 * obtained. */
int mfa_decode_paged_noalloc(const void* q, const void* k_pages, const void* v_pages,
                             const int32_t* block_table, const int32_t* seq_lens,
                             void* out, float* lse,
                             int B, int Hq, int Hkv, int D, int page_size, int num_pages,
                             int max_pages_per_seq, float scale, int num_splits, int dtype,
                             void* stream);

/* Bytes of workspace mfa_decode_paged_multi needs: B * Nq * Hq * S * (D + 1) * 4, with S the
 * number of key splits it uses for these sizes (0 if the arguments are invalid). */
size_t mfa_decode_multi_workspace_bytes(int B, int Nq, int Hq, int D, int page_size,
                                        int max_pages_per_seq, int num_splits);

/* Paged split-KV decode of Nq <= 4 new tokens per sequence, e.g. the verification step of
 * speculative decoding (mlx-mfa 2.5.2 feature list: the "Flash Decode" feature, a split-KV
 * decode in two phases for up to four query tokens; the packed-GQA verify kernel of the
 * MTPLX verify-attention page).  The new
 * tokens' keys are already in the cache: they are its last Nq positions, and new token n
 * sees the keys at positions <= seq_lens[b] - Nq + n (the visibility rule above with
 * Nk = seq_lens[b], causal).  The g * Nq query rows of one KV head are computed together.
 *   q    [B, Nq, Hq, D] dtype        out [B, Nq, Hq, D] dtype    lse [B, Nq, Hq] float32 or NULL
 *   k_pages, v_pages, block_table, seq_lens, page_size, num_pages, max_pages_per_seq,
 *   num_splits: as for mfa_decode_paged, with the same device-side contract; the automatic
 *   split count (num_splits 0) is lower than mfa_decode_paged's when Nq > 1 (longer
 *   chunks, since each split's partials are Nq times larger).
 *   workspace: at least mfa_decode_multi_workspace_bytes(...) bytes of device memory.
 * A row with no visible key (seq_lens[b] < Nq - n) gets O = 0 and LSE = -inf.
 * Errors: MFA_ERR_NULL, _DTYPE, _HEAD_DIM, _SHAPE (also Nq outside 1..4), _GQA, _PAGED,
 * _SCALE, _ALIGN, _WORKSPACE, _ARG, _OVERFLOW, _HIP. */
int mfa_decode_paged_multi(const void* q, const void* k_pages, const void* v_pages,
                           const int32_t* block_table, const int32_t* seq_lens,
                           void* out, float* lse,
                           int B, int Nq, int Hq, int Hkv, int D, int page_size, int num_pages,
                           int max_pages_per_seq, float scale, int num_splits,
                           void* workspace, size_t workspace_bytes, int dtype, void* stream);

/* What the last successful launch on this host thread ran (MXFlashAttn's per-dispatch
 * record: backend, operation, selection and split fields). */
typedef struct {
    char kernel[96];      /* kernel name of the main launch; forward names end with the
                             workgroup layout and order: groups=1|2, then ",chained"
                             (two complementary query tiles per workgroup), ",head-pairs",
                             ",seq-major" (packed sequences) or ",head-major" (dense),
                             when taken */
    int op;               /* 1 = forward, 2 = paged decode, 3 = packed varlen forward,
                             4 = packed queries over a paged cache, 5 = multi-token decode,
                             6 = forward with modifiers / block mask, 7 = backward */
    int BM, BN, waves;    /* forward tile configuration */
    int grid[3];          /* main launch grid */
    int block;            /* threads per workgroup */
    int num_splits;       /* decode: key splits (grid.x of the split kernel) */
    int chunk_tokens;     /* decode: logical tokens per split */
    long long planned;    /* forward: key tiles visited over all (b, h); varlen, paged: -1;
                             decode: 0 */
    int n_launches;       /* kernels enqueued by the call */
} mfa_dispatch_info;

/* Copy the calling thread's last dispatch record; MFA_ERR_NULL if out is NULL,
 * MFA_ERR_ARG if this thread has launched nothing yet. */
int mfa_last_dispatch(mfa_dispatch_info* out);

/* Static description of a status code ("unknown status" for a value that is not an
 * mfa_status).  The status codes follow the mlx-mfa 2.61.0 README: the raw native
 * entries carry the same guards as the Python wrappers (release notes), malformed inputs
 * are rejected before dispatch rather than returning silent wrong or NaN output
 * (input-validation contract), and a disabled fast path reports a reason code instead
 * of falling back silently ("Verify acceleration is active").  The string is static,
 * owned by the library; it must not be freed. */
const char* mfa_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int mfa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MFA_H */
