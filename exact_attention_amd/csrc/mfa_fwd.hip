// Fused exact-attention forward for gfx950.
//
// Computes O = softmax(scale * Q K^T + mask) V and LSE = log(sum exp(scaled scores))
// tile by tile with an fp32 online softmax (running max m and sum l per query row),
// as in the FlashAttention-2 forward shader of the mlx-bun flash-attention.ts page:
// per key tile, m' = max(m, rowmax S); alpha = exp(m - m'); P = exp(S - m');
// l = alpha * l + rowsum P; O = alpha * O + P V; at the end O / l and m + log l.
// That shader runs one thread per query row with scalar dot products; here both
// contractions run on the CDNA4 matrix cores and the loop is software-pipelined.
//
// Work decomposition
//   A query tile is BM = 128 rows of one (batch, head); a group of 4 waves covers it,
//   each wave owning 32 rows.  Large grids use one group per workgroup, two workgroups
//   per CU, which overlap each other's prologue and epilogue; longest tiles go first.
//   Small grids (at most two tiles per CU) use 8-wave workgroups whose two groups split
//   the tile's visited key range in halves, run concurrently (two waves per SIMD) and
//   merge their (O, m, l) through LDS at the end; for dense inputs with an even number
//   of query tiles such a workgroup then runs a second, complementary tile (T - 1 - r
//   after r), so every workgroup has the same causal work.  Large dense GQA grids with an
//   even group size use 8-wave workgroups too, whose two groups take the same tile of two
//   query heads that share a KV head, over one K/V stream.  Key tiles of BN = 64 keys
//   stream through LDS: K and V tiles are copied global -> LDS directly (buffer loads
//   with the LDS bit; the range check returns zeros past the last key row),
//   double-buffered per group.  Workgroups are ordered so that those reading one KV
//   head's K/V run on one XCD and share its L2: the query heads of a KV head on one XCD,
//   and with Hkv a multiple of 8 whole KV heads per XCD, run head by head (dense layouts)
//   or sequence by sequence (packed sequences).  O leaves through LDS as whole rows.
//
// Per wave and key tile (32x32x16 MFMA, fp32 accumulate):
//   S^T = K Q^T: A = K rows (keys) from LDS, B = Q^T held in registers for the whole
//     kernel.  The accumulator puts one query row in each lane (lane % 32) and 16 of
//     the 32 keys of a block in its registers, so the row max needs one exchange with
//     lane ^ 32 and the row sum none until the end.
//   The K rows fed to the A operand are permuted (key_perm) so that accumulator
//   register r of lane half g holds key 16*(r/8) + 8*g + r%8: each lane then owns runs
//   of 8 consecutive keys, which is exactly the B operand layout of the next product.
//   O^T += V^T P^T: A = V^T read from the row-major V tile with the gfx950 transposing
//     LDS read (ds_read_b64_tr_b16: 16 lanes read a 4-key x 16-column block and each
//     receives one column), B = P^T straight from the softmax registers (rounded to
//     the input type).  The O^T accumulator again has one query row per lane.
//
// Pipeline (iteration j, with S(j) already computed):
//   the direct loads of K(j+2) and V(j+1), spread over the stage;
//   row max of S(j) (raise the exponent offset if needed, rescale O and l);
//   the 16 MFMAs of S(j+1) = K(j+1) Q^T interleaved with the exponentials of S(j);
//   the 16 MFMAs of O += V(j)^T P(j)^T;  wait for the loads;  one barrier.
//   So the matrix cores work on tile j+1 while the vector ALUs finish tile j.
//
// Softmax details (log2 domain; scale * log2(e) is folded into one FMA that feeds
// the exponential):
//   * The exponent offset is only raised when a row's new maximum exceeds it by more
//     than 2^8 (kLazy), so P <= 256 and O, l are rescaled only on those (rare) tiles;
//     the offset cancels in O = o / l and enters LSE as m + log2 l.
//   * For fp16, l accumulates the P values after rounding to fp16 (one dot2 per pair),
//     i.e. exactly the weights the P V product uses; for bf16, whose rounding is 8x
//     coarser, l sums the fp32 values so that the LSE keeps fp32 accuracy.
//
// Masking and skipping (mlx-mfa 2.5.2 features "Causal tile-skip", "Sliding window";
// mlx-bun forward shader's fully-masked-tile guard): the workgroup visits only the key
// tiles of mfa_tile_range; element masks are applied only on tiles that
// mfa_tile_full rejects (the invisible scores become -inf, so exp2 gives P = 0); a
// row whose offset is still -inf uses 0 in its place so exp never sees
// (-inf) - (-inf).
#include <algorithm>

#include "mfa_device.h"
#include "mfa_geometry.h"
#include "mfa_internal.h"
#include "mfa_tile.h"

namespace {

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kGroupThreads = 256;   // one wave group: 4 waves x 32 query rows
constexpr float kLazy = 8.0f;

struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int32_t* tile_log;
    int B, Hq, Hkv, Nq, Nk, g;   // packed sequences: Nq, Nk = max_seqlen_q, max_seqlen_k
    int n_q_tiles;   // query tiles per (batch, head) (of max_seqlen_q for packed sequences)
    int n_rounds;    // grid = n_rounds * HB
    int HB;          // B * Hq
    int xcd_group;   // 1: group the query heads of one KV head on one XCD
    int chain;       // 1: each workgroup runs query tile n_q_tiles - 1 - r, then tile r
    int seqmajor;    // 1: packed sequences in sequence-major order per XCD (seq_major_item)
    int grid;        // workgroups of the launch
    int pair;        // 1: the two wave groups take two query heads of one KV head
    float scale_log2_abs;  // |scale| * log2(e)
    MfaMask mask;    // dense layout only (packed sequences build theirs per sequence)
    // packed sequences ([total, H, D] token-major, delimited by cu_seqlens)
    const int32_t* cu_q;
    const int32_t* cu_k;
    int total_q, total_k;
    int causal, left, right;
    // keys in a paged cache ([num_pages, 16, Hkv, D] pools, block_table [B, max_pages],
    // seq_lens_k [B]) for packed queries
    const int32_t* block_table;
    const int32_t* seq_lens_k;
    int max_pages, num_pages;
    // score modifiers and block-sparse mask (MODE 3)
    float scale;            // signed; applied before the modifiers
    float softcap;          // > 0: s -> softcap * tanh(s / softcap)
    const float* alibi;     // [Hq] or NULL: s -= slope_h * |i + off - j|
    const float* bias;      // or NULL: s += bias[b * bias_sb + h * bias_sh + j]
    long long bias_sb, bias_sh;
    const uint8_t* bmask;   // or NULL: block (i / block_q, j / block_k) of (b, h) computed iff != 0
    long long bm_sb, bm_sh;
    int bm_nkb, block_q, block_k;
};

constexpr int kMaxList = 2048;   // visited key tiles a block-sparse query tile may list

template <int D>
struct Tile {
    static constexpr int KCH = D / 8;                   // 16-byte chunks per row
    static constexpr int ELEMS = kBN * D;               // 16-bit elements per K or V tile
    static constexpr int LOADS = kBN * KCH / kGroupThreads;  // 16-byte direct loads per thread
    __device__ static __forceinline__ int k_phys(int row, int ch) { return swz_rows<KCH>(row, ch); }
    __device__ static __forceinline__ int v_phys(int row, int ch) { return swz_both<KCH>(row, ch); }
};

// Sequence s of a pack: tokens [cu[s], cu[s+1]) clamped into [0, total] and to at most
// max_len of them, so that every access stays inside the packed tensors whatever the
// offsets hold.  Uniform over the workgroup (scalar loads of a uniform index).
__device__ __forceinline__ void seq_bounds(const int32_t* cu, int s, int total, int max_len,
                                           int* start, int* len) {
    int s0 = mfa_uniform_load(cu + s);
    int s1 = mfa_uniform_load(cu + s + 1);
    s0 = s0 < 0 ? 0 : (s0 > total ? total : s0);
    s1 = s1 < s0 ? s0 : (s1 > total ? total : s1);
    *start = s0;
    *len = (s1 - s0) > max_len ? max_len : (s1 - s0);
}

// Sequence-major order of packed sequences (B <= 64, Hkv a multiple of 8).  The
// workgroups of XCD x = id % 8 (dispatch goes round-robin over the 8 XCDs) take the KV
// heads x, x + 8, ...; they run sequence after sequence, longest key range first, and
// within a sequence all query tiles of one KV head back to back (longest tile first, its
// g query heads side by side).  The workgroups that stream one sequence's K/V through the
// XCD's L2 then start together and read the same tiles at about the same time.  Lane i of
// every wave holds sequence i; k = id / 8 indexes the XCD's items.  Returns false past the
// XCD's last item.  (Uniform over the workgroup.)
template <bool PAGED>
__device__ __forceinline__ bool seq_major_item(const FwdArgs& a, int lane, int* b, int* h, int* qt,
                                               int* n_seq_tiles) {
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
    int ni = 0, key = -1;
    if (lane < a.B) {
        int s0 = a.cu_q[lane], s1 = a.cu_q[lane + 1];
        s0 = s0 < 0 ? 0 : (s0 > a.total_q ? a.total_q : s0);
        s1 = s1 < s0 ? s0 : (s1 > a.total_q ? a.total_q : s1);
        const int len = (s1 - s0) > a.Nq ? a.Nq : (s1 - s0);
        ni = (len + kBM - 1) / kBM;
        if constexpr (PAGED) {
            const int L = a.seq_lens_k[lane];
            key = L < 0 ? 0 : (L > a.Nk ? a.Nk : L);
        } else {
            int k0 = a.cu_k[lane], k1 = a.cu_k[lane + 1];
            k0 = k0 < 0 ? 0 : (k0 > a.total_k ? a.total_k : k0);
            k1 = k1 < k0 ? k0 : (k1 > a.total_k ? a.total_k : k1);
            key = (k1 - k0) > a.Nk ? a.Nk : (k1 - k0);
        }
    }
    // rank of this lane's sequence: longer key ranges first, ties by index
    int rank = 0;
    for (int j = 0; j < a.B; ++j) {
        const int kj = __builtin_amdgcn_readlane(key, j);
        rank += (kj > key || (kj == key && j < lane)) ? 1 : 0;
    }
    // items of this XCD before the sequence: (KV heads of the XCD) x g x tiles
    const int cnt = (a.Hkv >> 3) * a.g * ni;
    int excl = 0;
    for (int j = 0; j < a.B; ++j) {
        const int rj = __builtin_amdgcn_readlane(rank, j);
        const int cj = __builtin_amdgcn_readlane(cnt, j);
        excl += rj < rank ? cj : 0;
    }
    *n_seq_tiles = ni;   // (per lane: this lane's sequence)
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < a.B && k >= excl && k < excl + cnt);
    if (hit == 0) return false;
    const int sb = (int)__builtin_ctzll(hit);
    const int local = k - __builtin_amdgcn_readlane(excl, sb);
    const int nb = __builtin_amdgcn_readlane(ni, sb);
    const int per_kv = a.g * nb;
    const int mi = local / per_kv, rest = local - mi * per_kv;
    *b = sb;
    *qt = nb - 1 - rest / a.g;
    *h = (x + 8 * mi) * a.g + rest % a.g;
    return true;
}

// MODE 0: dense [B, H, N, D] tensors.
// MODE 1: packed variable-length sequences.  Q, O are [total_q, Hq, D] and K, V
//   [total_k, Hkv, D] (rows of one head are Hq * D / Hkv * D elements apart), sequence b
//   spans cu_q[b] .. cu_q[b+1] - 1 and cu_k[b] .. cu_k[b+1] - 1, and its mask is aligned
//   bottom-right on its own lengths.  LSE is [Hq, total_q].
// MODE 2: packed queries as in MODE 1; sequence b's seq_lens_k[b] keys sit in a paged
//   cache, token t in page block_table[b, t / 16], slot t % 16.
// MODE 3: dense tensors with score modifiers (softcap, ALiBi, an additive per-key bias)
//   and an optional block-sparse mask: the workgroup first lists the key tiles of its
//   causal / window range that hold a computed block (a compacted list in LDS, with
//   per-(wave, 32-key block) visibility bits and a no-mask flag), then walks the list.
template <int D, int DT, int GROUPS, bool TILELOG, bool NEG, int MODE, bool PAIR>
__global__ __launch_bounds__(GROUPS * kGroupThreads, 2) void mfa_fwd_kernel(FwdArgs a) {
    constexpr bool VAR = MODE == 1 || MODE == 2;   // packed sequences
    constexpr bool PAGED = MODE == 2;
    using T = Tile<D>;
    constexpr int BN = kBN;
    constexpr int NKB = D / 16;   // k-steps of S^T = K Q^T
    constexpr int NDB = D / 32;   // 32-row blocks of O^T
    constexpr int NNB = BN / 32;  // 32-key blocks of a tile

    // per wave group: K buffers 0, 1 then V buffers 0, 1 (one set for head pairs)
    static_assert(!PAIR || (MODE == 0 && GROUPS == 2), "head pairs: dense inputs, two groups");
    __shared__ __attribute__((aligned(1024))) uint16_t smem_all[(PAIR ? 1 : GROUPS) * 4 * T::ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int grp = GROUPS == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 8);   // wave group
    const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);    // wave within its group
    uint16_t* smem = smem_all + (PAIR ? 0 : grp * 4 * T::ELEMS);
    const int g32 = lane >> 5;
    const int l32 = lane & 31;

    // Chained tiles (dense inputs, two wave groups): a workgroup runs a long causal
    // query tile and then its complementary short one, so every workgroup has the same
    // work and the second tile starts without a new workgroup launch.
    constexpr bool CAN_CHAIN = MODE == 0 && GROUPS == 2 && !PAIR;
    const int n_rep = (CAN_CHAIN && a.chain) ? 2 : 1;
    for (int rep = 0; rep < n_rep; ++rep) {
    // ---- which (query tile, batch, head) -------------------------------------------
    const int id = blockIdx.x;
    const int round = id / a.HB;
    const int w = id - round * a.HB;
    // longest query tiles first: with one workgroup per CU, dynamic dispatch then
    // hands the short tiles to the CUs that finish early.  For packed sequences the
    // rounds count down the end of the tile's key range in BM-key units (below), which
    // orders the tiles of all sequences by causal work, whatever their lengths.
    int qt = rep == 0 ? a.n_q_tiles - 1 - round : round;
    int b, h;
    const bool sm = VAR && a.seqmajor;
    if (sm) {
        int ni = 0;
        const bool have = seq_major_item<PAGED>(a, lane, &b, &h, &qt, &ni);
        // the records of sequences with no query tile are written by the XCD's first
        // workgroup, for the query heads of the XCD's KV heads (lane i: sequence i)
        if (TILELOG && tid < 64 && (blockIdx.x >> 3) == 0 && lane < a.B && ni == 0) {
            for (int hh = 0; hh < a.Hq; ++hh) {
                if (((hh / a.g) & 7) != (int)(blockIdx.x & 7)) continue;
                for (int t = 0; t < a.n_q_tiles; ++t) {
                    int32_t* r = a.tile_log + ((size_t)(lane * a.Hq + hh) * a.n_q_tiles + t) * 4;
                    r[0] = -1;
                    r[1] = 0;
                    r[2] = 0;
                    r[3] = -1;
                }
            }
        }
        if (!have) return;   // past the XCD's last item (uniform)
    } else if (!VAR && !PAIR && GROUPS == 1 && a.seqmajor) {
        // head-major order per XCD (dense layout): XCD x takes KV heads x, x + 8, ...; for
        // each batch element it runs each KV head's query tiles longest first, the g query
        // heads of a tile side by side
        const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
        const int per_kv = a.g * a.n_q_tiles;
        const int per_b = (a.Hkv >> 3) * per_kv;
        b = k / per_b;
        const int r1 = k - b * per_b;
        const int mi = r1 / per_kv, r2 = r1 - mi * per_kv;
        qt = a.n_q_tiles - 1 - r2 / a.g;
        h = (x + 8 * mi) * a.g + r2 % a.g;
    } else if (a.xcd_group) {
        // consecutive workgroups go to different XCDs (id % 8); keep every query head
        // of one (batch, KV head) on the same XCD so its K/V stay in that L2
        const int x = w & 7, j = w >> 3;
        const int gg = PAIR ? a.g >> 1 : a.g;   // workgroups per (batch, KV head) and tile
        const int pair = x + 8 * (j / gg);
        b = pair / a.Hkv;
        h = (pair - b * a.Hkv) * gg + (j % gg);
    } else {
        const int hq = PAIR ? a.Hq >> 1 : a.Hq;
        b = w / hq;
        h = w - b * hq;
    }
    // head pairs: the workgroup's two groups take query heads 2h' and 2h' + 1 (one KV head)
    if (PAIR) h = 2 * h + grp;
    const int kvh = h / a.g;

    // this (batch, head)'s sequence: lengths, first tokens and mask
    int Nq = a.Nq, Nk = a.Nk;
    int qs = 0, ks = 0;
    MfaMask mask = a.mask;
    if constexpr (VAR) {
        seq_bounds(a.cu_q, b, a.total_q, a.Nq, &qs, &Nq);
        if constexpr (PAGED) {
            // cached tokens, clamped to the block table's capacity
            const int L = mfa_uniform_load(a.seq_lens_k + b);
            Nk = L < 0 ? 0 : (L > a.Nk ? a.Nk : L);
        } else {
            seq_bounds(a.cu_k, b, a.total_k, a.Nk, &ks, &Nk);
        }
        mask = mfa_make_mask(Nq, Nk, a.causal, a.left, a.right);
        // tile qt of this sequence ends its causal key range near off + (qt + 1) * BM, so
        // it runs in round n_rounds - 1 - qt - c with c = floor(off / BM) (0 if off < 0);
        // n_rounds >= ceil(Nq / BM) + c for every sequence, so each tile has one round
        const int n_tiles = (Nq + kBM - 1) / kBM;
        const int c = Nk > Nq ? (Nk - Nq) / kBM : 0;
        if (!sm) qt = a.n_rounds - 1 - round - c;
        // the records of tiles past this sequence's last one are written by the workgroup
        // of its last tile (in round order: by round 0's if it has none)
        if (TILELOG && (PAIR ? (tid & 255) : tid) == 0 && (n_tiles > 0 ? qt == n_tiles - 1 : !sm && round == 0)) {
            for (int t = n_tiles; t < a.n_q_tiles; ++t) {
                int32_t* r = a.tile_log + ((size_t)(b * a.Hq + h) * a.n_q_tiles + t) * 4;
                r[0] = -1;
                r[1] = 0;
                r[2] = 0;
                r[3] = -1;
            }
        }
        if (qt < 0 || qt >= n_tiles) return;   // no tile of this sequence here (uniform)
    }
    const int q0 = qt * kBM;
    // row strides (elements) and the first element of this head's rows
    const int SQ = VAR ? a.Hq * D : D;
    const int SK = VAR ? a.Hkv * D : D;

    // with two wave groups the visited key tiles [t_lo, t_hi) are split between them:
    // group 0 takes the first ceil(n/2), group 1 the rest (head pairs: each group walks all
    // of them, over the one K/V stream the workgroup shares)
    int t_lo, t_hi;
    mfa_tile_range(mask, Nq, kBM, BN, qt, &t_lo, &t_hi);
    int n_all = t_hi - t_lo;

    // block-sparse: list the tiles of [t_lo, t_hi) holding a computed block (one wave
    // scans 64 tiles per ballot); entry = tile | visibility bits (2 * wave + key block)
    // << 20 | no-mask flag << 28
    __shared__ int tlist[MODE == 3 ? kMaxList : 1];
    __shared__ int tcount;
    const bool use_list = MODE == 3 && a.bmask != nullptr;
    if constexpr (MODE == 3) {
        if (use_list) {
            if (tid < 64) {
                const uint8_t* bm = a.bmask + (size_t)b * a.bm_sb + (size_t)h * a.bm_sh;
                int cnt = 0;
                for (int base = t_lo; base < t_hi; base += 64) {
                    const int kt = base + lane;
                    bool any = false, all = true;
                    int bits = 0;
                    if (kt < t_hi) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const int r0 = q0 + 32 * w;
                            if (r0 >= Nq) {      // rows past the end: no constraint
                                bits |= 3 << (2 * w);
                                continue;
                            }
                            const int qb = r0 / a.block_q;
                            const int r1 = min(r0 + 31, Nq - 1);
                            const int64_t lo0 = mfa_row_lo(mask, r0), hi1 = mfa_row_hi(mask, r1);
#pragma unroll
                            for (int nb = 0; nb < 2; ++nb) {
                                // the 32 x 32 sub-block lies in one mask block; it is computed
                                // iff that block is on and some pair in it is causal / window
                                // visible (row bounds grow by one per row, so checking the
                                // first row's low end and the last row's high end suffices)
                                const int k0 = kt * BN + 32 * nb;
                                const int k1 = min(k0 + 31, Nk - 1);
                                const bool on = k0 < Nk && hi1 >= k0 && lo0 <= k1 &&
                                                bm[(size_t)qb * a.bm_nkb + k0 / a.block_k] != 0;
                                bits |= (on ? 1 : 0) << (2 * w + nb);
                                any |= on;
                                all &= on;
                            }
                        }
                    }
                    const uint64_t mk = __builtin_amdgcn_ballot_w64(any);
                    const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
                    if (any && pos < kMaxList)
                        tlist[pos] = kt | (bits << 20) | ((all && mfa_tile_full(mask, kBM, BN, qt, kt)) ? 1 << 28 : 0);
                    cnt += __builtin_popcountll(mk);
                }
                if (lane == 0) tcount = cnt < kMaxList ? cnt : kMaxList;
            }
            __syncthreads();
            n_all = tcount;
        }
    }
    const bool first = grp == 0 || PAIR;
    const int n0 = (GROUPS == 1 || PAIR) ? n_all : (n_all + 1) >> 1;
    const int kt_lo = first ? t_lo : t_lo + n0;
    const int n = first ? n0 : n_all - n0;   // this group's tiles (n0 or n0 - 1)
    const int lbase = first ? 0 : n0;        // this group's first list entry
    // list entry of this group's idx-th visited tile.  Block-sparse lists are walked from
    // the diagonal down: the workgroups of a head that run together then sit at nearby key
    // tiles all along (each starts at its own diagonal, one tile below the next), where
    // from key 0 up the late starters re-read the head's first keys long after the L2 has
    // dropped them.
    auto list_at = [&](int idx) { return lbase + n - 1 - idx; };
    // key tile of this group's idx-th visited tile
    auto tile_at = [&](int idx) {
        if constexpr (MODE == 3) {
            if (use_list) return __builtin_amdgcn_readfirstlane(lds_read_i32(tlist + list_at(idx)) & 0xfffff);
        }
        return kt_lo + idx;
    };

    const size_t q_base = VAR ? ((size_t)qs * a.Hq + h) * D : (size_t)(b * a.Hq + h) * (size_t)a.Nq * D;
    // (paged: the head's slice of the pool's page 0; pages are 16 * SK elements apart)
    const size_t kv_base = PAGED ? (size_t)kvh * D
                           : VAR ? ((size_t)ks * a.Hkv + kvh) * D
                                 : (size_t)(b * a.Hkv + kvh) * (size_t)a.Nk * D;
    const uint16_t* kg = a.k + kv_base;
    const uint16_t* vg = a.v + kv_base;

    const int qrow = q0 + wave * 32 + l32;
    const bool qvalid = qrow < Nq;

    // ---- Q^T operand in registers (rows past Nq read as zero) --------------------
    mfa_u32x4 qreg[NKB];
    {
        // the range ends with the last row's D elements, so rows >= Nq fall outside it
        const auto rq = mfa_rsrc(a.q + q_base, (uint32_t)((Nq - 1) * SQ + D) * 2);
        const uint32_t off = ((uint32_t)qrow * SQ + g32 * 8) * 2;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) qreg[kb] = mfa_load16(rq, off + kb * 32);
        // complete here, so that no wait for them is left to the key loop (vmcnt is one
        // counter, which the loop's own direct loads keep busy)
        __builtin_amdgcn_s_waitcnt(0x0f70);
    }

    // per-row visible key bounds (inclusive), clamped into int range
    const int64_t rlo64 = mfa_row_lo(mask, qrow);
    const int64_t rhi64 = mfa_row_hi(mask, qrow);
    const int row_lo = rlo64 > Nk ? Nk : (int)rlo64;
    const int row_hi = rhi64 < -1 ? -1 : (int)rhi64;
    const float alibi_slope = (MODE == 3 && a.alibi != nullptr)
                                  ? __builtin_bit_cast(float, mfa_uniform_load((const int32_t*)a.alibi + h))
                                  : 0.f;

    mfa_f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = mfa_f32x16{};
    float m_run = -MFA_INF;   // exponent offset (log2 domain, scaled)
    float l_run = 0.f;        // this lane's half of the row sum

    // ---- direct global -> LDS tile loads ------------------------------------------
    // The CW waves that share a tile's copies each make CL of them (head pairs: the
    // workgroup's eight waves, half as many copies each).  Copy i of copying wave w fills
    // the 1 KiB block b = CW*i + w of the tile (rows b*RPB .. b*RPB + RPB - 1, RPB = 64 / KCH
    // rows per block); lane l writes 16 bytes at LDS slot b*64 + l, i.e. (row, physical
    // chunk), fetching the logical chunk the swizzle maps there.  Blocks of one wave are
    // CW * RPB rows apart, a multiple of 16, which leaves the swizzles unchanged, so one
    // per-lane offset serves every copy of the thread and each copy only moves the buffer
    // base (scalar).
    constexpr int RPB = 64 / T::KCH;
    constexpr int CW = PAIR ? 8 : 4;
    constexpr int CL = T::LOADS * 4 / CW;
    const int cwave = PAIR ? grp * 4 + wave : wave;
    uint32_t kld_off, vld_off;
    {
        const int row = cwave * RPB + lane / T::KCH, phys = lane % T::KCH;
        kld_off = (uint32_t)(row * SK + T::k_phys(row, phys) * 8) * 2;
        vld_off = (uint32_t)(row * SK + T::v_phys(row, phys) * 8) * 2;
    }
    // One buffer range per tile: rows from k0 on (an empty range when the tile is not
    // needed, which makes the copies zero-filling no-ops into a free buffer); copy i of a
    // thread is at a fixed offset from the tile start, kept in a vector register of its
    // own (the range check applies to it).  Packed rows are SK apart, so there the range
    // ends with the last row's D elements.
    //
    // Paged keys: a key tile is BN / 16 pages, and the rows of copy i of copying wave w all lie
    // in page ((CW * i + w) * RPB) / 16 of the tile, at row (row & 15) of that page; the copy
    // gets a range over the page's valid rows of this head (empty for an unused or invalid
    // page).  The page ids of the tiles a stage copies are read one stage ahead.
    constexpr int PAGE = 16;
    struct PagedTile {
        int kt;
        bool need;
    };
    auto tile_rsrc = [&](const uint16_t* src, int kt, bool need) {
        if constexpr (PAGED) {
            return PagedTile{kt, need};
        } else {
            const int k0 = need ? kt * BN : 0;
            const int rows = need ? max(Nk - k0, 0) : 0;
            const int bytes = VAR ? (rows > 0 ? ((rows - 1) * SK + D) * 2 : 0) : rows * D * 2;
            return mfa_rsrc(src + (size_t)k0 * SK, (uint32_t)bytes);
        }
    };
    const uint32_t copy_step = (uint32_t)(CW * RPB * SK * 2);
    uint32_t kpg_off = 0, vpg_off = 0;
    if constexpr (PAGED) {
        const int row = cwave * RPB + lane / T::KCH, phys = lane % T::KCH;
        kpg_off = (uint32_t)((row & (PAGE - 1)) * SK + T::k_phys(row, phys) * 8) * 2;
        vpg_off = (uint32_t)((row & (PAGE - 1)) * SK + T::v_phys(row, phys) * 8) * 2;
    }
    const int32_t* bt_row = PAGED ? a.block_table + (size_t)b * a.max_pages : nullptr;
    auto page_slot = [&](int kt, int i) { return kt * (BN / PAGE) + ((CW * i + cwave) * RPB) / PAGE; };
    auto load_ids = [&](int kt, bool need, int(&ids)[T::LOADS]) {
#pragma unroll
        for (int i = 0; i < CL; ++i) {
            const int slot = page_slot(kt, i);
            ids[i] = (need && slot * PAGE < Nk) ? mfa_uniform_load(bt_row + slot) : -1;
        }
    };
    auto page_rsrc = [&](const uint16_t* pool, int kt, int i, int pid) {
        const int slot = page_slot(kt, i);
        const int rows = min(Nk - slot * PAGE, PAGE);
        const bool ok = pid >= 0 && pid < a.num_pages && rows > 0;
        return mfa_rsrc(pool + (ok ? (size_t)pid * (PAGE * SK) : 0),
                        ok ? (uint32_t)(((rows - 1) * SK + D) * 2) : 0u);
    };
    int kpid[T::LOADS], vpid[T::LOADS];   // ids of the tiles the current stage copies
    auto copy_k = [&](const auto& r, auto buf_c, int i) {
        constexpr int buf = decltype(buf_c)::value;
        if constexpr (PAGED)
            mfa_load16_lds(page_rsrc(kg, r.kt, i, r.need ? kpid[i] : -1),
                           smem + buf * T::ELEMS + (CW * i + cwave) * 512, kpg_off);
        else
            mfa_load16_lds(r, smem + buf * T::ELEMS + (CW * i + cwave) * 512, kld_off + i * copy_step);
    };
    auto copy_v = [&](const auto& r, auto buf_c, int i) {
        constexpr int buf = decltype(buf_c)::value;
        if constexpr (PAGED)
            mfa_load16_lds(page_rsrc(vg, r.kt, i, r.need ? vpid[i] : -1),
                           smem + (2 + buf) * T::ELEMS + (CW * i + cwave) * 512, vpg_off);
        else
            mfa_load16_lds(r, smem + (2 + buf) * T::ELEMS + (CW * i + cwave) * 512, vld_off + i * copy_step);
    };
    auto issue_k = [&](int kt, auto buf_c) {
        if constexpr (PAGED) {
            int ids[T::LOADS];
            load_ids(kt, true, ids);
#pragma unroll
            for (int i = 0; i < CL; ++i)
                mfa_load16_lds(page_rsrc(kg, kt, i, ids[i]), smem + decltype(buf_c)::value * T::ELEMS + (CW * i + cwave) * 512,
                               kpg_off);
        } else {
            const auto r = tile_rsrc(kg, kt, true);
#pragma unroll
            for (int i = 0; i < CL; ++i) copy_k(r, buf_c, i);
        }
    };
    auto issue_v = [&](int kt, auto buf_c) {
        if constexpr (PAGED) {
            int ids[T::LOADS];
            load_ids(kt, true, ids);
#pragma unroll
            for (int i = 0; i < CL; ++i)
                mfa_load16_lds(page_rsrc(vg, kt, i, ids[i]),
                               smem + (2 + decltype(buf_c)::value) * T::ELEMS + (CW * i + cwave) * 512, vpg_off);
        } else {
            const auto r = tile_rsrc(vg, kt, true);
#pragma unroll
            for (int i = 0; i < CL; ++i) copy_v(r, buf_c, i);
        }
    };

    // ---- per-lane LDS operand addresses (elements; buffer and block offsets are
    // compile-time immediates) --------------------------------------------------------
    // K (S^T A operand): row key_perm(l32) (+32 per key block), chunk 2*kb + g32.
    int k_rd[NKB];
    {
        const int row = key_perm(l32);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) k_rd[kb] = row * D + T::k_phys(row, 2 * kb + g32) * 8;
    }
    // V^T (PV A operand) via transposing reads: lane group qg = lane / 16 covers
    // columns 16*(qg%2) .. +15 of a 32-column block and keys 8*(qg/2) .. +3 (+4 for the
    // second read, v4 further); lane i of the group addresses row i/4, columns 4*(i%4) .. +3.
    const int v4 = tr4_delta<D>(lane);
    int v_rd[NDB];
    {
        const int qg = lane >> 4, i = lane & 15;
        const int row = 8 * (qg >> 1) + (i >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = db * 32 + 16 * (qg & 1) + 4 * (i & 3);
            v_rd[db] = row * D + T::v_phys(row, col >> 3) * 8 + (col & 7);
        }
    }

    const float sl2 = a.scale_log2_abs;
    int n_edge = 0;

    // ---- score modifiers (MODE 3): the scores become scale * q.k, softcapped, minus the
    // ALiBi distance penalty, plus the key bias (copied to LDS one stage ahead) ----------
    __shared__ __attribute__((aligned(16))) float sbias[MODE == 3 ? GROUPS * 2 * kBN : 4];
    auto copy_bias = [&](int kt, int buf) {
        const int k0 = kt * BN;
        const float* row = a.bias + (size_t)b * a.bias_sb + (size_t)h * a.bias_sh;
        const auto r = mfa_rsrc(row + k0, (uint32_t)max(Nk - k0, 0) * 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(sbias + (grp * 2 + buf) * kBN), 4,
            (uint32_t)lane * 4, 0, 0, 0);
    };
    auto apply_modifiers = [&](mfa_f32x16(&sc)[NNB], int kt, int buf) {
        const int k0 = kt * BN;
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) sc[nb] *= a.scale;
        if (a.softcap > 0.f) {   // c * tanh(x / c) = c - 2c / (exp(2x / c) + 1)
            const float c = a.softcap, k2 = 2.f * 1.4426950408889634f / c;
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float t = mfa_exp2(sc[nb][r] * k2);
                    sc[nb][r] = c - 2.f * c * __builtin_amdgcn_rcpf(t + 1.f);
                }
        }
        if (a.alibi != nullptr) {
            const float slope = alibi_slope;
            const int qpos = qrow + (Nk - Nq);
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + nb * 32 + 16 * (r >> 3) + 8 * g32 + (r & 7);
                    sc[nb][r] -= slope * fabsf((float)(qpos - key));
                }
        }
        if (a.bias != nullptr) {
            const float* bl = sbias + (grp * 2 + buf) * kBN;
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int kk = nb * 32 + 16 * hh + 8 * g32;
                    const mfa_f32x4 b0 = lds_read_f4(bl + kk), b1 = lds_read_f4(bl + kk + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sc[nb][8 * hh + e] += b0[e];
                        sc[nb][8 * hh + 4 + e] += b1[e];
                    }
                }
        }
    };

    // S^T = K Q^T for the key tile in K buffer KBUF into s
    auto qk_mfma = [&](auto kb_c, mfa_f32x16(&s)[NNB]) {
        constexpr int kbuf = decltype(kb_c)::value;
        const uint16_t* base = smem + kbuf * T::ELEMS;
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) s[nb] = mfa_f32x16{};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb) {
                const mfa_u32x4 kop = lds_read16(base + k_rd[kb] + nb * 32 * D);
                s[nb] = mfa_mfma32<DT>(kop, qreg[kb], s[nb]);
            }
        }
    };

    // O^T += V^T P^T with V from V buffer VBUF
    auto pv_mfma = [&](auto vb_c, const mfa_u32x4(&pop)[NNB][2], auto copy_v_part) {
        constexpr int vbuf = decltype(vb_c)::value;
        const uint16_t* base = smem + (2 + vbuf) * T::ELEMS;
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                copy_v_part(2 * nb + hh);
                const int kofs = (nb * 32 + hh * 16) * D;
                mfa_u32x4 vop[NDB];
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const mfa_u32x2 l2 = lds_read_tr(base + v_rd[db] + kofs);
                    const mfa_u32x2 h2 = lds_read_tr(base + v_rd[db] + kofs + v4);
                    vop[db] = mfa_u32x4{l2[0], l2[1], h2[0], h2[1]};
                }
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] = mfa_mfma32<DT>(vop[db], pop[nb][hh], oacc[db]);
            }
        }
    };

    // One pipeline stage; P = parity of j (selects the LDS buffers and which S register
    // set is current).  The stage always issues S(j+1): on the last tile that product
    // reads a stale buffer and is never used, which keeps the common path free of
    // branches.  On edge tiles the invisible scores of S(j) are first overwritten with
    // -inf (after the sign of scale), so the rest of the stage is the same code.
    auto stage = [&](const int j, auto p_c, mfa_f32x16(&s_cur)[NNB], mfa_f32x16(&s_next)[NNB]) {
        constexpr int P = decltype(p_c)::value;
        int kt = kt_lo + j;
        int ent = 0;   // block-sparse list entry of tile j
        int kt_k = kt + 2, kt_v = kt + 1;
        if constexpr (MODE == 3) {
            if (use_list) {
                ent = __builtin_amdgcn_readfirstlane(lds_read_i32(tlist + list_at(j)));
                kt = ent & 0xfffff;
                kt_k = j + 2 < n ? tile_at(j + 2) : 0;
                kt_v = j + 1 < n ? tile_at(j + 1) : 0;
            }
        }
        // copies of K(j+2) and V(j+1), spread over the stage (a burst of copies at the
        // start would queue every wave behind the CU's address path)
        const auto rk = tile_rsrc(kg, kt_k, j + 2 < n);
        const auto rv = tile_rsrc(vg, kt_v, j + 1 < n);
        if constexpr (MODE == 3) {
            if (a.bias != nullptr && wave == 0 && j + 1 < n) copy_bias(kt_v, P ^ 1);
            apply_modifiers(s_cur, kt, P);
        }
        int kpid_n[T::LOADS], vpid_n[T::LOADS];   // (paged) ids for the next stage's copies
        if constexpr (PAGED) {
            load_ids(kt + 3, j + 3 < n, kpid_n);
            load_ids(kt + 2, j + 2 < n, vpid_n);
        }
        // The first two K operands of S(j+1) (landed before the last barrier) are read now,
        // so that their LDS latency passes behind the mask, row max and offset raise below
        // (a read issued after that branch could not be moved above it).
        const uint16_t* kbase = smem + (P ^ 1) * T::ELEMS;
        const mfa_u32x4 kpre0 = lds_read16(kbase + k_rd[0]);
        const mfa_u32x4 kpre1 = lds_read16(kbase + k_rd[1]);

        const bool full = use_list ? ((ent >> 28) & 1) != 0 : mfa_tile_full(mask, kBM, BN, qt, kt);
        if (!full) {
            // element r of key block nb holds key base + c with c = 32 nb + 16 (r / 8) + r % 8
            // (a constant), base = kt * BN + 8 g32; it is visible iff lo <= c <= lo + span with
            // the row's bounds rebased to base: one unsigned compare per element.  A row that
            // sees no key gets lo far below every c, so every compare fails.
            const int base = kt * BN + 8 * g32;
            const bool any = row_hi >= row_lo;
            const int lo = any ? row_lo - base : -(1 << 30);
            const uint32_t span = any ? (uint32_t)(row_hi - row_lo) : 0u;
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int c = nb * 32 + 16 * (r >> 3) + (r & 7);
                    const bool vis = (uint32_t)(c - lo) <= span &&
                                     (!use_list || ((ent >> (20 + 2 * wave + nb)) & 1) != 0);
                    s_cur[nb][r] = vis ? s_cur[nb][r] : (NEG ? MFA_INF : -MFA_INF);
                }
            if (TILELOG) ++n_edge;
        }

        // row max of S(j) (signed); lazy offset raise
        float tmax = -MFA_INF;
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, NEG ? -s_cur[nb][r] : s_cur[nb][r]);
        tmax = mfa_pair_max(tmax);
        const float tmax_s = (tmax == -MFA_INF) ? -MFA_INF : tmax * sl2;
        const bool raise = tmax_s > m_run + kLazy;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
            const float m_new = raise ? tmax_s : m_run;
            const float alpha = (m_run == -MFA_INF) ? 0.f : mfa_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
            m_run = m_new;
        }
        const float m_use = (m_run == -MFA_INF) ? 0.f : m_run;

        // S(j+1) on the matrix cores, interleaved (in program order) with the
        // exponentials of S(j), in two phases: phase 0 computes key block 0 of S(j+1)
        // while exponentiating block 1 of S(j); phase 1 computes block 1 of S(j+1)
        // (in the registers block 1 of S(j) just freed) while exponentiating block 0.
        // The K operands are read two steps ahead of their MFMA (a ring of three).
        static_assert(NNB == 2, "two key blocks per tile");
        mfa_u32x4 pop[NNB][2];
        constexpr int PAIRS = 8 / NKB;   // score pairs exponentiated per MFMA step
#pragma unroll
        for (int ph = 0; ph < 2; ++ph) {
            const int nbm = ph;          // key block of S(j+1) on the matrix cores
            const int nbe = 1 - ph;      // key block of S(j) on the vector ALUs
            mfa_f32x16 acc = mfa_f32x16{};
            mfa_u32x4 kop[3];
            if (ph == 0) {
                kop[0] = kpre0;
                kop[1] = kpre1;
            } else {
                kop[0] = lds_read16(kbase + k_rd[0] + nbm * 32 * D);
                kop[1] = lds_read16(kbase + k_rd[1] + nbm * 32 * D);
            }
#pragma unroll
            for (int step = 0; step < NKB; ++step) {
                // K copies: CL per stage, at evenly spaced steps of the two phases
                constexpr int every = 2 * NKB / CL;
                if ((ph * NKB + step) % every == 1) copy_k(rk, MfaInt<P>{}, (ph * NKB + step) / every);
                if (step + 2 < NKB)
                    kop[(step + 2) % 3] = lds_read16(kbase + k_rd[step + 2] + nbm * 32 * D);
                acc = mfa_mfma32<DT>(kop[step % 3], qreg[step], acc);
#pragma unroll
                for (int e = 0; e < PAIRS; ++e) {
                    const int pr = step * PAIRS + e;   // pair index 0..7 within block nbe
                    const int hh = pr >> 2, e2 = pr & 3;
                    const int r0 = 8 * hh + 2 * e2, r1 = r0 + 1;
                    const float x0 = NEG ? -s_cur[nbe][r0] : s_cur[nbe][r0];
                    const float x1 = NEG ? -s_cur[nbe][r1] : s_cur[nbe][r1];
                    // masked scores are -inf here and give exp2(-inf) = 0
                    const float p0 = mfa_exp2(__builtin_fmaf(x0, sl2, -m_use));
                    const float p1 = mfa_exp2(__builtin_fmaf(x1, sl2, -m_use));
                    const uint32_t pk = mfa_pack2<DT>(p0, p1);
                    pop[nbe][hh][e2] = pk;
                    if constexpr (DT == MFA_DT_F16)
                        l_run = mfa_sum2<DT>(pk, l_run);
                    else
                        l_run += p0 + p1;
                }
            }
            s_next[nbm] = acc;
        }

        // O += V(j)^T P(j)^T
        pv_mfma(MfaInt<P>{}, pop, [&](int q) {
            // V copies: CL per stage over the 2 * NNB PV steps
            if (q % (2 * NNB / CL) == 0) copy_v(rv, MfaInt<P ^ 1>{}, q / (2 * NNB / CL));
        });

        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this stage's direct loads landed
        block_barrier();
        if constexpr (PAGED) {
#pragma unroll
            for (int i = 0; i < CL; ++i) {
                kpid[i] = kpid_n[i];
                vpid[i] = vpid_n[i];
            }
        }
    };

    // Barriers are workgroup-wide, so both groups run n0 stages; a group with fewer
    // tiles passes its spare stage with the barrier only.
    mfa_f32x16 sA[NNB], sB[NNB];
    if (n0 > 0) {
        if (n > 0) {
            issue_k(tile_at(0), MfaInt<0>{});
            issue_v(tile_at(0), MfaInt<0>{});
            if constexpr (MODE == 3) {
                if (a.bias != nullptr && wave == 0) copy_bias(tile_at(0), 0);
            }
            if (n > 1) issue_k(tile_at(1), MfaInt<1>{});
            if constexpr (PAGED) {
                load_ids(kt_lo + 2, 2 < n, kpid);
                load_ids(kt_lo + 1, 1 < n, vpid);
            }
            __builtin_amdgcn_s_waitcnt(0x0f70);
        }
        block_barrier();
        if (n > 0) qk_mfma(MfaInt<0>{}, sA);
        block_barrier();   // S(0)'s K reads are done before K buffer 0 is refilled
    }
    for (int j = 0; j < n0; j += 2) {
        if (j < n)
            stage(j, MfaInt<0>{}, sA, sB);
        else
            block_barrier();
        if (j + 1 < n0) {
            if (j + 1 < n)
                stage(j + 1, MfaInt<1>{}, sB, sA);
            else
                block_barrier();
        }
    }

    // Global stores of a wave's 32 x D output block staged row-major in LDS (16-byte chunks
    // XOR-swizzled by row): each store instruction covers 64 / KCH whole rows.  (The lane
    // index is made opaque so that the addresses are formed here rather than hoisted out of
    // the tile loop, where they would hold registers.)
    auto store_block = [&](const uint16_t* stg) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        constexpr int RPS = 64 / T::KCH;   // rows per store instruction
        const int rr = ln / T::KCH, ch = ln % T::KCH;
#pragma unroll
        for (int k = 0; k < 32 / RPS; ++k) {
            const int row = k * RPS + rr;
            const mfa_u32x4 val = *(const mfa_u32x4*)(stg + row * D + (ch ^ (row & (T::KCH - 1))) * 8);
            const int srow = q0 + wave * 32 + row;
            if (srow < Nq) *(mfa_u32x4*)(a.o + q_base + (size_t)srow * SQ + ch * 8) = val;
        }
    };
    // With two key-splitting groups, group 0 merges and stages its block in group 1's V
    // buffers (which the exchange below does not reach), and group 1, idle by then, stores it.
    constexpr bool SPLIT_STORE = GROUPS == 2 && !PAIR;
    uint16_t* const stg_all = PAIR ? smem_all + grp * 2 * T::ELEMS : GROUPS == 2 ? smem_all + 6 * T::ELEMS : smem;

    // ---- merge the two groups' partial states (same rows, disjoint keys) ---------
    // Group 1 leaves (m, l, o) of each lane in LDS (struct-of-arrays, conflict-free);
    // group 0 combines them with its own: M = max(m0, m1), f_i = exp2(m_i - M).
    if constexpr (GROUPS == 2 && !PAIR) {
        constexpr int NC = NDB * 16 + 2;   // o values, m, l per lane
        float* xch = reinterpret_cast<float*>(smem_all);
        __shared__ int edge_cnt;
        const int slot = wave * 64 + lane;
        if (grp == 1) {
            xch[0 * 256 + slot] = m_run;
            xch[1 * 256 + slot] = l_run;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) xch[(2 + db * 16 + r) * 256 + slot] = oacc[db][r];
            if (TILELOG && tid == 256) edge_cnt = n_edge;
        }
        static_assert(NC * 256 * 4 <= GROUPS * 4 * T::ELEMS * 2, "exchange fits in the tile buffers");
        __syncthreads();
        if (grp == 1) {
            __syncthreads();   // group 0 has staged its block
            store_block(stg_all + wave * 32 * D);
            if (n_rep == 1) return;
            __syncthreads();   // the block is read before the next tile's copies
            continue;
        }
        const float m1 = xch[0 * 256 + slot];
        const float l1 = xch[1 * 256 + slot];
        const float M = fmaxf(m_run, m1);
        const float f0 = (m_run == -MFA_INF) ? 0.f : mfa_exp2(m_run - M);
        const float f1 = (m1 == -MFA_INF) ? 0.f : mfa_exp2(m1 - M);
        l_run = f0 * l_run + f1 * l1;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = f0 * oacc[db][r] + f1 * xch[(2 + db * 16 + r) * 256 + slot];
        m_run = M;
        if (TILELOG) n_edge += edge_cnt;
    }

    // ---- epilogue: O = o / l, LSE = (m + log2 l) * ln 2 --------------------------
    const float l_tot = mfa_pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    // O leaves through LDS: the wave writes its 32 x D block row-major (16-byte chunks
    // XOR-swizzled by row) into free tile memory, from where whole rows are stored.  The
    // tile buffers are free here: the last stage ended with every copy landed and every
    // read done.  The two groups of a head pair use K buffers 0, 1 and V buffers 0, 1.
    {
        uint16_t* stg = stg_all + wave * 32 * D;
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lr = ln & 31, lh = ln >> 5;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mfa_u32x2 w2;
                w2[0] = mfa_pack2<DT>(oacc[db][4 * j + 0] * inv, oacc[db][4 * j + 1] * inv);
                w2[1] = mfa_pack2<DT>(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
                const int c = db * 4 + j;   // 16-byte chunk of the row: columns 8c .. 8c + 7
                *(mfa_u32x2*)(stg + lr * D + (c ^ (lr & (T::KCH - 1))) * 8 + 4 * lh) = w2;
            }
        }
        if (!SPLIT_STORE) store_block(stg);
    }
    if (qvalid && a.lse != nullptr && g32 == 0) {
        const size_t li = VAR ? (size_t)h * a.total_q + qs + qrow : (size_t)(b * a.Hq + h) * a.Nq + qrow;
        a.lse[li] = l_tot > 0.f ? (m_run + mfa_log2(l_tot)) * MFA_LN2 : -MFA_INF;
    }
    if (TILELOG && (PAIR ? (tid & 255) : tid) == 0) {
        int32_t* t = a.tile_log + ((size_t)(b * a.Hq + h) * a.n_q_tiles + qt) * 4;
        int first = t_lo, last = t_hi;
        if (use_list && n_all > 0) {
            first = tlist[0] & 0xfffff;
            last = (tlist[n_all - 1] & 0xfffff) + 1;
        }
        t[0] = n_all ? first : -1;
        t[1] = n_all;
        t[2] = n_edge;
        t[3] = n_all ? last : -1;
    }
    if (SPLIT_STORE) __syncthreads();   // the block is staged: group 1 stores it
    if (n_rep > 1) __syncthreads();
    }   // rep
}

template <int D, int DT, int G, bool TL, int MODE, bool PAIR = false>
void launch_sign(const FwdArgs& a, dim3 grid, hipStream_t stream, bool neg) {
    const dim3 block(G * kGroupThreads);
    if (neg)
        hipLaunchKernelGGL((mfa_fwd_kernel<D, DT, G, TL, true, MODE, PAIR>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((mfa_fwd_kernel<D, DT, G, TL, false, MODE, PAIR>), grid, block, 0, stream, a);
}

template <int D, int DT, int MODE>
int launch(const FwdArgs& a, hipStream_t stream, int groups, bool tilelog, bool neg,
           mfa_dispatch_info* info) {
    const dim3 grid((unsigned)a.grid);
    if (a.pair) {
        if constexpr (MODE == 0) {
            if (tilelog) launch_sign<D, DT, 2, true, MODE, true>(a, grid, stream, neg);
            else launch_sign<D, DT, 2, false, MODE, true>(a, grid, stream, neg);
        }
    } else if (groups == 2) {
        if (tilelog) launch_sign<D, DT, 2, true, MODE>(a, grid, stream, neg);
        else launch_sign<D, DT, 2, false, MODE>(a, grid, stream, neg);
    } else {
        if (tilelog) launch_sign<D, DT, 1, true, MODE>(a, grid, stream, neg);
        else launch_sign<D, DT, 1, false, MODE>(a, grid, stream, neg);
    }
    snprintf(info->kernel, sizeof(info->kernel), "mfa_fwd_kernel<D=%d,%s,BM=%d,BN=%d,groups=%d%s%s%s%s>", D,
             DT == MFA_DT_F16 ? "f16" : "bf16", kBM, kBN, groups,
             MODE == 3 ? ",ext" : MODE == 2 ? ",varlen,paged" : MODE == 1 ? ",varlen" : "",
             tilelog ? ",tilelog" : "", neg ? ",neg" : "",
             a.chain ? ",chained" : a.pair ? ",head-pairs" : !a.seqmajor ? "" : (MODE == 1 || MODE == 2) ? ",seq-major" : ",head-major");
    info->BM = kBM;
    info->BN = kBN;
    info->waves = groups * kGroupThreads / 64;
    info->grid[0] = (int)grid.x;
    info->grid[1] = 1;
    info->grid[2] = 1;
    info->block = groups * kGroupThreads;
    return hipGetLastError() == hipSuccess ? MFA_OK : MFA_ERR_HIP;
}



template <int MODE>
int launch_dt(const MfaFwdProblem& pr, const FwdArgs& a, hipStream_t stream, int groups, bool tl,
              bool neg, mfa_dispatch_info* info) {
    if (pr.D == 128)
        return pr.dtype == MFA_F16 ? launch<128, MFA_DT_F16, MODE>(a, stream, groups, tl, neg, info)
                                   : launch<128, MFA_DT_BF16, MODE>(a, stream, groups, tl, neg, info);
    return pr.dtype == MFA_F16 ? launch<64, MFA_DT_F16, MODE>(a, stream, groups, tl, neg, info)
                               : launch<64, MFA_DT_BF16, MODE>(a, stream, groups, tl, neg, info);
}

}  // namespace

int mfa_fwd_bn(int) { return kBN; }

// Wave groups per workgroup.  Two workgroups of one group share a CU and overlap
// each other's prologue and epilogue, which is best when the grid has many query
// tiles.  A small grid (at most two workgroups per CU: every workgroup resident at
// once, so the longest query tile bounds the run) instead gets one 8-wave workgroup
// per CU whose two groups split the key range of the query tile; for dense inputs with
// an even number of query tiles such a workgroup then runs two complementary tiles.
int mfa_fwd_groups(long long q_tiles, int Hq, int num_cus) {
    return q_tiles * Hq <= 2LL * num_cus ? 2 : 1;
}
int mfa_fwd_bm() { return kBM; }

int mfa_fwd_launch(const MfaFwdProblem& pr, hipStream_t stream, mfa_dispatch_info* info) {
    FwdArgs a;
    a.q = (const uint16_t*)pr.q;
    a.k = (const uint16_t*)pr.k;
    a.v = (const uint16_t*)pr.v;
    a.o = (uint16_t*)pr.out;
    a.lse = pr.lse;
    a.tile_log = pr.tile_log;
    a.B = pr.B;
    a.Hq = pr.Hq;
    a.Hkv = pr.Hkv;
    a.Nq = pr.Nq;
    a.Nk = pr.Nk;
    a.g = pr.Hq / pr.Hkv;
    a.n_q_tiles = (pr.Nq + kBM - 1) / kBM;
    a.n_rounds = pr.cu_seqlens_q != nullptr ? std::max(a.n_q_tiles, (pr.Nk + kBM - 1) / kBM) : a.n_q_tiles;
    a.HB = pr.B * pr.Hq;
    a.xcd_group = ((pr.B * pr.Hkv) % 8 == 0) ? 1 : 0;
    a.cu_q = pr.cu_seqlens_q;
    a.cu_k = pr.cu_seqlens_k;
    a.total_q = pr.total_q;
    a.total_k = pr.total_k;
    a.causal = pr.causal;
    a.left = pr.left;
    a.right = pr.right;
    a.block_table = pr.block_table;
    a.seq_lens_k = pr.seq_lens_k;
    a.max_pages = pr.max_pages;
    a.num_pages = pr.num_pages;
    a.scale = pr.scale;
    a.softcap = pr.ext ? pr.ext->softcap : 0.f;
    a.alibi = pr.ext ? pr.ext->alibi_slopes : nullptr;
    a.bias = pr.ext ? pr.ext->bias : nullptr;
    a.bias_sb = pr.ext ? pr.ext->bias_stride_b : 0;
    a.bias_sh = pr.ext ? pr.ext->bias_stride_h : 0;
    a.bmask = pr.ext ? pr.ext->block_mask : nullptr;
    a.bm_sb = pr.ext ? pr.ext->mask_stride_b : 0;
    a.bm_sh = pr.ext ? pr.ext->mask_stride_h : 0;
    a.bm_nkb = pr.ext ? pr.ext->mask_k_blocks : 0;
    a.block_q = pr.ext ? pr.ext->block_q : 0;
    a.block_k = pr.ext ? pr.ext->block_k : 0;
    const bool var = pr.cu_seqlens_q != nullptr;
    const int mode = pr.ext != nullptr ? 3 : pr.block_table != nullptr ? 2 : var ? 1 : 0;
    // |scale| * log2(e), kept >= 1e-30 so that a masked (-inf) score times it stays
    // -inf; for scale = 0 the visible scores then all scale to ~0, i.e. the same
    // uniform weights up to fp32 rounding
    a.scale_log2_abs = fmaxf(fabsf(pr.scale) * 1.4426950408889634f, 1e-30f);
    // (MODE 3 applies the signed scale itself, before the modifiers)
    if (mode == 3) a.scale_log2_abs = 1.4426950408889634f;
    a.mask = mfa_make_mask(pr.Nq, pr.Nk, pr.causal, pr.left, pr.right);
    const bool tl = pr.tile_log != nullptr;
    const bool neg = mode != 3 && pr.scale < 0.f;
    // query tiles that hold rows: every tile of the grid for dense inputs; for packed
    // sequences at most total_q / BM + B of the grid's B * ceil(max_seqlen_q / BM)
    long long q_tiles = (long long)a.n_q_tiles * pr.B;
    if (var && (long long)pr.total_q / kBM + pr.B < q_tiles) q_tiles = (long long)pr.total_q / kBM + pr.B;
    int groups = mfa_fwd_groups(q_tiles, pr.Hq, mfa_num_cus());
    a.chain = (mode == 0 && groups == 2 && a.n_q_tiles % 2 == 0) ? 1 : 0;
    // Dense GQA with many tiles: one 8-wave workgroup per pair of query heads that share a
    // KV head instead of two 4-wave workgroups, so that each K/V tile is copied to LDS once
    // for both heads (half the copies per FLOP).  Packed sequences keep two 4-wave
    // workgroups per CU: there the pairs measured 11-19% slower.
    a.pair = (mode == 0 && groups == 1 && a.g % 2 == 0) ? 1 : 0;
    if (a.pair) {
        groups = 2;
        a.HB = pr.B * pr.Hq / 2;
    }
    // Each XCD owns whole KV heads when Hkv is a multiple of 8.  Packed sequences (at most
    // 64) then run in sequence-major order per XCD; the grid covers at most
    // floor(total_q / BM) + B query tiles per head, and the workgroups past an XCD's last
    // item exit at once.  Dense layouts with one 4-wave group per workgroup run in
    // head-major order per XCD (same grid).  Both keep the workgroups that stream one K/V
    // through an XCD's L2 running together.
    a.seqmajor = (pr.Hkv % 8 == 0 && ((var && mode != 3 && pr.B <= 64) ||
                                      (!var && groups == 1 && !a.pair))) ? 1 : 0;
    if (a.seqmajor && var)
        a.grid = 8 * (pr.Hkv / 8) * a.g * (pr.total_q / kBM + pr.B);
    else
        a.grid = (a.chain ? a.n_rounds / 2 : a.n_rounds) * a.HB;
    if (mode == 3) return launch_dt<3>(pr, a, stream, groups, tl, neg, info);
    if (mode == 2) return launch_dt<2>(pr, a, stream, groups, tl, neg, info);
    if (mode == 1) return launch_dt<1>(pr, a, stream, groups, tl, neg, info);
    return launch_dt<0>(pr, a, stream, groups, tl, neg, info);
}
