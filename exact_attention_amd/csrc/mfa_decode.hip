// Paged split-KV flash-decode for gfx950: one query token per sequence against a
// paged KV cache.
//
// Pass 1 (mfa_decode_split_kernel): the cached tokens of every sequence are cut into
// contiguous chunks of logical token positions; one workgroup handles one chunk of one
// (sequence, group of query heads sharing a KV head) and writes a partial result
// (O_s normalised, LSE_s) to the workspace.  The grid holds only the non-empty chunks
// (decode_item), and the KV cache, read exactly once, is loaded with the non-temporal
// cache policy.  Pass 2 (mfa_decode_combine_kernel) merges
// the partials of each (sequence, head): M = max_s LSE_s, w_s = exp(LSE_s - M),
// O = sum w_s O_s / sum w_s, LSE = M + log sum w_s.  This is the two-phase split-KV
// decode of the mlx-mfa 2.5.2 page ("Flash Decode", "V2 split-K") over the page pool
// and block table of its "Paged KV" feature and of the MXFlashAttn 1.5.0 page (M1
// paged Split-KV decode).  Every split owns its own workspace slots and writes only
// the slots of its own heads (the per-split slot race described on the MXFlashAttn
// page came from lanes of invalid query heads writing into a neighbour's slot).
//
// Inside a workgroup (4 waves, each a contiguous run of pages of the chunk), per page:
//   S^T = K Q^T on a 16x16x32 MFMA, read straight from the page: the A operand holds
//   the page's 16 token rows (lane % 16 = token, lane / 16 = 64-byte quarter of the
//   row), the B operand the workgroup's HPW query heads replicated over the 16
//   columns.  Lane (G = lane / 16, c = lane % 16) then holds the scores of tokens
//   4G .. 4G+3 for head c % HPW; the other heads' scores come from the lanes of the
//   same quad through DPP.
//   The same lane loads one 16-byte column chunk (c) of V for those 4 tokens and keeps
//   its own online softmax state (m, l) and output slice o[head][8] per head — so the
//   output accumulator is 8 * HPW registers and no reduction is needed in the loop.
//   At the end the partial states of the 4 token groups of every wave are merged in
//   LDS (same max-rescale rule as the combine pass).
// Tokens at or past seq_lens[b] (tail slots of the last page, which may hold any bit
// pattern) are never read: each page is addressed through a buffer resource whose
// range ends at the last valid token, so such loads return zeros, and their scores
// are set to -inf.
#include <mutex>

#include "mfa_device.h"
#include "mfa_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kPage = 16;
constexpr int kPG = 2;   // pages per online-softmax step
constexpr float kLazy = 8.0f;

struct DecArgs {
    const uint16_t* q;
    const uint16_t* kp;
    const uint16_t* vp;
    const int32_t* block_table;
    const int32_t* seq_lens;
    float* ws_o;     // [B, Hq, S, D]
    float* ws_lse;   // [B, Hq, S]  (log2 domain)
    uint16_t* out;
    float* lse;
    int B, Hq, Hkv, g;
    int nq;          // query tokens per sequence (q, out: [B, nq, Hq, D]; LSE [B, nq, Hq])
    int num_pages, max_pages;
    int S, chunk_pages;
    float scale_log2;
};

__device__ __forceinline__ int clamp_len(int L, int max_pages) {
    const int cap = max_pages * kPage;
    return L < 0 ? 0 : (L > cap ? cap : L);
}

// Value of x held by the lane of this quad whose index within the quad is SRC.
template <int SRC>
__device__ __forceinline__ float quad_bcast(float x) {
    constexpr int ctrl = SRC | (SRC << 2) | (SRC << 4) | (SRC << 6);
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), ctrl, 0xf, 0xf, false));
}

// Which (sequence b, head group hg, chunk s) a workgroup of the split kernels takes, and
// b's clamped length L.
//   FLAT (at most kFlatMaxB sequences): the 1-D grid enumerates only the non-empty chunks,
//   sequence by sequence, and within a sequence head group by head group with its chunks
//   consecutive; ids past the last one return false.  Each wave reads seq_lens with one
//   vector load per 64 sequences and finds its item by a prefix sum over the lanes and a
//   ballot.  (Against the 3-D grid this removes the workgroups of empty chunks, 45% of the
//   decode workload's grid, and measured 4% faster; ordering the head groups fastest
//   instead, so that concurrent workgroups read slices of the same pages, gained nothing.)
//   Otherwise the grid is (chunk, head group, sequence) and empty chunks return false.
constexpr int kFlatMaxB = 256;

template <bool FLAT>
__device__ __forceinline__ bool decode_item(const DecArgs& a, int HG, int* b, int* hg, int* s, int* L) {
    if constexpr (!FLAT) {
        *s = blockIdx.x;
        *hg = blockIdx.y;
        *b = blockIdx.z;
        *L = clamp_len(mfa_uniform_load(a.seq_lens + blockIdx.z), a.max_pages);
        return *s * a.chunk_pages < (*L + kPage - 1) / kPage;
    } else {
        const int lane = threadIdx.x & 63;
        const int item = blockIdx.x;
        int before = 0;   // items of the sequences before this group of 64
        for (int base = 0; base < a.B; base += 64) {
            const int bb = base + lane;
            int Lb = 0, n = 0;   // n: this sequence's items (its chunks times HG)
            if (bb < a.B) {
                Lb = clamp_len(a.seq_lens[bb], a.max_pages);
                n = ((Lb + kPage - 1) / kPage + a.chunk_pages - 1) / a.chunk_pages * HG;
            }
            int incl = n;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int t = __shfl_up(incl, d, 64);
                if (lane >= d) incl += t;
            }
            const int excl = incl - n;
            const uint64_t hit =
                __builtin_amdgcn_ballot_w64(n > 0 && item >= before + excl && item < before + incl);
            if (hit != 0) {
                const int src = (int)__builtin_ctzll(hit);
                const int r = item - before - __shfl(excl, src, 64);
                const int nc = __shfl(n, src, 64) / HG;   // chunks of sequence b
                *b = __builtin_amdgcn_readfirstlane(base + src);
                *L = __builtin_amdgcn_readfirstlane(__shfl(Lb, src, 64));
                *hg = __builtin_amdgcn_readfirstlane(r / nc);
                *s = __builtin_amdgcn_readfirstlane(r - (r / nc) * nc);
                return true;
            }
            before += __shfl(incl, 63, 64);
        }
        return false;
    }
}

template <int D, int DT, int HPW, bool FLAT>
__global__ __launch_bounds__(kThreads, 3) void mfa_decode_split_kernel(DecArgs a) {
    constexpr int NKB = D / 32;       // k-steps (16-byte chunks per lane per K row)
    constexpr int NCH = D / 8;        // 16-byte chunks per V row
    constexpr int NT = D / 32;        // tokens per lane per page (4 for D=128, 2 for D=64)
    int s, hg, b, L;
    // an empty chunk has no workgroup (FLAT) or returns here: its slots are neither written
    // nor read
    if (!decode_item<FLAT>(a, a.Hq / HPW, &b, &hg, &s, &L)) return;
    const int h0 = hg * HPW;
    const int kvh = h0 / a.g;

    const int n_pages_b = (L + kPage - 1) / kPage;
    const int page_begin = s * a.chunk_pages;
    const int page_end = min(page_begin + a.chunk_pages, n_pages_b);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = lane >> 4;
    const int c = lane & 15;
    const int ppw = a.chunk_pages / kWaves;
    const int w_begin = page_begin + wave * ppw;
    const int w_end = min(w_begin + ppw, page_end);

    // B operand: query head (c % HPW) of the group, k-chunks 4*kb + G
    mfa_u32x4 qb[NKB];
    {
        const uint16_t* qp = a.q + ((size_t)b * a.Hq + h0 + (c % HPW)) * D;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) qb[kb] = *(const mfa_u32x4*)(qp + (4 * kb + G) * 8);
    }

    // this lane's V slice: chunk vch of tokens vt0 .. vt0 + NT - 1 of each page
    const int vch = c % NCH;
    const int vt0 = 4 * G + NT * (c / NCH);
    const uint32_t tok_bytes = (uint32_t)a.Hkv * D * 2;
    const uint32_t k_off = (uint32_t)(c * a.Hkv * D) * 2;            // A row = token c
    const uint32_t v_off = (uint32_t)(vt0 * a.Hkv * D + vch * 8) * 2;

    float m[HPW], l[HPW], o[HPW][8];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        m[hh] = -MFA_INF;
        l[hh] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[hh][i] = 0.f;
    }

    const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
    const size_t page_elems = (size_t)kPage * a.Hkv * D;

    // Page ids are read one step ahead (right after the step's own loads are issued), so
    // a step's K/V loads never wait for a block-table read.
    int pid_next[kPG];
#pragma unroll
    for (int j = 0; j < kPG; ++j) pid_next[j] = w_begin + j < w_end ? bt[w_begin + j] : -1;

    for (int pg = w_begin; pg < w_end; pg += kPG) {
        mfa_u32x4 kr[kPG][NKB], vr[kPG][NT];
        int nv[kPG];
        int pid_cur[kPG];
#pragma unroll
        for (int j = 0; j < kPG; ++j) pid_cur[j] = __builtin_amdgcn_readfirstlane(pid_next[j]);
#pragma unroll
        for (int j = 0; j < kPG; ++j) {
            const int pi = pg + j;
            const int pid = pid_cur[j];
            const bool pvalid = pid >= 0 && pid < a.num_pages;
            // valid tokens of this page (0 if the page index is out of range)
            nv[j] = pvalid ? min(kPage, L - pi * kPage) : 0;
            const uint16_t* base = (pvalid ? pid : 0) * page_elems + (size_t)kvh * D + a.kp;
            const uint16_t* vbase = (pvalid ? pid : 0) * page_elems + (size_t)kvh * D + a.vp;
            const uint32_t bytes = (uint32_t)nv[j] * tok_bytes;
            const auto rk = mfa_rsrc(base, bytes);
            const auto rv = mfa_rsrc(vbase, bytes);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) kr[j][kb] = mfa_load16_nt(rk, k_off + (4 * kb + G) * 16);
#pragma unroll
            for (int t = 0; t < NT; ++t) vr[j][t] = mfa_load16_nt(rv, v_off + t * tok_bytes);
        }
#pragma unroll
        for (int j = 0; j < kPG; ++j) pid_next[j] = pg + kPG + j < w_end ? bt[pg + kPG + j] : -1;
        // every load of the step is issued before the first use of its data
        __builtin_amdgcn_sched_barrier(0);
        // scores: sc[j][hh][i] for token 4G + i (i < 4) of page j, head hh
        float sc[kPG][HPW][4];
#pragma unroll
        for (int j = 0; j < kPG; ++j) {
            mfa_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) acc = mfa_mfma16<DT>(kr[j][kb], qb[kb], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = 4 * G + i < nv[j];
                const float x = acc[i] * a.scale_log2;
                // head hh's score lives in the quad lane with index hh (HPW = 4),
                // hh + 2*(k/2) (HPW = 2), or in every lane (HPW = 1)
                if constexpr (HPW == 4) {
                    sc[j][0][i] = valid ? quad_bcast<0>(x) : -MFA_INF;
                    sc[j][1][i] = valid ? quad_bcast<1>(x) : -MFA_INF;
                    sc[j][2][i] = valid ? quad_bcast<2>(x) : -MFA_INF;
                    sc[j][3][i] = valid ? quad_bcast<3>(x) : -MFA_INF;
                } else if constexpr (HPW == 2) {
                    const float x0 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                        __builtin_bit_cast(int, x), 0xA0, 0xf, 0xf, false));   // quad_perm 0,0,2,2
                    const float x1 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                        __builtin_bit_cast(int, x), 0xF5, 0xf, 0xf, false));   // quad_perm 1,1,3,3
                    sc[j][0][i] = valid ? x0 : -MFA_INF;
                    sc[j][1][i] = valid ? x1 : -MFA_INF;
                } else {
                    sc[j][0][i] = valid ? x : -MFA_INF;
                }
            }
        }
        // this lane's own tokens: i = NT * (c / NCH) + t (a select, not a dynamic index)
        const bool upper = (NCH < 16) && (c >= NCH);
        auto own = [&](int j, int hh, int t) -> float {
            if constexpr (NCH == 16) return sc[j][hh][t];
            else return upper ? sc[j][hh][NT + t] : sc[j][hh][t];
        };
        // online softmax over this lane's tokens; the offset is raised lazily
        float mb[HPW];
        bool raise_any = false;
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            float t = -MFA_INF;
#pragma unroll
            for (int j = 0; j < kPG; ++j)
#pragma unroll
                for (int i = 0; i < NT; ++i) t = fmaxf(t, own(j, hh, i));
            mb[hh] = t;
            raise_any |= t > m[hh] + kLazy;
        }
        if (__builtin_amdgcn_ballot_w64(raise_any) != 0) {
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) {
                const bool r = mb[hh] > m[hh] + kLazy;
                const float m_new = r ? mb[hh] : m[hh];
                const float alpha = (m[hh] == -MFA_INF) ? 0.f : mfa_exp2(m[hh] - m_new);
                l[hh] *= alpha;
#pragma unroll
                for (int i = 0; i < 8; ++i) o[hh][i] *= alpha;
                m[hh] = m_new;
            }
        }
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            const float mu = (m[hh] == -MFA_INF) ? 0.f : m[hh];
#pragma unroll
            for (int j = 0; j < kPG; ++j) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const float x = own(j, hh, t);
                    const float p = (x == -MFA_INF) ? 0.f : mfa_exp2(x - mu);
                    l[hh] += p;
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        o[hh][2 * e2] += p * mfa_lo<DT>(vr[j][t][e2]);
                        o[hh][2 * e2 + 1] += p * mfa_hi<DT>(vr[j][t][e2]);
                    }
                }
            }
        }
    }

    // merge the partial states in LDS: for each head, NP partials of (m, l, o[D])
    constexpr int GROUPS = 4 * (16 / NCH);           // token groups per wave
    constexpr int NP = kWaves * GROUPS;               // partials per head
    __shared__ float sm_m[HPW][NP];
    __shared__ float sm_l[HPW][NP];
    __shared__ __attribute__((aligned(16))) float sm_o[HPW][NP][D];
    const int part = wave * GROUPS + G * (16 / NCH) + c / NCH;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        float* dst = &sm_o[hh][part][vch * 8];
        *(mfa_f32x4*)dst = mfa_f32x4{o[hh][0], o[hh][1], o[hh][2], o[hh][3]};
        *(mfa_f32x4*)(dst + 4) = mfa_f32x4{o[hh][4], o[hh][5], o[hh][6], o[hh][7]};
        if (vch == 0) {
            sm_m[hh][part] = m[hh];
            sm_l[hh][part] = l[hh];
        }
    }
    __syncthreads();

    for (int idx = tid; idx < HPW * D; idx += kThreads) {
        const int hh = idx / D, d = idx - hh * D;
        float M = -MFA_INF;
#pragma unroll
        for (int p = 0; p < NP; ++p) M = fmaxf(M, sm_m[hh][p]);
        float lt = 0.f, ot = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const float f = (sm_m[hh][p] == -MFA_INF) ? 0.f : mfa_exp2(sm_m[hh][p] - M);
            lt += f * sm_l[hh][p];
            ot += f * sm_o[hh][p][d];
        }
        const size_t slot = ((size_t)b * a.Hq + h0 + hh) * a.S + s;
        a.ws_o[slot * D + d] = lt > 0.f ? ot / lt : 0.f;
        if (d == 0) a.ws_lse[slot] = lt > 0.f ? M + mfa_log2(lt) : -MFA_INF;
    }
}

// Multi-token decode (nq <= 4 new tokens per sequence, e.g. speculative verification):
// the nq tokens are the last nq cached positions, and token n sees the keys at positions
// <= L - nq + n.  One workgroup per (split, group of HPW query heads, sequence) as in the
// single-token kernel, but both products run on the matrix cores, with the HPW * nq
// <= 16 query rows of one KV head packed into the 16 columns of a 16x16x32 MFMA:
//   S^T = K Q^T: A = 16 token rows of a page read straight from HBM (lane % 16 = token,
//     lane / 16 = 16-byte chunk of each 64-byte quarter), B = column c = query row
//     (token c / HPW, head c % HPW).  Lane (G = lane / 16, c) then holds the scores of
//     tokens 4G .. 4G+3 of the page for row c.
//   O^T += V^T P^T over the 32 tokens of two pages, with the k index ordered so that
//     k-group G is {tokens 4G .. 4G+3 of page 0, tokens 4G .. 4G+3 of page 1}: the B
//     operand P^T is then exactly the lane's own 8 exponentials, and the A operand V^T
//     (16 columns x those 8 tokens per lane group) comes from two transposing LDS reads
//     of the wave's own copy of the two pages (direct global -> LDS loads, XOR-swizzled
//     16-byte chunks; no other wave touches it, so no barrier is needed).
// A row's max is shared by its four lanes (two exchanges); each lane keeps its own part
// of the row sum.  The four waves' partial states are merged in LDS at the end.
template <int D>
__device__ __forceinline__ int dec_v_phys(int row, int ch) {
    // the 4 rows a transposing read touches land on distinct 16-byte chunks
    return (D == 128) ? (ch ^ ((row & 3) << 1)) : (ch ^ (((row >> 1) & 1) << 1));
}

template <int D, int DT, int HPW, bool FLAT>
__global__ __launch_bounds__(kThreads, 2) void mfa_decode_mq_split_kernel(DecArgs a) {
    constexpr int NKB = D / 32;                  // k-steps of S^T
    constexpr int NDB = D / 16;                  // 16-column blocks of O^T
    constexpr int KCH = D / 8;                   // 16-byte chunks per token row
    constexpr int VLOADS = kPage * KCH / 64;     // direct loads per page (4 or 2)
    constexpr int TILE = kPG * kPage * D;        // 16-bit elements of a wave's V copy
    static_assert(kPG == 2, "two pages per step");
    __shared__ __attribute__((aligned(1024))) uint16_t sv_all[kWaves * TILE];
    __shared__ float sm_m[kWaves][16];
    __shared__ float sm_l[kWaves][16];

    int s, hg, b, L;
    if (!decode_item<FLAT>(a, a.Hq / HPW, &b, &hg, &s, &L)) return;   // (an empty chunk)
    const int h0 = hg * HPW;
    const int kvh = h0 / a.g;
    const int nq = a.nq;

    const int n_pages_b = (L + kPage - 1) / kPage;
    const int page_begin = s * a.chunk_pages;
    const int page_end = min(page_begin + a.chunk_pages, n_pages_b);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = lane >> 4;
    const int c = lane & 15;
    const int ppw = a.chunk_pages / kWaves;
    const int w_begin = page_begin + wave * ppw;
    const int w_end = min(w_begin + ppw, page_end);
    uint16_t* sv = sv_all + wave * TILE;

    // column c of the score tile: query token n_c, head h0 + c % HPW (c >= HPW * nq: unused)
    const bool col_ok = c < HPW * nq;
    const int n_c = c / HPW;
    const int lim = L - nq + n_c;   // last visible key position of row c
    mfa_u32x4 qb[NKB];
    {
        const uint16_t* qp = a.q + (((size_t)b * nq + (col_ok ? n_c : 0)) * a.Hq + h0 + c % HPW) * D;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            qb[kb] = col_ok ? *(const mfa_u32x4*)(qp + (4 * kb + G) * 8) : mfa_u32x4{0u, 0u, 0u, 0u};
    }

    const uint32_t tok_bytes = (uint32_t)a.Hkv * D * 2;
    const uint32_t k_off = (uint32_t)c * tok_bytes;   // A row = token c of the page
    // direct V load i of page j: LDS slots (j * VLOADS + i) * 64 + lane, i.e. step row
    // r = slot / KCH (token r - 16 j of page j), physical chunk slot % KCH, which holds
    // logical chunk dec_v_phys(r, phys); the swizzle depends on r only through bits that
    // do not change with i or j, so one per-lane offset serves every load
    uint32_t v_off;
    {
        const int r = lane / KCH, phys = lane % KCH;
        v_off = (uint32_t)r * tok_bytes + (uint32_t)dec_v_phys<D>(r, phys) * 16;
    }
    constexpr int TOK_PER_LOAD = 64 / KCH;
    // transposing reads: lane group G' = G reads rows 4G' + i / 4 of a page, columns
    // 16 db + 4 (i % 4) .. +3, i = lane % 16
    int v_rd[NDB];
    {
        const int i = lane & 15;
        const int r = 4 * G + (i >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = 16 * db + 4 * (i & 3);
            v_rd[db] = r * D + dec_v_phys<D>(r, col >> 3) * 8 + (col & 7);
        }
    }

    float m_run = -MFA_INF;   // row c's exponent offset (log2 domain), same in its 4 lanes
    float l_run = 0.f;        // this lane's part of row c's sum
    mfa_f32x4 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = mfa_f32x4{0.f, 0.f, 0.f, 0.f};

    const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
    const size_t page_elems = (size_t)kPage * a.Hkv * D;
    // page j of the step at page pg: its offset in the pools, and its valid tokens
    auto page_at = [&](int pg, int j, int pid, int& nvj) {
        const bool pvalid = pid >= 0 && pid < a.num_pages && pg + j < w_end;
        nvj = pvalid ? min(kPage, L - (pg + j) * kPage) : 0;
        return (size_t)(pvalid ? pid : 0) * page_elems + (size_t)kvh * D;
    };
    auto issue_k = [&](int pg, const int (&pid)[kPG], mfa_u32x4 (&kr)[kPG][NKB], int (&nv)[kPG]) {
#pragma unroll
        for (int j = 0; j < kPG; ++j) {
            const size_t pbase = page_at(pg, j, pid[j], nv[j]);
            const auto rk = mfa_rsrc(a.kp + pbase, (uint32_t)nv[j] * tok_bytes);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) kr[j][kb] = mfa_load16_nt(rk, k_off + (4 * kb + G) * 16);
        }
    };
    auto issue_v = [&](int pg, const int (&pid)[kPG]) {
#pragma unroll
        for (int j = 0; j < kPG; ++j) {
            int nvj;
            const size_t pbase = page_at(pg, j, pid[j], nvj);
            const auto rv = mfa_rsrc(a.vp + pbase, (uint32_t)nvj * tok_bytes);
#pragma unroll
            for (int i = 0; i < VLOADS; ++i)
                mfa_load16_lds_nt(rv, sv + (j * VLOADS + i) * 512, v_off + (uint32_t)(i * TOK_PER_LOAD) * tok_bytes);
        }
    };
    auto load_pids = [&](int pg, int (&pid)[kPG]) {
#pragma unroll
        for (int j = 0; j < kPG; ++j) pid[j] = pg + j < w_end ? mfa_uniform_load(bt + pg + j) : -1;
    };

    // Pipelined: the next step's K loads are issued once this step's score products have
    // read the K registers, and its V copies once this step's P V reads have returned, so
    // both are in flight during this step's softmax and products.  Page ids are read two
    // steps ahead.
    int pid_nx[kPG];
    mfa_u32x4 kr[kPG][NKB];
    int nv[kPG];
    {
        int pid0[kPG];
        load_pids(w_begin, pid0);
        load_pids(w_begin + kPG, pid_nx);
        if (w_begin < w_end) {
            issue_k(w_begin, pid0, kr, nv);
            issue_v(w_begin, pid0);
        }
    }
    for (int pg = w_begin; pg < w_end; pg += kPG) {
        const bool more = pg + kPG < w_end;   // uniform
        // scores (log2 domain), masked: position p visible iff p < L and p <= lim
        float x[kPG][4];
#pragma unroll
        for (int j = 0; j < kPG; ++j) {
            mfa_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) acc = mfa_mfma16<DT>(kr[j][kb], qb[kb], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * G + i;
                const bool vis = t < nv[j] && (pg + j) * kPage + t <= lim;
                x[j][i] = vis ? acc[i] * a.scale_log2 : -MFA_INF;
            }
        }
        int nv_n[kPG];
        if (more) issue_k(pg + kPG, pid_nx, kr, nv_n);
        float tmax = -MFA_INF;
#pragma unroll
        for (int j = 0; j < kPG; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, x[j][i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const bool raise = tmax > m_run + kLazy;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
            const float m_new = raise ? tmax : m_run;
            const float alpha = (m_run == -MFA_INF) ? 0.f : mfa_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
            m_run = m_new;
        }
        const float m_use = (m_run == -MFA_INF) ? 0.f : m_run;
        mfa_u32x4 pb;
#pragma unroll
        for (int j = 0; j < kPG; ++j)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float p0 = mfa_exp2(x[j][2 * e] - m_use);
                const float p1 = mfa_exp2(x[j][2 * e + 1] - m_use);
                const uint32_t pk = mfa_pack2<DT>(p0, p1);
                pb[2 * j + e] = pk;
                if constexpr (DT == MFA_DT_F16)
                    l_run = mfa_sum2<DT>(pk, l_run);
                else
                    l_run += p0 + p1;
            }

        // O^T += V^T P^T from the wave's LDS copy of the two pages: this step's V copies
        // have landed once at most the next step's kPG * NKB K loads are outstanding
        static_assert(kPG * NKB == 8 || kPG * NKB == 4, "vmcnt immediate");
        if (more) {
            if constexpr (kPG * NKB == 8)
                __builtin_amdgcn_s_waitcnt(0x0f78);   // vmcnt(8)
            else
                __builtin_amdgcn_s_waitcnt(0x0f74);   // vmcnt(4)
        } else {
            __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const mfa_u32x2 lo = mfa_lds_read_tr16(sv + v_rd[db]);
            const mfa_u32x2 hi = mfa_lds_read_tr16(sv + kPage * D + v_rd[db]);
            oacc[db] = mfa_mfma16<DT>(mfa_u32x4{lo[0], lo[1], hi[0], hi[1]}, pb, oacc[db]);
        }
        // the next step's copies overwrite the buffer: its reads must have returned
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
        if (more) {
            issue_v(pg + kPG, pid_nx);
#pragma unroll
            for (int j = 0; j < kPG; ++j) nv[j] = nv_n[j];
            load_pids(pg + 2 * kPG, pid_nx);
        }
    }

    // merge the four waves' partial states of each row in LDS (reusing the V buffers)
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);   // the row's four lanes: c + 16 G
    l_tot += __shfl_xor(l_tot, 32, 64);
    __syncthreads();
    float* sm_o = reinterpret_cast<float*>(sv_all);   // [kWaves][16][D]
    static_assert(kWaves * 16 * D * 4 <= kWaves * TILE * 2, "merge buffer fits");
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        *(mfa_f32x4*)&sm_o[(wave * 16 + c) * D + 16 * db + 4 * G] = oacc[db];
    if (G == 0) {
        sm_m[wave][c] = m_run;
        sm_l[wave][c] = l_tot;
    }
    __syncthreads();
    const int R = HPW * nq;
    for (int idx = tid; idx < R * D; idx += kThreads) {
        const int row = idx / D, d = idx - row * D;
        float M = -MFA_INF;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][row]);
        float lt = 0.f, ot = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = (sm_m[w][row] == -MFA_INF) ? 0.f : mfa_exp2(sm_m[w][row] - M);
            lt += f * sm_l[w][row];
            ot += f * sm_o[(w * 16 + row) * D + d];
        }
        const int n = row / HPW, hh = row - n * HPW;
        const size_t slot = (((size_t)b * nq + n) * a.Hq + h0 + hh) * a.S + s;
        a.ws_o[slot * D + d] = lt > 0.f ? ot / lt : 0.f;
        if (d == 0) a.ws_lse[slot] = lt > 0.f ? M + mfa_log2(lt) : -MFA_INF;
    }
}

// One workgroup of 256 threads per (sequence, token, head).  The splits are taken in
// chunks of ROWS * KPT: thread (row r, column group c) loads the LSE and the 4 columns
// 4c .. 4c + 3 of splits r, r + ROWS, ... of the chunk, all at once, and keeps a running
// (max, weight sum, weighted O) for its row, rescaled when a chunk raises the max.  The
// ROWS rows are then merged in LDS with the same rule:
//   M = max_r m_r,  W = sum_r 2^(m_r - M) w_r,  O = sum_r 2^(m_r - M) o_r / W.
template <int D, int DT>
__global__ __launch_bounds__(256) void mfa_decode_combine_kernel(DecArgs a) {
    constexpr int TPR = D / 4;          // threads per split row (one float4 each)
    constexpr int ROWS = 256 / TPR;     // split rows per chunk
    constexpr int KPT = 8;              // splits per thread per chunk
    const int bh = blockIdx.x;   // (b * nq + n) * Hq + h
    const int b = bh / (a.Hq * a.nq);
    const int t = threadIdx.x;
    const int c = t % TPR, r = t / TPR;
    const int L = clamp_len(a.seq_lens[b], a.max_pages);
    const int n_pages_b = (L + kPage - 1) / kPage;
    const int n_used = (n_pages_b + a.chunk_pages - 1) / a.chunk_pages;
    const float* lse_s = a.ws_lse + (size_t)bh * a.S;
    const float* o_s = a.ws_o + (size_t)bh * a.S * D + 4 * c;

    float m = -MFA_INF, w = 0.f;
    mfa_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int base = 0; base < n_used; base += ROWS * KPT) {
        float ls[KPT];
        mfa_f32x4 ov[KPT];
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int s = base + r + ROWS * k;
            const bool ok = s < n_used;
            ls[k] = ok ? lse_s[s] : -MFA_INF;
            ov[k] = ok ? *(const mfa_f32x4*)(o_s + (size_t)s * D) : mfa_f32x4{0.f, 0.f, 0.f, 0.f};
        }
        float mc = m;
#pragma unroll
        for (int k = 0; k < KPT; ++k) mc = fmaxf(mc, ls[k]);
        if (mc == -MFA_INF) continue;   // nothing seen yet (uniform per row)
        const float f = (m == -MFA_INF) ? 0.f : mfa_exp2(m - mc);
        w *= f;
        acc *= f;
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const float e = (ls[k] == -MFA_INF) ? 0.f : mfa_exp2(ls[k] - mc);
            w += e;
            acc += e * ov[k];
        }
        m = mc;
    }

    __shared__ mfa_f32x4 sm_acc[ROWS][TPR];
    __shared__ float sm_m[ROWS], sm_w[ROWS];
    sm_acc[r][c] = acc;
    if (c == 0) {
        sm_m[r] = m;
        sm_w[r] = w;
    }
    __syncthreads();
    if (t >= TPR) return;
    float M = -MFA_INF;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) M = fmaxf(M, sm_m[i]);
    const float M_use = (M == -MFA_INF) ? 0.f : M;
    float Wt = 0.f;
    mfa_f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const float f = (sm_m[i] == -MFA_INF) ? 0.f : mfa_exp2(sm_m[i] - M_use);
        Wt += f * sm_w[i];
        o += f * sm_acc[i][t];
    }
    const float inv = Wt > 0.f ? 1.f / Wt : 0.f;
    mfa_u32x2 packed;
    packed[0] = mfa_pack2<DT>(o[0] * inv, o[1] * inv);
    packed[1] = mfa_pack2<DT>(o[2] * inv, o[3] * inv);
    *(mfa_u32x2*)(a.out + (size_t)bh * D + 4 * t) = packed;
    if (a.lse != nullptr && t == 0) a.lse[bh] = Wt > 0.f ? (M_use + mfa_log2(Wt)) * MFA_LN2 : -MFA_INF;
}

// Grid of the split kernels: every (chunk, head group, sequence), flattened when FLAT.
dim3 split_grid(const DecArgs& a, int HPW, bool flat) {
    if (flat) return dim3((unsigned)(a.S * (a.Hq / HPW) * a.B), 1, 1);
    return dim3((unsigned)a.S, (unsigned)(a.Hq / HPW), (unsigned)a.B);
}
bool use_flat(const DecArgs& a, int HPW) {
    return a.B <= kFlatMaxB && (long long)a.S * (a.Hq / HPW) * a.B <= 0x7fffffffLL;
}

template <int D, int DT, int HPW>
int launch(const DecArgs& a, hipStream_t stream, mfa_dispatch_info* info) {
    const bool flat = use_flat(a, HPW);
    const dim3 grid1 = split_grid(a, HPW, flat);
    if (flat)
        hipLaunchKernelGGL((mfa_decode_split_kernel<D, DT, HPW, true>), grid1, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((mfa_decode_split_kernel<D, DT, HPW, false>), grid1, dim3(kThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MFA_ERR_HIP;
    hipLaunchKernelGGL((mfa_decode_combine_kernel<D, DT>), dim3((unsigned)(a.B * a.Hq)), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MFA_ERR_HIP;
    snprintf(info->kernel, sizeof(info->kernel), "mfa_decode_split_kernel<D=%d,%s,HPW=%d%s>", D,
             DT == MFA_DT_F16 ? "f16" : "bf16", HPW, flat ? ",flat" : "");
    info->grid[0] = (int)grid1.x;
    info->grid[1] = (int)grid1.y;
    info->grid[2] = (int)grid1.z;
    info->block = kThreads;
    info->waves = kWaves;
    info->n_launches = 2;
    return MFA_OK;
}

template <int D, int DT>
int launch_hpw(const DecArgs& a, hipStream_t stream, mfa_dispatch_info* info) {
    if (a.g % 4 == 0) return launch<D, DT, 4>(a, stream, info);
    if (a.g % 2 == 0) return launch<D, DT, 2>(a, stream, info);
    return launch<D, DT, 1>(a, stream, info);
}

template <int D, int DT, int HPW>
int launch_mq(const DecArgs& a, hipStream_t stream, mfa_dispatch_info* info) {
    const bool flat = use_flat(a, HPW);
    const dim3 grid1 = split_grid(a, HPW, flat);
    if (flat)
        hipLaunchKernelGGL((mfa_decode_mq_split_kernel<D, DT, HPW, true>), grid1, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((mfa_decode_mq_split_kernel<D, DT, HPW, false>), grid1, dim3(kThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MFA_ERR_HIP;
    hipLaunchKernelGGL((mfa_decode_combine_kernel<D, DT>), dim3((unsigned)(a.B * a.nq * a.Hq)), dim3(256), 0,
                       stream, a);
    if (hipGetLastError() != hipSuccess) return MFA_ERR_HIP;
    snprintf(info->kernel, sizeof(info->kernel), "mfa_decode_mq_split_kernel<D=%d,%s,HPW=%d,nq=%d%s>", D,
             DT == MFA_DT_F16 ? "f16" : "bf16", HPW, a.nq, flat ? ",flat" : "");
    info->grid[0] = (int)grid1.x;
    info->grid[1] = (int)grid1.y;
    info->grid[2] = (int)grid1.z;
    info->block = kThreads;
    info->waves = kWaves;
    info->n_launches = 2;
    return MFA_OK;
}

// Query heads per workgroup: the largest of 4, 2, 1 that divides g with HPW * nq <= 16.
template <int D, int DT>
int launch_mq_hpw(const DecArgs& a, hipStream_t stream, mfa_dispatch_info* info) {
    if (a.g % 4 == 0 && 4 * a.nq <= 16) return launch_mq<D, DT, 4>(a, stream, info);
    if (a.g % 2 == 0 && 2 * a.nq <= 16) return launch_mq<D, DT, 2>(a, stream, info);
    return launch_mq<D, DT, 1>(a, stream, info);
}

}  // namespace

// Fixed scratch for callers that cannot allocate (mfa_decode_paged_noalloc): the split
// partials live in this file-scope device array instead of a caller workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  On the host the array's
// name is not a device address: host code uses only the address hipGetSymbolAddress gives
// for the current device, looked up once per device on its first call.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kDecodeScratchBytes];

int mfa_decode_scratch(void** ptr, size_t* bytes) {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MFA_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return MFA_ERR_HIP;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = kDecodeScratchBytes;
    return MFA_OK;
}

int mfa_decode_chunk_pages(int max_pages_per_seq, int num_splits, int nq) {
    // Auto, one new token: about 32 splits per sequence of maximal length, between 8 and
    // 64 pages (128 .. 1024 tokens) per split (on the decode workload 1024-token chunks
    // measured 199 us per call against 204 us with 512-token ones).  Several new tokens:
    // about 24 splits, up to 128 pages each; their partials are nq times larger, and on
    // the 4-token decode workload 1408-token chunks measured 182 us against 198 us with
    // 512-token ones.  Chunks are a multiple of 8 pages (2 per wave).
    int want;
    if (num_splits > 0)
        want = (max_pages_per_seq + num_splits - 1) / num_splits;
    else
        want = nq > 1 ? max_pages_per_seq / 24 : max_pages_per_seq / 32;
    int c = ((want + 7) / 8) * 8;
    if (c < 8) c = 8;
    const int cap = nq > 1 ? 128 : 64;
    if (num_splits == 0 && c > cap) c = cap;
    return c;
}

int mfa_decode_launch(const MfaDecodeProblem& pr, hipStream_t stream, mfa_dispatch_info* info) {
    DecArgs a;
    a.q = (const uint16_t*)pr.q;
    a.kp = (const uint16_t*)pr.k_pages;
    a.vp = (const uint16_t*)pr.v_pages;
    a.block_table = pr.block_table;
    a.seq_lens = pr.seq_lens;
    a.out = (uint16_t*)pr.out;
    a.lse = pr.lse;
    a.B = pr.B;
    a.Hq = pr.Hq;
    a.Hkv = pr.Hkv;
    a.g = pr.Hq / pr.Hkv;
    a.nq = pr.nq;
    a.num_pages = pr.num_pages;
    a.max_pages = pr.max_pages_per_seq;
    a.chunk_pages = pr.chunk_pages;
    a.S = pr.num_splits;
    a.scale_log2 = pr.scale * 1.4426950408889634f;
    a.ws_o = (float*)pr.workspace;
    a.ws_lse = a.ws_o + (size_t)pr.B * pr.nq * pr.Hq * pr.num_splits * pr.D;
    info->num_splits = a.S;
    info->chunk_tokens = a.chunk_pages * kPage;
    if (pr.multi) {
        if (pr.D == 128)
            return pr.dtype == MFA_F16 ? launch_mq_hpw<128, MFA_DT_F16>(a, stream, info)
                                       : launch_mq_hpw<128, MFA_DT_BF16>(a, stream, info);
        return pr.dtype == MFA_F16 ? launch_mq_hpw<64, MFA_DT_F16>(a, stream, info)
                                   : launch_mq_hpw<64, MFA_DT_BF16>(a, stream, info);
    }
    if (pr.D == 128)
        return pr.dtype == MFA_F16 ? launch_hpw<128, MFA_DT_F16>(a, stream, info)
                                   : launch_hpw<128, MFA_DT_BF16>(a, stream, info);
    return pr.dtype == MFA_F16 ? launch_hpw<64, MFA_DT_F16>(a, stream, info)
                               : launch_hpw<64, MFA_DT_BF16>(a, stream, info);
}
