// Paged split-KV flash-decode for gfx950: one query token per sequence against a
// paged KV cache.
//
// Pass 1 (mfa_decode_split_kernel): the cached tokens of every sequence are cut into
// contiguous chunks of logical token positions; one workgroup handles one chunk of one
// (sequence, group of query heads sharing a KV head) and writes a partial result
// (O_s normalised, LSE_s) to the workspace.  Pass 2 (mfa_decode_combine_kernel) merges
// the partials of each (sequence, head): M = max_s LSE_s, w_s = exp(LSE_s - M),
// O = sum w_s O_s / sum w_s, LSE = M + log sum w_s.  This is the two-phase split-KV
// decode of the mlx-mfa 2.5.2 page ("Flash Decode", "V2 split-K") over the page pool
// and block table of its "Paged KV" feature and of the MXFlashAttn 1.5.0 page (M1
// paged Split-KV decode).  Every split owns its own workspace slots and writes only
// the slots of its own heads (the per-split slot race described on the MXFlashAttn
// page came from lanes of invalid query heads writing into a neighbour's slot).
//
// Inside a workgroup (4 waves, each a contiguous run of pages of the chunk):
//   lane = (G = lane / 16, t = lane % 16).  Page slot t is token t of the page.
//   S = Q K^T on a 16x16x32 MFMA: the A operand holds the workgroup's query heads,
//   replicated over the 16 rows, so that every lane's accumulator holds the scores of
//   all those heads for token t; the B operand is read straight from the page (16-byte
//   loads, lane group G reads one 64-byte quarter of each K row).
//   Each lane then keeps its own running (m, l, o) per head for the tokens in slot t
//   of its pages (o over the D/4 columns it loaded from V) — an online softmax per
//   lane, so no cross-lane reduction is needed inside the loop.  At the end the 16
//   slots are merged with DPP row reductions, and the 4 waves through LDS.
// Tokens at or past seq_lens[b] (tail slots of the last page, which may hold any bit
// pattern) are neither loaded nor counted: their scores are -inf and their V rows 0.
#include "mfa_device.h"
#include "mfa_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kPage = 16;
constexpr int kPG = 2;   // pages per online-softmax step of a lane

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
    int num_pages, max_pages;
    int S, chunk_pages;
    float scale_log2;
};

__device__ __forceinline__ int clamp_len(int L, int max_pages) {
    const int cap = max_pages * kPage;
    return L < 0 ? 0 : (L > cap ? cap : L);
}

template <int D, int DT, int HPW>
__global__ __launch_bounds__(kThreads) void mfa_decode_split_kernel(DecArgs a) {
    constexpr int NKB = D / 32;     // 16-byte chunks per lane per K/V row
    constexpr int NO = NKB * 8;     // output columns per lane
    const int s = blockIdx.x;
    const int hg = blockIdx.y;
    const int b = blockIdx.z;
    const int h0 = hg * HPW;
    const int kvh = h0 / a.g;

    const int L = clamp_len(a.seq_lens[b], a.max_pages);
    const int n_pages_b = (L + kPage - 1) / kPage;
    const int page_begin = s * a.chunk_pages;
    if (page_begin >= n_pages_b) return;   // empty split: its slots are neither written nor read
    const int page_end = min(page_begin + a.chunk_pages, n_pages_b);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int G = lane >> 4;
    const int t16 = lane & 15;
    const int ppw = a.chunk_pages / kWaves;
    const int w_begin = page_begin + wave * ppw;
    const int w_end = min(w_begin + ppw, page_end);

    // A operand: head (t16 % HPW) of the group, k-chunks 4*kb + G
    mfa_u32x4 qa[NKB];
    {
        const uint16_t* qp = a.q + ((size_t)b * a.Hq + h0 + (t16 % HPW)) * D;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) qa[kb] = *(const mfa_u32x4*)(qp + (4 * kb + G) * 8);
    }

    float m[HPW], l[HPW], o[HPW][NO];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        m[hh] = -MFA_INF;
        l[hh] = 0.f;
#pragma unroll
        for (int i = 0; i < NO; ++i) o[hh][i] = 0.f;
    }

    const size_t tok_stride = (size_t)a.Hkv * D;
    const int32_t* bt = a.block_table + (size_t)b * a.max_pages;

    for (int pg = w_begin; pg < w_end; pg += kPG) {
        mfa_u32x4 kr[kPG][NKB], vr[kPG][NKB];
        bool tv[kPG];
#pragma unroll
        for (int j = 0; j < kPG; ++j) {
            const int pi = pg + j;
            int pid = pi < w_end ? bt[pi] : -1;
            const bool pvalid = pid >= 0 && pid < a.num_pages;
            tv[j] = pvalid && (pi * kPage + t16) < L;
            const size_t base = ((size_t)(pvalid ? pid : 0) * kPage + t16) * tok_stride + (size_t)kvh * D;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                kr[j][kb] = tv[j] ? *(const mfa_u32x4*)(a.kp + base + (4 * kb + G) * 8) : mfa_u32x4{0, 0, 0, 0};
                vr[j][kb] = tv[j] ? *(const mfa_u32x4*)(a.vp + base + (4 * kb + G) * 8) : mfa_u32x4{0, 0, 0, 0};
            }
        }
        float sc[kPG][HPW];
#pragma unroll
        for (int j = 0; j < kPG; ++j) {
            mfa_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) acc = mfa_mfma16<DT>(qa[kb], kr[j][kb], acc);
#pragma unroll
            for (int hh = 0; hh < HPW; ++hh) sc[j][hh] = tv[j] ? acc[hh] * a.scale_log2 : -MFA_INF;
        }
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
            float mb = sc[0][hh];
#pragma unroll
            for (int j = 1; j < kPG; ++j) mb = fmaxf(mb, sc[j][hh]);
            const float m_new = fmaxf(m[hh], mb);
            const float m_use = (m_new == -MFA_INF) ? 0.f : m_new;
            const float alpha = mfa_exp2(m[hh] - m_use);
            float p[kPG];
            float ps = 0.f;
#pragma unroll
            for (int j = 0; j < kPG; ++j) {
                p[j] = mfa_exp2(sc[j][hh] - m_use);
                ps += p[j];
            }
            l[hh] = l[hh] * alpha + ps;
            m[hh] = m_new;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    float x0 = o[hh][kb * 8 + 2 * e2] * alpha;
                    float x1 = o[hh][kb * 8 + 2 * e2 + 1] * alpha;
#pragma unroll
                    for (int j = 0; j < kPG; ++j) {
                        x0 += p[j] * mfa_lo<DT>(vr[j][kb][e2]);
                        x1 += p[j] * mfa_hi<DT>(vr[j][kb][e2]);
                    }
                    o[hh][kb * 8 + 2 * e2] = x0;
                    o[hh][kb * 8 + 2 * e2 + 1] = x1;
                }
            }
        }
    }

    // merge the 16 token slots of each DPP row (same columns, different tokens)
    __shared__ float sm_m[kWaves][HPW];
    __shared__ float sm_l[kWaves][HPW];
    __shared__ __attribute__((aligned(16))) float sm_o[kWaves][HPW][D];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        const float M = mfa_row16_max(m[hh]);
        const float f = (m[hh] == -MFA_INF) ? 0.f : mfa_exp2(m[hh] - M);
        const float lr = mfa_row16_sum(l[hh] * f);
#pragma unroll
        for (int i = 0; i < NO; ++i) o[hh][i] = mfa_row16_sum(o[hh][i] * f);
        if (t16 == 0) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                float* dst = &sm_o[wave][hh][(4 * kb + G) * 8];
                *(mfa_f32x4*)dst = mfa_f32x4{o[hh][kb * 8 + 0], o[hh][kb * 8 + 1], o[hh][kb * 8 + 2], o[hh][kb * 8 + 3]};
                *(mfa_f32x4*)(dst + 4) = mfa_f32x4{o[hh][kb * 8 + 4], o[hh][kb * 8 + 5], o[hh][kb * 8 + 6], o[hh][kb * 8 + 7]};
            }
            if (G == 0) {
                sm_m[wave][hh] = M;
                sm_l[wave][hh] = lr;
            }
        }
    }
    __syncthreads();

    // merge the waves and write this split's partial (O_s, LSE_s) per head
    for (int idx = tid; idx < HPW * D; idx += kThreads) {
        const int hh = idx / D, d = idx - hh * D;
        float M = -MFA_INF;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][hh]);
        float lt = 0.f, ot = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = (sm_m[w][hh] == -MFA_INF) ? 0.f : mfa_exp2(sm_m[w][hh] - M);
            lt += f * sm_l[w][hh];
            ot += f * sm_o[w][hh][d];
        }
        const size_t slot = ((size_t)b * a.Hq + h0 + hh) * a.S + s;
        a.ws_o[slot * D + d] = lt > 0.f ? ot / lt : 0.f;
        if (d == 0) a.ws_lse[slot] = lt > 0.f ? M + mfa_log2(lt) : -MFA_INF;
    }
}

template <int D, int DT>
__global__ __launch_bounds__(64) void mfa_decode_combine_kernel(DecArgs a) {
    constexpr int PER = D / 64;
    const int bh = blockIdx.x;
    const int b = bh / a.Hq;
    const int lane = threadIdx.x;
    const int L = clamp_len(a.seq_lens[b], a.max_pages);
    const int n_pages_b = (L + kPage - 1) / kPage;
    const int n_used = (n_pages_b + a.chunk_pages - 1) / a.chunk_pages;
    const float* lse_s = a.ws_lse + (size_t)bh * a.S;
    const float* o_s = a.ws_o + (size_t)bh * a.S * D;

    float M = -MFA_INF;
    for (int s = lane; s < n_used; s += 64) M = fmaxf(M, lse_s[s]);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x, 64));
    const float M_use = (M == -MFA_INF) ? 0.f : M;

    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    float W = 0.f;
    for (int s = 0; s < n_used; ++s) {
        const float ls = lse_s[s];
        const float w = (ls == -MFA_INF) ? 0.f : mfa_exp2(ls - M_use);
        W += w;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] += w * o_s[(size_t)s * D + lane * PER + i];
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    uint16_t* op = a.out + (size_t)bh * D + lane * PER;
    if constexpr (PER == 2) {
        *(uint32_t*)op = mfa_pack2<DT>(acc[0] * inv, acc[1] * inv);
    } else {
        const uint32_t w2 = mfa_pack2<DT>(acc[0] * inv, 0.f);
        *op = (uint16_t)(w2 & 0xffffu);
    }
    if (a.lse != nullptr && lane == 0) a.lse[bh] = W > 0.f ? (M_use + mfa_log2(W)) * MFA_LN2 : -MFA_INF;
}

template <int D, int DT, int HPW>
int launch(const DecArgs& a, hipStream_t stream, mfa_dispatch_info* info) {
    const dim3 grid1((unsigned)a.S, (unsigned)(a.Hq / HPW), (unsigned)a.B);
    hipLaunchKernelGGL((mfa_decode_split_kernel<D, DT, HPW>), grid1, dim3(kThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MFA_ERR_HIP;
    hipLaunchKernelGGL((mfa_decode_combine_kernel<D, DT>), dim3((unsigned)(a.B * a.Hq)), dim3(64), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MFA_ERR_HIP;
    snprintf(info->kernel, sizeof(info->kernel), "mfa_decode_split_kernel<D=%d,%s,HPW=%d>", D,
             DT == MFA_DT_F16 ? "f16" : "bf16", HPW);
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

}  // namespace

int mfa_decode_chunk_pages(int max_pages_per_seq, int num_splits) {
    // Auto: about 16 splits per sequence of maximal length, between 8 and 32 pages
    // (128 .. 512 tokens) per split.  Chunks are a multiple of 8 pages (2 per wave).
    int want;
    if (num_splits > 0)
        want = (max_pages_per_seq + num_splits - 1) / num_splits;
    else
        want = max_pages_per_seq / 16;
    int c = ((want + 7) / 8) * 8;
    if (c < 8) c = 8;
    if (num_splits == 0 && c > 32) c = 32;
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
    a.num_pages = pr.num_pages;
    a.max_pages = pr.max_pages_per_seq;
    a.chunk_pages = pr.chunk_pages;
    a.S = pr.num_splits;
    a.scale_log2 = pr.scale * 1.4426950408889634f;
    a.ws_o = (float*)pr.workspace;
    a.ws_lse = a.ws_o + (size_t)pr.B * pr.Hq * pr.num_splits * pr.D;
    info->num_splits = a.S;
    info->chunk_tokens = a.chunk_pages * kPage;
    if (pr.D == 128)
        return pr.dtype == MFA_F16 ? launch_hpw<128, MFA_DT_F16>(a, stream, info)
                                   : launch_hpw<128, MFA_DT_BF16>(a, stream, info);
    return pr.dtype == MFA_F16 ? launch_hpw<64, MFA_DT_F16>(a, stream, info)
                               : launch_hpw<64, MFA_DT_BF16>(a, stream, info);
}
