// Fused exact-attention forward for gfx950.
//
// Computes O = softmax(scale * Q K^T + mask) V and LSE = log(sum exp(scaled scores))
// tile by tile with an fp32 online softmax (running max m and sum l per query row),
// as in the FlashAttention-2 forward shader of the mlx-bun flash-attention.ts page:
// per key tile, m' = max(m, rowmax S); alpha = exp(m - m'); P = exp(S - m');
// l = alpha * l + rowsum P; O = alpha * O + P V; at the end O / l and m + log l.
// That shader runs one thread per query row with scalar dot products; here both
// contractions run on the CDNA4 matrix cores instead.
//
// Work decomposition
//   One workgroup = 4 waves = one query tile of BM = 128 rows of one (batch, head).
//   Each wave owns 32 query rows.  Key tiles of BN keys are streamed through LDS,
//   double-buffered: the global loads of tile j+1 are in flight while tile j is
//   consumed, and one barrier per tile separates the buffers.  Global loads go
//   through buffer resources, whose range check returns zeros past the last key row.
//
// Per wave and key tile (32x32x16 MFMA, fp32 accumulate):
//   S^T = K Q^T: A = K rows (keys) from LDS, B = Q^T held in registers for the whole
//     kernel.  The accumulator puts one query row in each lane (lane % 32) and 16 of
//     the 32 keys of a block in its registers, so the row max needs one exchange with
//     lane ^ 32 and the row sum none until the end.
//   The K rows fed to the A operand are permuted (key_perm) so that accumulator
//   register r of lane half g holds key 16*(r/8) + 8*g + r%8: each lane then owns runs
//   of 8 consecutive keys, which is exactly the B operand layout of the next product.
//   O^T += V^T P^T: A = V^T from LDS (V is transposed while it is written to LDS),
//     B = P^T straight from the softmax registers (rounded to the input type).  The
//     O^T accumulator again has one query row per lane, so rescaling is a per-lane
//     scalar multiply.
//
// Softmax details (all in the log2 domain; scale * log2(e) is folded into one FMA that
// feeds the exponential):
//   * The running max used as the exponent offset is only raised when a row's new
//     maximum exceeds it by more than 2^8 (kLazy), so P <= 256 and O, l are rescaled
//     only on those (rare) tiles; the result is the same up to rounding because the
//     offset cancels in O = o / l and enters LSE as m + log2 l.
//   * For fp16, l accumulates the P values after rounding to fp16 (one dot2 per pair),
//     i.e. exactly the weights the P V product uses; for bf16, whose rounding is 8x
//     coarser, l sums the fp32 values so that the LSE keeps fp32 accuracy.
//
// Masking and skipping (mlx-mfa 2.5.2 features "Causal tile-skip", "Sliding window";
// mlx-bun forward shader's fully-masked-tile guard): the workgroup visits only the key
// tiles of mfa_tile_range; element masks are applied only on tiles that
// mfa_tile_full rejects; a row whose offset is still -inf uses 0 in its place so exp
// never sees (-inf) - (-inf), and masked scores get P = 0 explicitly.
#include "mfa_device.h"
#include "mfa_geometry.h"
#include "mfa_internal.h"

namespace {

constexpr int kBM = 128;
constexpr int kThreads = 256;
constexpr float kLazy = 8.0f;

struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int32_t* tile_log;
    int B, Hq, Hkv, Nq, Nk, g;
    int n_q_tiles;
    int HB;          // B * Hq
    int xcd_group;   // 1: group the query heads of one KV head on one XCD
    int snake;       // 1: pair heavy and light query tiles (grid fits in one pass)
    float scale_log2_abs;  // |scale| * log2(e)
    MfaMask mask;
};

// K row (within a 32-key block) fed to A-operand row i.
__device__ __forceinline__ int key_perm(int i) {
    return 16 * (i >> 4) + 8 * ((i >> 2) & 1) + 4 * ((i >> 3) & 1) + (i & 3);
}

template <int D, int BN>
struct Tile {
    static constexpr int KCH = D / 8;              // 16-byte chunks per K row
    static constexpr int VCH = BN / 8;             // 16-byte chunks per V^T row
    // Rows are padded by 16 bytes: 16 consecutive rows read at one column then fall
    // into 16 distinct 16-byte bank groups (conflict-free MFMA operand reads), and
    // every operand address is a per-lane base plus a compile-time offset.
    static constexpr int KP = D + 8;               // K row pitch (elements)
    static constexpr int VP = BN + 8;              // V^T row pitch (elements)
    static constexpr int K_ELEMS = BN * KP;        // 16-bit elements per K buffer
    static constexpr int V_ELEMS = D * VP;
    static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
    static constexpr int K_LOADS = BN * KCH / kThreads;   // 16-byte K loads per thread
    static constexpr int VW = D * BN / (8 * kThreads);    // V columns per thread (8 keys each)
    static constexpr int VGROUPS = D / VW;                // column groups of V
    static_assert(BN * KCH % kThreads == 0, "K tile must split evenly");
    static_assert(VW == 2 || VW == 4, "V tile: one 8-key x VW-column block per thread");

    __device__ static __forceinline__ int k_off(int row, int ch) { return row * KP + ch * 8; }
    __device__ static __forceinline__ int v_off(int d, int ch) { return K_ELEMS + d * VP + ch * 8; }
};

template <int D, int DT, int BN, bool TILELOG, bool NEG>
__global__ __launch_bounds__(kThreads, 2) void mfa_fwd_kernel(FwdArgs a) {
    using T = Tile<D, BN>;
    constexpr int NKB = D / 16;   // k-steps of S^T = K Q^T
    constexpr int NDB = D / 32;   // 32-row blocks of O^T
    constexpr int NNB = BN / 32;  // 32-key blocks of a tile

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::BUF_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g32 = lane >> 5;
    const int l32 = lane & 31;

    // ---- which (query tile, batch, head) -------------------------------------------
    const int id = blockIdx.x;
    const int round = id / a.HB;
    const int w = id - round * a.HB;
    int qt;
    if (a.snake) {
        // first half of the grid: heaviest tiles downwards; second half: lightest
        // upwards, so the two workgroups sharing a CU carry complementary work
        const int half = (a.n_q_tiles + 1) >> 1;
        qt = round < half ? a.n_q_tiles - 1 - round : round - half;
    } else {
        qt = a.n_q_tiles - 1 - round;   // longest first
    }
    int b, h;
    if (a.xcd_group) {
        // consecutive workgroups go to different XCDs (id % 8); keep every query head
        // of one (batch, KV head) on the same XCD so its K/V stay in that L2
        const int x = w & 7, j = w >> 3;
        const int pair = x + 8 * (j / a.g);
        b = pair / a.Hkv;
        h = (pair - b * a.Hkv) * a.g + (j % a.g);
    } else {
        b = w / a.Hq;
        h = w - b * a.Hq;
    }
    const int kvh = h / a.g;
    const int q0 = qt * kBM;

    int kt_lo, kt_hi;
    mfa_tile_range(a.mask, a.Nq, kBM, BN, qt, &kt_lo, &kt_hi);

    const size_t head_q = (size_t)(b * a.Hq + h) * (size_t)a.Nq;
    const size_t head_kv = (size_t)(b * a.Hkv + kvh) * (size_t)a.Nk;
    const uint16_t* kg = a.k + head_kv * D;
    const uint16_t* vg = a.v + head_kv * D;

    const int qrow = q0 + wave * 32 + l32;
    const bool qvalid = qrow < a.Nq;

    // ---- Q^T operand in registers (rows past Nq read as zero) --------------------
    mfa_u32x4 qreg[NKB];
    {
        const auto rq = mfa_rsrc(a.q + head_q * D, (uint32_t)a.Nq * D * 2);
        const uint32_t off = ((uint32_t)qrow * D + g32 * 8) * 2;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) qreg[kb] = mfa_load16(rq, off + kb * 32);
    }

    // per-row visible key bounds (inclusive), clamped into int range
    const int64_t rlo64 = mfa_row_lo(a.mask, qrow);
    const int64_t rhi64 = mfa_row_hi(a.mask, qrow);
    const int row_lo = rlo64 > a.Nk ? a.Nk : (int)rlo64;
    const int row_hi = rhi64 < -1 ? -1 : (int)rhi64;

    mfa_f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = mfa_f32x16{};
    float m_run = -MFA_INF;   // exponent offset (log2 domain, scaled)
    float l_run = 0.f;        // this lane's half of the row sum

    // ---- loader mapping ----------------------------------------------------------
    // K: 16-byte chunks; V: an 8-key x VW-column block per thread, transposed into V^T.
    constexpr int VW = T::VW;
    const int v_c = tid % T::VGROUPS;
    const int v_a = tid / T::VGROUPS;
    uint32_t k_voff[T::K_LOADS];
#pragma unroll
    for (int p = 0; p < T::K_LOADS; ++p) {
        const int c = p * kThreads + tid;
        k_voff[p] = (uint32_t)((c / T::KCH) * D + (c % T::KCH) * 8) * 2;
    }
    const uint32_t v_voff = (uint32_t)(v_a * 8 * D + v_c * VW) * 2;
    mfa_u32x4 kreg[T::K_LOADS];
    mfa_u32x2 vreg[8];   // VW == 2 uses the first word only

    auto load_tile = [&](int kt) {
        const int k0 = kt * BN;
        const uint32_t bytes = (uint32_t)(a.Nk - k0) * D * 2;
        const auto rk = mfa_rsrc(kg + (size_t)k0 * D, bytes);
        const auto rv = mfa_rsrc(vg + (size_t)k0 * D, bytes);
#pragma unroll
        for (int p = 0; p < T::K_LOADS; ++p) kreg[p] = mfa_load16(rk, k_voff[p]);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if constexpr (VW == 4) {
                vreg[r] = mfa_load8(rv, v_voff + r * D * 2);
            } else {
                vreg[r][0] = mfa_load4(rv, v_voff + r * D * 2);
                vreg[r][1] = 0;
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* s = smem + buf * T::BUF_ELEMS;
#pragma unroll
        for (int p = 0; p < T::K_LOADS; ++p) {
            const int c = p * kThreads + tid;
            *(mfa_u32x4*)(s + T::k_off(c / T::KCH, c % T::KCH)) = kreg[p];
        }
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            mfa_u32x4 col;
#pragma unroll
            for (int m2 = 0; m2 < 4; ++m2)
                col[m2] = __builtin_amdgcn_perm(vreg[2 * m2 + 1][e >> 1], vreg[2 * m2][e >> 1], sel);
            *(mfa_u32x4*)(s + T::v_off(v_c * VW + e, v_a)) = col;
        }
    };

    const float sl2 = a.scale_log2_abs;
    int n_visit = 0, n_edge = 0;
    if (kt_lo < kt_hi) {
        load_tile(kt_lo);
        store_tile(0);
        __syncthreads();
    }

    for (int kt = kt_lo; kt < kt_hi; ++kt) {
        const int cur = (kt - kt_lo) & 1;
        const bool has_next = kt + 1 < kt_hi;
        if (has_next) load_tile(kt + 1);
        const uint16_t* s = smem + cur * T::BUF_ELEMS;

        // S^T = K Q^T for the NNB 32-key blocks of the tile (independent chains)
        mfa_f32x16 sacc[NNB];
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) sacc[nb] = mfa_f32x16{};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb) {
                const int krow = nb * 32 + key_perm(l32);
                const mfa_u32x4 kop = *(const mfa_u32x4*)(s + T::k_off(krow, 2 * kb + g32));
                sacc[nb] = mfa_mfma32<DT>(kop, qreg[kb], sacc[nb]);
            }
        }

        // signed raw scores (the sign of scale folded in), masked on edge tiles
        const bool edge = !mfa_tile_full(a.mask, kBM, BN, qt, kt);
        const int k0 = kt * BN;
        float tmax = -MFA_INF;
        if (edge) {
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + nb * 32 + 16 * (r >> 3) + 8 * g32 + (r & 7);
                    const float x = NEG ? -sacc[nb][r] : sacc[nb][r];
                    sacc[nb][r] = (key >= row_lo && key <= row_hi) ? x : -MFA_INF;
                    tmax = fmaxf(tmax, sacc[nb][r]);
                }
            }
        } else {
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (NEG) sacc[nb][r] = -sacc[nb][r];
                    tmax = fmaxf(tmax, sacc[nb][r]);
                }
            }
        }
        tmax = fmaxf(tmax, mfa_swap_halves(tmax));
        // raise the offset only when the row max outgrows it by more than kLazy
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

        mfa_u32x4 pop[NNB][2];
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const float x0 = sacc[nb][8 * hh + 2 * e2];
                    const float x1 = sacc[nb][8 * hh + 2 * e2 + 1];
                    float p0 = mfa_exp2(__builtin_fmaf(x0, sl2, -m_use));
                    float p1 = mfa_exp2(__builtin_fmaf(x1, sl2, -m_use));
                    if (edge) {
                        p0 = (x0 == -MFA_INF) ? 0.f : p0;
                        p1 = (x1 == -MFA_INF) ? 0.f : p1;
                    }
                    const uint32_t pk = mfa_pack2<DT>(p0, p1);
                    pop[nb][hh][e2] = pk;
                    // f16: sum the rounded weights with one dot2 (rounding 2^-12);
                    // bf16 rounds too coarsely (2^-9) for the LSE, so sum in fp32
                    if constexpr (DT == MFA_DT_F16)
                        l_run = mfa_sum2<DT>(pk, l_run);
                    else
                        l_run += p0 + p1;
                }
            }
        }

        // O^T += V^T P^T (the NDB accumulators are independent chains)
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                mfa_u32x4 vop[NDB];
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    vop[db] = *(const mfa_u32x4*)(s + T::v_off(db * 32 + l32, 4 * nb + 2 * hh + g32));
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] = mfa_mfma32<DT>(vop[db], pop[nb][hh], oacc[db]);
            }
        }

        if (has_next) store_tile(cur ^ 1);
        __syncthreads();
        if (TILELOG) {
            ++n_visit;
            n_edge += edge ? 1 : 0;
        }
    }

    // ---- epilogue: O = o / l, LSE = (m + log2 l) * ln 2 --------------------------
    const float l_tot = l_run + mfa_swap_halves(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qvalid) {
        uint16_t* op = a.o + (head_q + (size_t)qrow) * D + 4 * g32;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mfa_u32x2 w2;
                w2[0] = mfa_pack2<DT>(oacc[db][4 * j + 0] * inv, oacc[db][4 * j + 1] * inv);
                w2[1] = mfa_pack2<DT>(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
                *(mfa_u32x2*)(op + db * 32 + 8 * j) = w2;
            }
        }
        if (a.lse != nullptr && g32 == 0)
            a.lse[head_q + qrow] = l_tot > 0.f ? (m_run + mfa_log2(l_tot)) * MFA_LN2 : -MFA_INF;
    }
    if (TILELOG && tid == 0) {
        int32_t* t = a.tile_log + ((size_t)(b * a.Hq + h) * a.n_q_tiles + qt) * 4;
        t[0] = n_visit ? kt_lo : -1;
        t[1] = n_visit;
        t[2] = n_edge;
        t[3] = n_visit ? kt_lo + n_visit : -1;
    }
}

template <int D, int DT, int BN, bool TL>
void launch_sign(const FwdArgs& a, dim3 grid, dim3 block, hipStream_t stream, bool neg) {
    if (neg)
        hipLaunchKernelGGL((mfa_fwd_kernel<D, DT, BN, TL, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((mfa_fwd_kernel<D, DT, BN, TL, false>), grid, block, 0, stream, a);
}

template <int D, int DT, int BN>
int launch(const FwdArgs& a, hipStream_t stream, bool tilelog, bool neg, mfa_dispatch_info* info) {
    const dim3 grid((unsigned)a.n_q_tiles * (unsigned)a.HB);
    const dim3 block(kThreads);
    if (tilelog)
        launch_sign<D, DT, BN, true>(a, grid, block, stream, neg);
    else
        launch_sign<D, DT, BN, false>(a, grid, block, stream, neg);
    snprintf(info->kernel, sizeof(info->kernel), "mfa_fwd_kernel<D=%d,%s,BM=%d,BN=%d%s%s>", D,
             DT == MFA_DT_F16 ? "f16" : "bf16", kBM, BN, tilelog ? ",tilelog" : "",
             neg ? ",neg" : "");
    info->BM = kBM;
    info->BN = BN;
    info->waves = kThreads / 64;
    info->grid[0] = (int)grid.x;
    info->grid[1] = 1;
    info->grid[2] = 1;
    info->block = kThreads;
    return hipGetLastError() == hipSuccess ? MFA_OK : MFA_ERR_HIP;
}

}  // namespace

int mfa_fwd_bn(int) { return 64; }
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
    a.HB = pr.B * pr.Hq;
    a.xcd_group = ((pr.B * pr.Hkv) % 8 == 0) ? 1 : 0;
    // heavy/light pairing helps when every workgroup is resident at once (2 per CU)
    a.snake = (pr.causal && (long long)a.n_q_tiles * a.HB <= 2LL * mfa_num_cus()) ? 1 : 0;
    a.scale_log2_abs = fabsf(pr.scale) * 1.4426950408889634f;
    a.mask = mfa_make_mask(pr.Nq, pr.Nk, pr.causal, pr.left, pr.right);
    const bool tl = pr.tile_log != nullptr;
    const bool neg = pr.scale < 0.f;
    if (pr.D == 128) {
        return pr.dtype == MFA_F16 ? launch<128, MFA_DT_F16, 64>(a, stream, tl, neg, info)
                                   : launch<128, MFA_DT_BF16, 64>(a, stream, tl, neg, info);
    }
    return pr.dtype == MFA_F16 ? launch<64, MFA_DT_F16, 64>(a, stream, tl, neg, info)
                               : launch<64, MFA_DT_BF16, 64>(a, stream, tl, neg, info);
}
