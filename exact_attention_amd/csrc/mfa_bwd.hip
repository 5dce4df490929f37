// Backward pass of exact attention for gfx950: dQ, dK, dV from Q, K, V, the forward's
// output O, its row log-sum-exp and the upstream gradient dO, in the passes of the
// FlashAttention-2 backward of the mlx-bun flash-attention.ts page (its D-vector pass is
// folded into the dQ pass, which reads each query row once anyway):
//   dQ:    per query tile: D_i = sum_d dO_id O_id and the LSE in the log2 domain for its
//          rows (also written out), then over the key tiles: P = exp(scale S - LSE),
//          dP = dO V^T, dS = P (dP - D), dQ += scale dS K;
//   dK/dV: per key tile, over the query tiles (and the g query heads of a KV head), after
//          the dQ pass: the same P and dS, dV += P^T dO, dK += scale dS^T Q.
// The probabilities are recomputed from the saved LSE (no running maximum is needed: P <= 1),
// dQ is accumulated by its own pass rather than with atomics, so every result is
// deterministic, and every product runs on the 32x32x16 MFMA:
//   dK/dV pass, one wave = 32 keys (its K^T operand in registers, V in LDS):
//     S = Q K^T and dP = dO V^T with the query rows fed in key_perm order, so that each
//     lane owns one key column and runs of 8 consecutive query rows; the packed P and dS
//     are then directly the B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A
//     operands come from transposing LDS reads of the Q and dO tiles.
//   dQ pass, one wave = 32 query rows (its Q^T and dO^T operands in registers):
//     S^T = K Q^T and dP^T = V dO^T with the key rows in key_perm order, then
//     dQ^T += K^T dS^T with K^T from transposing reads of the K tile.
// Workgroups have 8 waves in two halves that split the steps (dK/dV: alternate query
// tiles; dQ: the two 32-key halves of each key tile) and add their partial sums through
// LDS at the end.  Tiles stream through LDS with direct global -> LDS loads, one step
// ahead; the workgroups of one (batch, head) run on one XCD and walk the shared tiles in
// the same order, so the copies hit L2.  A wave skips a 32 x 32 block holding no visible
// (query, key) pair, and masks only blocks that are not wholly visible.
#include "mfa_device.h"
#include "mfa_geometry.h"
#include "mfa_internal.h"
#include "mfa_tile.h"

namespace {

constexpr int kThreads8 = 512;  // 8 waves (dK/dV and dQ)

// The Q / dO (dK/dV pass) and K / V (dQ pass) tiles are read as row operands and
// transposed: they use the swz_both layout.
// Workgroups are handed to the 8 XCDs in turn (id % 8).  When the count divides evenly,
// renumber them so that XCD x runs the contiguous logical range [x n / 8, (x + 1) n / 8):
// the workgroups of one (batch, head) then share that XCD's L2, and each XCD still starts
// its range in order.
__device__ __forceinline__ int xcd_logical_id(int n) {
    const int id = (int)(blockIdx.x + gridDim.x * blockIdx.y);
    return (n & 7) ? id : (id & 7) * (n >> 3) + (id >> 3);
}

__device__ __forceinline__ void lds_write_f4(float* __restrict__ p, mfa_f32x4 v) {
    typedef __attribute__((address_space(3))) mfa_f32x4 lds_f32x4;
    *(lds_f32x4*)p = v;
}

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    float* lse2;    // [B, Hq, Nq]: LSE * log2(e), +inf for rows with no visible key
    float* dvec;    // [B, Hq, Nq]: D_i
    int B, Hq, Hkv, Nq, Nk, g;
    float scale;       // signed
    float scale_log2;  // scale * log2(e)
    MfaMask mask;
    int chain_q;       // 1: a dQ workgroup runs query tile qt, then nqt - 1 - qt
};

// Visibility of a 32 x 32 block (rows r0 .. r0 + 31 < Nq at least partly, keys
// c0 .. c0 + 31): any visible pair, and every pair visible.  The row bounds of the mask
// grow by at most one per row, so the first row's low end and the last row's high end
// decide whether any pair is visible.
__device__ __forceinline__ bool block_any(const MfaMask& m, int Nq, int r0, int c0) {
    if (r0 >= Nq || c0 >= m.Nk) return false;
    const int r1 = min(r0 + 31, Nq - 1);
    const int64_t c1 = c0 + 31 < m.Nk ? c0 + 31 : m.Nk - 1;
    return mfa_row_hi(m, r1) >= c0 && mfa_row_lo(m, r0) <= c1;
}
__device__ __forceinline__ bool block_all(const MfaMask& m, int Nq, int r0, int c0) {
    return r0 + 31 < Nq && mfa_tile_full(m, 32, 32, r0 / 32, c0 / 32);
}

// ---- dK, dV ------------------------------------------------------------------------
// Workgroup = 128 keys of one (batch, KV head), 8 waves: wave w owns the 32 keys
// 32 (w % 4) .. +31 and the steps of parity w / 4, so that the two 4-wave halves walk
// alternate steps side by side (the heaviest workgroup of a causal mask then takes half as
// long) and add their partial dK / dV through LDS at the end, in a fixed order.  Steps =
// (query head of the group, 32-row query tile) over the tiles that see any of the 128 keys.
template <int D, int DT>
__global__ __launch_bounds__(kThreads8, 1) void mfa_bwd_dkv_kernel(BwdArgs a) {
    constexpr int KCH = D / 8;            // 16-byte chunks per row
    constexpr int NKB = D / 16;           // k-steps over D
    constexpr int NDB = D / 32;           // 32-row blocks of dK^T / dV^T
    constexpr int TROWS = 32;             // query rows per step
    constexpr int TILE = TROWS * D;       // 16-bit elements of a Q or dO tile
    constexpr int RPB = 64 / KCH;         // rows per 1 KiB block
    constexpr int LOADS = TROWS / RPB / 4;   // direct loads per wave per tile (4 waves a step)
    // V in the register layout of the B operand of dP: 1 KiB block (32-key block, k-step)
    // holds lane (key l32, k-group g32)'s 16 bytes at 16 * lane
    __shared__ __attribute__((aligned(1024))) uint16_t sv[128 * D];
    // the two pipeline buffers are separate objects, picked by a compile-time index, so
    // that the compiler sees that a copy into one never touches reads from the other
    // (per buffer: parity 0 Q, dO, then parity 1 Q, dO; lse2 and dvec likewise)
    __shared__ __attribute__((aligned(1024))) uint16_t sq0[2 * 2 * TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sq1[2 * 2 * TILE];
    __shared__ __attribute__((aligned(16))) float sl0[2 * 2 * 64];
    __shared__ __attribute__((aligned(16))) float sl1[2 * 2 * 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kblk = wave & 3;            // key block of this wave
    const int par = wave >> 2;            // step parity of this wave
    const int pw = wave & 3;              // wave index within its half
    const int g32 = lane >> 5;
    const int l32 = lane & 31;
    const MfaMask& m = a.mask;
    const int nkt = (a.Nk + 127) >> 7;
    const int lid = xcd_logical_id(nkt * a.B * a.Hkv);
    const int bk = lid / nkt;             // b * Hkv + kvh
    // causal masks give the low key tiles the most query rows: they start first (a mask
    // bounded on the left only is the mirror image)
    const int kt = (m.left >= 0 && m.right_eff < 0) ? nkt - 1 - (lid - bk * nkt) : lid - bk * nkt;
    const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
    const int k0 = kt * 128;
    const int kw0 = k0 + kblk * 32;       // this wave's first key
    const size_t kv_base = (size_t)bk * a.Nk * D;

    // V of the workgroup's 128 keys -> LDS in operand layout (keys past Nk read as zero),
    // and this wave's K^T operand: lane (key l32, k-group g32) holds K[key][16 kb + 8 g32 .. +7]
    {
        // (k0 < Nk; a clamp from both sides would become a vector med3 and put the
        // resource in vector registers)
        const auto rv = mfa_rsrc(a.v + kv_base + (size_t)k0 * D, (uint32_t)min(a.Nk - k0, 128) * D * 2);
#pragma unroll
        for (int i = 0; i < 128 * KCH / kThreads8; ++i) {
            const int blk = i * 8 + wave;                     // 32-key block * NKB + k-step
            const int row = (blk / NKB) * 32 + l32, col = (blk % NKB) * 16 + g32 * 8;
            mfa_load16_lds(rv, sv + blk * 512, (uint32_t)(row * D + col) * 2);
        }
    }
    mfa_u32x4 kb_op[NKB];
    {
        const auto rk = mfa_rsrc(a.k + kv_base, (uint32_t)a.Nk * D * 2);
        const uint32_t off = ((uint32_t)(kw0 + l32) * D + g32 * 8) * 2;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) kb_op[kb] = mfa_load16(rk, off + kb * 32);
    }

    // query rows that see any of the 128 keys: [q_lo, q_hi]
    const int off32 = (int)m.off;
    const int d_lo = m.left < 0 ? INT_MIN : -m.left;
    const int d_hi = m.right_eff < 0 ? INT_MAX : m.right_eff;
    const int k1 = min(k0 + 127, a.Nk - 1);
    int64_t q_lo = 0, q_hi = a.Nq - 1;
    if (m.right_eff >= 0) q_lo = max((int64_t)0, (int64_t)k0 - m.off - m.right_eff);
    if (m.left >= 0) q_hi = min((int64_t)a.Nq - 1, (int64_t)k1 - m.off + m.left);
    const int t_lo = (int)(q_lo / TROWS);
    const int n_t = q_hi >= q_lo ? (int)(q_hi / TROWS) - t_lo + 1 : 0;
    const int n_steps = n_t * a.g;
    const int n_iter = (n_steps + 1) >> 1;   // iteration i: steps 2 i and 2 i + 1
    // step j = hh n_t + r: query head hh of the group, tile t_lo + n_t - 1 - r.  The tiles
    // of a head are walked from the last down, so that under a causal mask every key tile
    // of the head reads the same query tiles at about the same time (shared through L2).
    // (hh, r) of this half's current step is carried from step to step (j grows by 2)
    // instead of dividing.
    int hh_c = 0, r_c = par;
    while (r_c >= n_t && n_t > 0) {
        r_c -= n_t;
        ++hh_c;
    }

    mfa_f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
        dkt[i] = mfa_f32x16{};
        dvt[i] = mfa_f32x16{};
    }

    const int pofs = par * 2 * TILE;      // this half's tiles within a buffer
    // direct loads of step (hh, r) (it exists): Q and dO rows of its tile (32 rows), lse2
    // and dvec
    auto issue = [&](int hh, int r, auto bufc) {
        uint16_t* dst = (decltype(bufc)::value == 0 ? sq0 : sq1) + pofs;
        float* dl = (decltype(bufc)::value == 0 ? sl0 : sl1) + par * 128;
        const int t = t_lo + n_t - 1 - r;
        const int h = kvh * a.g + hh;
        const int q0 = t * TROWS;
        const size_t row0 = ((size_t)(b * a.Hq + h) * a.Nq + q0);
        const uint32_t bytes = (uint32_t)min(a.Nq - q0, TROWS) * D * 2;   // q0 < Nq
        const auto rq = mfa_rsrc(a.q + row0 * D, bytes);
        const auto rd = mfa_rsrc(a.dout + row0 * D, bytes);
#pragma unroll
        for (int l = 0; l < LOADS; ++l) {
            const int blk = l * 4 + pw;
            const int row = blk * RPB + lane / KCH, phys = lane % KCH;
            const uint32_t off = (uint32_t)(row * D + swz_both<KCH>(row, phys) * 8) * 2;
            mfa_load16_lds(rq, dst + blk * 512, off);
            mfa_load16_lds(rd, dst + TILE + blk * 512, off);
        }
        if (pw == 0) {
            const uint32_t nb = (uint32_t)min(a.Nq - q0, 64) * 4;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(mfa_rsrc(a.lse2 + row0, nb),
                (__attribute__((address_space(3))) void*)dl, 4, (uint32_t)lane * 4, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(mfa_rsrc(a.dvec + row0, nb),
                (__attribute__((address_space(3))) void*)(dl + 64), 4, (uint32_t)lane * 4, 0, 0, 0);
        }
    };

    // per-lane LDS addresses (offsets within a buffer, this half's tiles included):
    // A-operand rows of S = Q K^T / dP = dO V^T (query row key_perm(l32), chunk 2 kb + g32);
    // transposing reads of Q^T / dO^T (lane group qg: columns 16 (qg % 2) .. +15 of a
    // 32-column block, query rows 8 (qg / 2) .. +3, and 4 rows further at t_rd + t4, where
    // the layout flips chunk bit 0: t4 = 4 D -+ 8 by this lane's chunk parity);
    // B operand of dP: this lane's 16 bytes of block (kblk, kb) of the V operand layout.
    // The A-operand offset of k-step kb is a_b + ((2 kb) ^ a_x) * 8: the layout splits into
    // a lane term (in a_b) and one that XORs the k-step's chunk pair; it is formed at each
    // read (two VALU) rather than held in NKB registers.
    int a_b, a_x, t_rd[NDB], t4;
    {
        const int row = key_perm(l32);
        const int x = swz_x<KCH>(row);
        a_x = x & (KCH - 2);
        a_b = pofs + row * D + (g32 ^ (x & 1)) * 8;
        const int qg = lane >> 4, i = lane & 15;
        const int trow = 8 * (qg >> 1) + (i >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = db * 32 + 16 * (qg & 1) + 4 * (i & 3);
            t_rd[db] = pofs + trow * D + swz_both<KCH>(trow, col >> 3) * 8 + (col & 7);
        }
        t4 = tr4_delta<D>(lane);
    }
    const int v_rd = kblk * NKB * 512 + lane * 8;

    if (par < n_steps) issue(hh_c, r_c, MfaInt<0>{});
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): V rows, K operand, first tiles
    __syncthreads();

    const int key = kw0 + l32;
    const bool key_ok = key < a.Nk;
    // P and dS of the 32 x 32 block, packed as B operands (register r of this lane: query
    // row q0 + 16 (r / 8) + 8 g32 + r % 8, key kw0 + l32); MASKED = 0 for a block whose
    // pairs are all visible
    auto probs = [&](auto maskc, const mfa_f32x16& s, const mfa_f32x16& dp, const float* tl,
                     int q0, mfa_u32x4 (&pp)[2], mfa_u32x4 (&dsp)[2]) {
#pragma unroll
        for (int hk = 0; hk < 2; ++hk) {
            const int rr = 16 * hk + 8 * g32;   // first of this run's 8 query rows
            const mfa_f32x4 l0 = lds_read_f4(tl + rr), l1 = lds_read_f4(tl + rr + 4);
            const mfa_f32x4 d0 = lds_read_f4(tl + 64 + rr), d1 = lds_read_f4(tl + 64 + rr + 4);
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float pv[2], dv2[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int e = 2 * e2 + u;         // 0..7 within the run
                    const int r = 8 * hk + e;
                    const float lse2 = e < 4 ? l0[e] : l1[e - 4];
                    const float dvv = e < 4 ? d0[e] : d1[e - 4];
                    float x = __builtin_fmaf(s[r], a.scale_log2, -lse2);
                    if constexpr (decltype(maskc)::value) {
                        // visible iff 0 <= key < Nk, qi < Nq and d_lo <= key - qi - off <=
                        // d_hi (bitwise, not short-circuit, so that no branch is made); a
                        // masked pair's exponent is -inf and the exp itself gives 0
                        const int qi = q0 + rr + e;
                        const int dd = key - qi - off32;
                        const bool vis = key_ok & (qi < a.Nq) & (dd >= d_lo) & (dd <= d_hi);
                        x = vis ? x : -MFA_INF;
                    }
                    const float p = mfa_exp2(x);
                    pv[u] = p;
                    dv2[u] = p * (dp[r] - dvv);
                }
                pp[hk][e2] = mfa_pack2<DT>(pv[0], pv[1]);
                dsp[hk][e2] = mfa_pack2<DT>(dv2[0], dv2[1]);
            }
        }
    };
    auto iter = [&](int i, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        // this half's next step (hh_n, r_n): j + 2
        int hh_n = hh_c, r_n = r_c + 2;
        while (r_n >= n_t) {
            r_n -= n_t;
            ++hh_n;
        }
        if (2 * i + 2 + par < n_steps) issue(hh_n, r_n, MfaInt<buf ^ 1>{});
        const int j = 2 * i + par;
        const int q0 = (t_lo + n_t - 1 - r_c) * TROWS;
        if (j < n_steps && block_any(m, a.Nq, q0, kw0)) {   // uniform per wave
            const uint16_t* tq = buf == 0 ? sq0 : sq1;   // + pofs, folded into the offsets
            const uint16_t* td = tq + TILE;
            const float* tl = (buf == 0 ? sl0 : sl1) + par * 128;
            int ax = a_x;
            asm volatile("" : "+v"(ax));   // keep the per-step offsets from being hoisted
            mfa_f32x16 s = mfa_f32x16{}, dp = mfa_f32x16{};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int ao = a_b + (((2 * kb) ^ ax) << 3);
                s = mfa_mfma32<DT>(lds_read16(tq + ao), kb_op[kb], s);
                dp = mfa_mfma32<DT>(lds_read16(td + ao), lds_read16(sv + v_rd + kb * 512), dp);
            }
            mfa_u32x4 pp[2], dsp[2];
            if (block_all(m, a.Nq, q0, kw0))
                probs(MfaInt<0>{}, s, dp, tl, q0, pp, dsp);
            else
                probs(MfaInt<1>{}, s, dp, tl, q0, pp, dsp);
            // dV^T += dO^T P, dK^T += Q^T dS (k-steps over the two runs of 16 query rows)
#pragma unroll
            for (int hk = 0; hk < 2; ++hk) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int ofs = hk * 16 * D;
                    const int t2 = t_rd[db] + t4;
                    const mfa_u32x2 a0 = lds_read_tr(td + t_rd[db] + ofs), a1 = lds_read_tr(td + t2 + ofs);
                    dvt[db] = mfa_mfma32<DT>(mfa_u32x4{a0[0], a0[1], a1[0], a1[1]}, pp[hk], dvt[db]);
                    const mfa_u32x2 b0 = lds_read_tr(tq + t_rd[db] + ofs), b1 = lds_read_tr(tq + t2 + ofs);
                    dkt[db] = mfa_mfma32<DT>(mfa_u32x4{b0[0], b0[1], b1[0], b1[1]}, dsp[hk], dkt[db]);
                }
            }
        }
        hh_c = hh_n;
        r_c = r_n;
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): the next iteration's tiles landed
        block_barrier();
    };
    for (int i = 0; i < n_iter; i += 2) {
        iter(i, MfaInt<0>{});
        if (i + 1 < n_iter) iter(i + 1, MfaInt<1>{});
    }

    // the odd-step half hands its partial sums to the even-step half through LDS (the
    // tile buffers, free now: no copy is in flight), dK^T first, then dV^T; the first
    // half of the 32-column blocks goes through one buffer, the second through the other
    static_assert(sizeof(sq0) >= 4 * (NDB / 2) * 16 * 64 * sizeof(float), "exchange buffer");
    auto exchange = [&](mfa_f32x16 (&acc)[NDB]) {
        if (par == 1) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    float* red = (float*)(db < NDB / 2 ? sq0 : sq1);
                    const int idx = ((kblk * (NDB / 2) + db % (NDB / 2)) * 4 + r4) * 64 + lane;
                    lds_write_f4(red + idx * 4, mfa_f32x4{acc[db][4 * r4], acc[db][4 * r4 + 1],
                                                          acc[db][4 * r4 + 2], acc[db][4 * r4 + 3]});
                }
        }
        block_barrier();
        if (par == 0) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const float* red = (const float*)(db < NDB / 2 ? sq0 : sq1);
                    const int idx = ((kblk * (NDB / 2) + db % (NDB / 2)) * 4 + r4) * 64 + lane;
                    const mfa_f32x4 o = lds_read_f4(red + idx * 4);
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[db][4 * r4 + c] += o[c];
                }
        }
        block_barrier();
    };
    exchange(dkt);
    exchange(dvt);
    if (par == 1) return;

    // write dK = scale (dK^T)^T and dV: register r of block db holds d = 32 db + 8 (r / 4)
    // + 4 g32 + r % 4 of key kw0 + l32; runs of 4 consecutive d are one 8-byte store
    if (key_ok) {
        uint16_t* dkp = a.dk + kv_base + (size_t)key * D;
        uint16_t* dvp = a.dv + kv_base + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * db + 8 * r4 + 4 * g32;
                mfa_u32x2 wk, wv;
                wk[0] = mfa_pack2<DT>(dkt[db][4 * r4] * a.scale, dkt[db][4 * r4 + 1] * a.scale);
                wk[1] = mfa_pack2<DT>(dkt[db][4 * r4 + 2] * a.scale, dkt[db][4 * r4 + 3] * a.scale);
                wv[0] = mfa_pack2<DT>(dvt[db][4 * r4], dvt[db][4 * r4 + 1]);
                wv[1] = mfa_pack2<DT>(dvt[db][4 * r4 + 2], dvt[db][4 * r4 + 3]);
                *(mfa_u32x2*)(dkp + d) = wk;
                *(mfa_u32x2*)(dvp + d) = wv;
            }
    }
}

// ---- dQ ----------------------------------------------------------------------------
// Workgroup = 128 query rows of one (batch, head), 8 waves: wave w owns the 32 rows
// 32 (w % 4) .. +31 and the 32-key half w / 4 of every 64-key K / V tile, over the key
// tiles the query tile sees (the forward's tile range); the two halves add their partial
// dQ through LDS at the end, in a fixed order.
template <int D, int DT>
__global__ __launch_bounds__(kThreads8, 1) void mfa_bwd_dq_kernel(BwdArgs a) {
    constexpr int KCH = D / 8;
    constexpr int NKB = D / 16;
    constexpr int NDB = D / 32;
    constexpr int BN = 64;
    constexpr int TILE = BN * D;
    constexpr int RPB = 64 / KCH;
    constexpr int LOADS = BN / RPB / 8;
    // the two pipeline buffers are separate objects (see the dK/dV kernel)
    __shared__ __attribute__((aligned(1024))) uint16_t st0[2 * TILE];   // K, V tiles
    __shared__ __attribute__((aligned(1024))) uint16_t st1[2 * TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rblk = wave & 3;            // row block of this wave
    const int kh = wave >> 2;             // key half of every tile
    const int g32 = lane >> 5;
    const int l32 = lane & 31;
    const MfaMask& m = a.mask;
    const int nqt = (a.Nq + 127) >> 7;
    // Chained tiles: a workgroup runs a query tile and then its mirror image
    // nqt - 1 - qt, so that under a causal mask every workgroup has the same work and the
    // second tile starts without a new workgroup launch.
    const int n_rep = a.chain_q ? 2 : 1;
    const int n_units = nqt / n_rep;
    const int lid = xcd_logical_id(n_units * a.B * a.Hq);
    const int bh = lid / n_units;
    for (int rep = 0; rep < n_rep; ++rep) {
    // causal masks give the last query tiles the most keys: they start first
    const int qt_first = (m.right_eff >= 0 && m.left < 0) ? nqt - 1 - (lid - bh * n_units) : lid - bh * n_units;
    const int qt = rep == 0 ? qt_first : nqt - 1 - qt_first;
    const int b = bh / a.Hq, h = bh - b * a.Hq;
    const int kvh = h / a.g;
    const int qw0 = qt * 128 + rblk * 32;   // this wave's first query row
    const int qrow = qw0 + l32;
    const size_t q_base = (size_t)bh * a.Nq * D;
    const size_t kv_base = (size_t)(b * a.Hkv + kvh) * a.Nk * D;

    // Q^T and dO^T operands: lane (query l32, k-group g32) holds row[16 kb + 8 g32 .. +7]
    // and this row's D_i = sum_d dO_id O_id from the same chunks of O (the other half of
    // the row is in lane ^ 32); D_i and the LSE in the log2 domain are also written out for
    // the dK/dV pass, which runs after this one
    mfa_u32x4 qb[NKB], db_op[NKB];
    float dpart = 0.f;
    {
        const auto rq = mfa_rsrc(a.q + q_base, (uint32_t)a.Nq * D * 2);
        const auto rd = mfa_rsrc(a.dout + q_base, (uint32_t)a.Nq * D * 2);
        const auto ro = mfa_rsrc(a.o + q_base, (uint32_t)a.Nq * D * 2);
        const uint32_t off = ((uint32_t)qrow * D + g32 * 8) * 2;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            qb[kb] = mfa_load16(rq, off + kb * 32);
            db_op[kb] = mfa_load16(rd, off + kb * 32);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const mfa_u32x4 o4 = mfa_load16(ro, off + kb * 32);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dpart += mfa_lo<DT>(o4[e]) * mfa_lo<DT>(db_op[kb][e]) + mfa_hi<DT>(o4[e]) * mfa_hi<DT>(db_op[kb][e]);
        }
    }
    const bool qvalid = qrow < a.Nq;
    const float lraw = qvalid ? a.lse[(size_t)bh * a.Nq + qrow] : -MFA_INF;
    __builtin_amdgcn_s_waitcnt(0x0f70);
    const float dvv = mfa_pair_sum(dpart);
    const float lse2 = lraw == -MFA_INF ? MFA_INF : lraw * 1.4426950408889634f;
    if (qvalid && kh == 0 && g32 == 0) {
        a.dvec[(size_t)bh * a.Nq + qrow] = dvv;
        a.lse2[(size_t)bh * a.Nq + qrow] = lse2;
    }
    const int64_t rlo64 = mfa_row_lo(m, qrow), rhi64 = mfa_row_hi(m, qrow);
    const int row_lo = rlo64 > a.Nk ? a.Nk : (int)rlo64;
    const int row_hi = rhi64 < -1 ? -1 : (int)rhi64;

    int t_lo, t_hi;
    mfa_tile_range(m, a.Nq, 128, BN, qt, &t_lo, &t_hi);
    const int n = t_hi - t_lo;

    mfa_f32x16 dqt[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dqt[i] = mfa_f32x16{};

    auto issue = [&](int kt, auto bufc) {
        uint16_t* dst = decltype(bufc)::value == 0 ? st0 : st1;
        const int kk0 = kt * BN;
        const uint32_t bytes = (uint32_t)max(a.Nk - kk0, 0) * D * 2;
        const auto rk = mfa_rsrc(a.k + kv_base + (size_t)kk0 * D, bytes);
        const auto rv = mfa_rsrc(a.v + kv_base + (size_t)kk0 * D, bytes);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int blk = i * 8 + wave;
            const int row = blk * RPB + lane / KCH, phys = lane % KCH;
            const uint32_t off = (uint32_t)(row * D + swz_both<KCH>(row, phys) * 8) * 2;
            mfa_load16_lds(rk, dst + blk * 512, off);
            mfa_load16_lds(rv, dst + TILE + blk * 512, off);
        }
    };

    // A-operand rows of S^T = K Q^T and dP^T = V dO^T (key row key_perm(l32) of this
    // wave's 32-key half, chunk 2 kb + g32); transposing reads of K^T (lane group qg:
    // columns 16 (qg % 2) .. +15 of a 32-column block, keys 8 (qg / 2) .. +3 (+4))
    // (the second transposing read of a k-group is 4 rows further, at t_rd + t4)
    int a_rd[NKB], t_rd[NDB], t4;
    {
        const int row = kh * 32 + key_perm(l32);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) a_rd[kb] = row * D + swz_both<KCH>(row, 2 * kb + g32) * 8;
        const int qg = lane >> 4, i = lane & 15;
        const int trow = kh * 32 + 8 * (qg >> 1) + (i >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = db * 32 + 16 * (qg & 1) + 4 * (i & 3);
            t_rd[db] = trow * D + swz_both<KCH>(trow, col >> 3) * 8 + (col & 7);
        }
        t4 = tr4_delta<D>(lane);
    }

    if (n > 0) issue(t_lo, MfaInt<0>{});
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    // dS^T of the 32 x 32 block packed as the B operand (register r: key c0 + 16 (r / 8) +
    // 8 g32 + r % 8, query row qrow); MASKED = 0 for a block whose pairs are all visible
    auto dscores = [&](auto maskc, const mfa_f32x16& s, const mfa_f32x16& dp, int c0,
                       mfa_u32x4 (&dsp)[2]) {
#pragma unroll
        for (int hk = 0; hk < 2; ++hk)
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float w[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int r = 8 * hk + 2 * e2 + u;
                    float x = __builtin_fmaf(s[r], a.scale_log2, -lse2);
                    if constexpr (decltype(maskc)::value) {
                        const int key = c0 + 16 * hk + 8 * g32 + 2 * e2 + u;
                        const bool vis = qvalid & (key >= row_lo) & (key <= row_hi);
                        x = vis ? x : -MFA_INF;
                    }
                    const float p = mfa_exp2(x);
                    w[u] = p * (dp[r] - dvv);
                }
                dsp[hk][e2] = mfa_pack2<DT>(w[0], w[1]);
            }
    };
    auto iter = [&](int j, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const int kt = t_lo + j;
        if (j + 1 < n) issue(kt + 1, MfaInt<buf ^ 1>{});
        const uint16_t* tk = buf == 0 ? st0 : st1;
        const uint16_t* tv = tk + TILE;
        const int c0 = kt * BN + kh * 32;
        if (block_any(m, a.Nq, qw0, c0)) {   // uniform per wave
            mfa_f32x16 s = mfa_f32x16{}, dp = mfa_f32x16{};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                s = mfa_mfma32<DT>(lds_read16(tk + a_rd[kb]), qb[kb], s);
                dp = mfa_mfma32<DT>(lds_read16(tv + a_rd[kb]), db_op[kb], dp);
            }
            mfa_u32x4 dsp[2];
            if (block_all(m, a.Nq, qw0, c0))
                dscores(MfaInt<0>{}, s, dp, c0, dsp);
            else
                dscores(MfaInt<1>{}, s, dp, c0, dsp);
            // dQ^T += K^T dS^T
#pragma unroll
            for (int hk = 0; hk < 2; ++hk)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int ofs = hk * 16 * D;
                    const mfa_u32x2 a0 = lds_read_tr(tk + t_rd[db] + ofs),
                                    a1 = lds_read_tr(tk + t_rd[db] + t4 + ofs);
                    dqt[db] = mfa_mfma32<DT>(mfa_u32x4{a0[0], a0[1], a1[0], a1[1]}, dsp[hk], dqt[db]);
                }
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);
        block_barrier();
    };
    for (int j = 0; j < n; j += 2) {
        iter(j, MfaInt<0>{});
        if (j + 1 < n) iter(j + 1, MfaInt<1>{});
    }

    // the second key half hands its partial dQ^T to the first through LDS (the tile
    // buffers, free now; the first half of the 32-column blocks through one, the second
    // through the other)
    static_assert(sizeof(st0) >= 4 * (NDB / 2) * 16 * 64 * sizeof(float), "exchange buffer");
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float* red = (float*)(db < NDB / 2 ? st0 : st1);
                const int idx = ((rblk * (NDB / 2) + db % (NDB / 2)) * 4 + r4) * 64 + lane;
                lds_write_f4(red + idx * 4, mfa_f32x4{dqt[db][4 * r4], dqt[db][4 * r4 + 1],
                                                      dqt[db][4 * r4 + 2], dqt[db][4 * r4 + 3]});
            }
    }
    block_barrier();
    if (kh == 1) {
        if (n_rep == 1) return;
        block_barrier();   // the other half has read the exchange (next tile's copies)
        continue;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const float* red = (const float*)(db < NDB / 2 ? st0 : st1);
            const int idx = ((rblk * (NDB / 2) + db % (NDB / 2)) * 4 + r4) * 64 + lane;
            const mfa_f32x4 o = lds_read_f4(red + idx * 4);
#pragma unroll
            for (int c = 0; c < 4; ++c) dqt[db][4 * r4 + c] += o[c];
        }

    if (qvalid) {
        uint16_t* dqp = a.dq + q_base + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * db + 8 * r4 + 4 * g32;
                mfa_u32x2 w;
                w[0] = mfa_pack2<DT>(dqt[db][4 * r4] * a.scale, dqt[db][4 * r4 + 1] * a.scale);
                w[1] = mfa_pack2<DT>(dqt[db][4 * r4 + 2] * a.scale, dqt[db][4 * r4 + 3] * a.scale);
                *(mfa_u32x2*)(dqp + d) = w;
            }
    }
    if (n_rep > 1) block_barrier();
    }   // rep
}

template <int D, int DT>
int launch(const BwdArgs& a, hipStream_t stream, mfa_dispatch_info* info) {
    // dQ first: it also writes D_i and the log2-domain LSE that the dK/dV pass reads
    const dim3 g2((unsigned)((a.Nq + 127) / 128 / (a.chain_q ? 2 : 1)), (unsigned)(a.B * a.Hq));
    hipLaunchKernelGGL((mfa_bwd_dq_kernel<D, DT>), g2, dim3(kThreads8), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MFA_ERR_HIP;
    const dim3 g1((unsigned)((a.Nk + 127) / 128), (unsigned)(a.B * a.Hkv));
    hipLaunchKernelGGL((mfa_bwd_dkv_kernel<D, DT>), g1, dim3(kThreads8), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MFA_ERR_HIP;
    snprintf(info->kernel, sizeof(info->kernel), "mfa_bwd_dkv_kernel+mfa_bwd_dq_kernel<D=%d,%s%s>", D,
             DT == MFA_DT_F16 ? "f16" : "bf16", a.chain_q ? ",dq chained" : "");
    info->grid[0] = (int)g1.x;
    info->grid[1] = (int)g1.y;
    info->grid[2] = 1;
    info->block = kThreads8;
    info->waves = 8;
    info->BM = 32;
    info->BN = 128;
    info->n_launches = 2;
    return MFA_OK;
}

}  // namespace

int mfa_bwd_launch(const MfaBwdProblem& p, hipStream_t stream, mfa_dispatch_info* info) {
    BwdArgs a;
    a.q = (const uint16_t*)p.q;
    a.k = (const uint16_t*)p.k;
    a.v = (const uint16_t*)p.v;
    a.o = (const uint16_t*)p.out;
    a.dout = (const uint16_t*)p.dout;
    a.lse = p.lse;
    a.dq = (uint16_t*)p.dq;
    a.dk = (uint16_t*)p.dk;
    a.dv = (uint16_t*)p.dv;
    a.lse2 = (float*)p.workspace;
    a.dvec = a.lse2 + (size_t)p.B * p.Hq * p.Nq;
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.Nq = p.Nq;
    a.Nk = p.Nk;
    a.g = p.Hq / p.Hkv;
    a.scale = p.scale;
    a.scale_log2 = p.scale * 1.4426950408889634f;
    a.mask = mfa_make_mask(p.Nq, p.Nk, p.causal, p.left, p.right);
    a.chain_q = ((p.Nq + 127) / 128) % 2 == 0 ? 1 : 0;
    if (p.D == 128)
        return p.dtype == MFA_F16 ? launch<128, MFA_DT_F16>(a, stream, info) : launch<128, MFA_DT_BF16>(a, stream, info);
    return p.dtype == MFA_F16 ? launch<64, MFA_DT_F16>(a, stream, info) : launch<64, MFA_DT_BF16>(a, stream, info);
}
