// Key-tile geometry of the forward pass, shared by the host planner and the kernel so
// that the tiles the kernel visits are, by construction, the tiles the plan reports.
//
// Visibility follows the causal mask of the mlx-bun forward shader and the
// window_size=(left, right) convention of the mlx-mfa 2.5.2 "Sliding window" feature
// (-1 = unbounded), with both window ends inclusive and bottom-right alignment
// off = Nk - Nq.  A key tile is visited iff it holds at least one visible pair
// (the "Causal tile-skip" feature: key tiles wholly above the diagonal are never
// visited).  The skip decision is
// uniform over the workgroup (a per-lane skip around a barrier is undefined).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define MFA_HD __host__ __device__ inline
#else
#define MFA_HD inline
#endif

struct MfaMask {
    int64_t off;       // Nk - Nq
    int64_t Nk;
    int left;          // -1 = unbounded
    int right_eff;     // -1 = unbounded; 0 under the causal mask (min with 0)
};

MFA_HD MfaMask mfa_make_mask(int Nq, int Nk, int causal, int left, int right) {
    MfaMask m;
    m.off = (int64_t)Nk - (int64_t)Nq;
    m.Nk = Nk;
    m.left = left;
    // the causal mask caps the right end of the window at the query's own position
    m.right_eff = causal ? 0 : right;
    return m;
}

// Inclusive visible key range of query row i (empty when lo > hi).
MFA_HD int64_t mfa_row_lo(const MfaMask& m, int64_t i) {
    if (m.left < 0) return 0;
    int64_t lo = i + m.off - m.left;
    return lo < 0 ? 0 : lo;
}
MFA_HD int64_t mfa_row_hi(const MfaMask& m, int64_t i) {
    if (m.right_eff < 0) return m.Nk - 1;
    int64_t hi = i + m.off + m.right_eff;
    return hi > m.Nk - 1 ? m.Nk - 1 : hi;
}

// Half-open key-tile range [kt_lo, kt_hi) of query tile qt (rows q0 .. q1 < Nq).
MFA_HD void mfa_tile_range(const MfaMask& m, int Nq, int BM, int BN, int qt, int* kt_lo, int* kt_hi) {
    int64_t q0 = (int64_t)qt * BM;
    int64_t q1 = q0 + BM - 1;
    if (q1 > Nq - 1) q1 = Nq - 1;
    int64_t lo = mfa_row_lo(m, q0);
    int64_t hi = mfa_row_hi(m, q1);
    if (lo > hi || q0 > q1) { *kt_lo = 0; *kt_hi = 0; return; }
    *kt_lo = (int)(lo / BN);
    *kt_hi = (int)(hi / BN) + 1;
}

// True if key tile kt needs no element mask for any row of query tile qt: every key of
// the tile exists and is visible to every row q0 .. q0 + BM - 1 (rows past Nq included,
// which only makes the test stricter).
MFA_HD bool mfa_tile_full(const MfaMask& m, int BM, int BN, int qt, int kt) {
    int64_t q0 = (int64_t)qt * BM;
    int64_t qlast = q0 + BM - 1;
    int64_t k0 = (int64_t)kt * BN;
    int64_t k1 = k0 + BN - 1;
    if (k1 > m.Nk - 1) return false;
    if (m.right_eff >= 0 && k1 > q0 + m.off + m.right_eff) return false;
    if (m.left >= 0 && k0 < qlast + m.off - m.left) return false;
    return true;
}
