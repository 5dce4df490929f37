// Tile-level building blocks shared by the forward and backward kernels: the row order
// fed to a 32x32x16 MFMA A operand, the XOR swizzles of LDS tiles, LDS operand reads with
// their own alias scope, and the bare workgroup barrier of the tile pipelines.
#pragma once
#include "mfa_device.h"

namespace {

template <int N>
struct MfaInt {
    static constexpr int value = N;
};

// Row of a 32-row block fed to A-operand row i.  With this order, accumulator register r
// of lane half g (lane / 32) holds row 16 * (r / 8) + 8 * g + r % 8: every lane then owns
// runs of 8 consecutive rows, which is the k-group layout of an operand of the next
// product (two k-steps of 16).
__device__ __forceinline__ int key_perm(int i) {
    return 16 * (i >> 4) + 8 * ((i >> 2) & 1) + 4 * ((i >> 3) & 1) + (i & 3);
}

// XOR swizzles on the 16-byte chunks of an LDS tile with KCH chunks per row (rows are not
// padded, so that a wave's direct load fills 1 KiB of consecutive LDS).  Row reads: the
// 16 rows one MFMA operand read touches at a logical chunk land in 16 distinct bank
// groups.
template <int KCH>
__device__ __forceinline__ int swz_rows(int row, int ch) {
    return (KCH == 16) ? (ch ^ (row & 15)) : (ch ^ ((row >> 1) & 7));
}

// A layout for tiles read both ways, and for transposing reads by 32 lanes at once:
// chunk ch of row r sits at ch ^ x(r).  Row reads need x to be a bijection on each block
// of 16 rows; a transposing read covers 4 consecutive rows with two adjacent chunks per
// 16 lanes, the 16 lanes beside them two chunks further, so the 4 rows must differ in the
// chunk bits above bit 1.  With 16 chunks a row (a row spans the 64 banks)
// x(r) = ((r & 3) << 2) | ((r >> 2) & 3) meets both; with 8 chunks (two rows per 64 banks)
// x = h((r >> 1) & 7), h(s) = ((s & 1) << 2) | (s >> 1).  (swz_rows puts rows 4k and
// 4k + 1 of a transposing read on the same banks; XOR-ing the chunk with (r & 3) << 1
// separates them within 16 lanes but not across 32.)  x depends on row % 16 only.  Between a transposing read and the
// one 4 rows below it the layout flips chunk bit 0, so the second read is
// tr4_delta elements further, by the lane's chunk parity.
template <int KCH>
__device__ __forceinline__ int swz_x(int row) {
    if constexpr (KCH == 16) {
        return ((row & 3) << 2) | ((row >> 2) & 3);
    } else {
        const int s = (row >> 1) & 7;
        return ((s & 1) << 2) | (s >> 1);
    }
}
template <int KCH>
__device__ __forceinline__ int swz_both(int row, int ch) { return ch ^ swz_x<KCH>(row); }
// (lane i of a 16-lane group of the transposing read pattern: rows 8 (group / 2) + i / 4,
// columns 32 db + 16 (group % 2) + 4 (i % 4))
template <int D>
__device__ __forceinline__ int tr4_delta(int lane) {
    return 4 * D + ((((lane & 15) >> 1) & 1) ? -8 : 8);
}

// Workgroup barrier of the tile pipelines.  __syncthreads() also fences memory, which
// waits for every outstanding load, including direct-to-LDS copies meant to stay in
// flight; here each wave has already waited for the copies the next stage reads
// (vmcnt), waits for its own LDS reads to return (lgkmcnt(0): no buffer is refilled
// while a read of it is pending) and then meets the others.  The empty asm statements
// keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS operand reads.  The restrict-qualified parameter gives each read an alias scope of
// its own; without one the compiler orders every LDS read after all direct-to-LDS copies
// still in flight (a vmcnt(0) before the read), which the tile pipelines already order
// themselves with vmcnt waits and barriers.
__device__ __forceinline__ mfa_u32x4 lds_read16(const uint16_t* __restrict__ p) {
    typedef __attribute__((address_space(3))) const mfa_u32x4 lds_u32x4;
    return *(lds_u32x4*)p;
}
__device__ __forceinline__ mfa_u32x2 lds_read_tr(const uint16_t* __restrict__ p) {
    return mfa_lds_read_tr16(p);
}
__device__ __forceinline__ int lds_read_i32(const int* __restrict__ p) {
    typedef __attribute__((address_space(3))) const int lds_i32;
    return *(lds_i32*)p;
}
__device__ __forceinline__ mfa_f32x4 lds_read_f4(const float* __restrict__ p) {
    typedef __attribute__((address_space(3))) const mfa_f32x4 lds_f32x4;
    return *(lds_f32x4*)p;
}

}  // namespace
