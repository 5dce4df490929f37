// Device helpers for gfx950 (CDNA4): MFMA wrappers, 16-bit conversions, lane exchange.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 mfa_f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 mfa_bf16x8 __attribute__((ext_vector_type(8)));
typedef float mfa_f32x16 __attribute__((ext_vector_type(16)));
typedef float mfa_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mfa_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mfa_u32x2 __attribute__((ext_vector_type(2)));
typedef float mfa_f32x2 __attribute__((ext_vector_type(2)));

#define MFA_DT_F16 0
#define MFA_DT_BF16 1

#define MFA_INF __builtin_inff()
#define MFA_LN2 0.69314718055994530942f

// D(32x32, fp32) += A(32x16) * B(16x32).  Operands: 8 16-bit values per lane; lane l
// holds row (A) / column (B) l % 32 and the k-group l / 32.
template <int DT>
__device__ __forceinline__ mfa_f32x16 mfa_mfma32(mfa_u32x4 a, mfa_u32x4 b, mfa_f32x16 c) {
    if constexpr (DT == MFA_DT_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(mfa_f16x8, a),
                                                       __builtin_bit_cast(mfa_f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(mfa_bf16x8, a),
                                                        __builtin_bit_cast(mfa_bf16x8, b), c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32) * B(32x16).  Lane l holds row/column l % 16, k-group l / 16.
template <int DT>
__device__ __forceinline__ mfa_f32x4 mfa_mfma16(mfa_u32x4 a, mfa_u32x4 b, mfa_f32x4 c) {
    if constexpr (DT == MFA_DT_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mfa_f16x8, a),
                                                       __builtin_bit_cast(mfa_f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mfa_bf16x8, a),
                                                        __builtin_bit_cast(mfa_bf16x8, b), c, 0, 0, 0);
}

// Round two fp32 values to the 16-bit type (nearest, ties to even) and pack lo | hi<<16.
template <int DT>
__device__ __forceinline__ uint32_t mfa_pack2(float lo, float hi) {
    if constexpr (DT == MFA_DT_F16) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        h2 r = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, r);
    } else {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        b2 r = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, r);
    }
}

// Widen the low / high 16-bit half of a packed word to fp32 (exact).
template <int DT>
__device__ __forceinline__ float mfa_lo(uint32_t w) {
    if constexpr (DT == MFA_DT_F16)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    else
        return __builtin_bit_cast(float, w << 16);
}
template <int DT>
__device__ __forceinline__ float mfa_hi(uint32_t w) {
    if constexpr (DT == MFA_DT_F16)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    else
        return __builtin_bit_cast(float, w & 0xffff0000u);
}

__device__ __forceinline__ float mfa_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum of the two 16-bit values of a packed word, accumulated into c in fp32.
template <int DT>
__device__ __forceinline__ float mfa_sum2(uint32_t w, float c) {
    if constexpr (DT == MFA_DT_F16) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w), one, c, false);
    } else {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        const b2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w), one, c, false);
    }
}

// Buffer resource over [base, base + bytes): loads past the end return zero, with no
// branch and a 32-bit per-lane offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mfa_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ mfa_u32x4 mfa_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(mfa_u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds_base + 16 * l (lds_base must be the same for the whole wave).
__device__ __forceinline__ void mfa_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, off, 0, 0, 0);
}

// The same loads with the non-temporal cache policy (the nt bit), for data read exactly
// once (a decode's KV cache): on this chip a plain streaming read of 1 GiB measured
// 5.9 TB/s with the default policy and 6.7 TB/s with nt.
constexpr int kMfaNonTemporal = 2;
__device__ __forceinline__ mfa_u32x4 mfa_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(mfa_u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kMfaNonTemporal));
}
__device__ __forceinline__ void mfa_load16_lds_nt(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, off, 0, 0,
                                             kMfaNonTemporal);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): in each group of 16 lanes, lane i
// names 4 consecutive 16-bit values (row i/4, columns 4*(i%4) .. +3 of a 4 x 16 block)
// and receives column i of the block (rows 0..3), packed low to high.
__device__ __forceinline__ mfa_u32x2 mfa_lds_read_tr16(const void* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(mfa_u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<void*>(p))));
}

__device__ __forceinline__ float mfa_log2(float x) { return __builtin_amdgcn_logf(x); }

// Wave-uniform read of an int32 the kernel never writes, through the scalar data cache
// (a scalar load, counted by lgkmcnt rather than vmcnt).  p must be uniform.
__device__ __forceinline__ int32_t mfa_uniform_load(const int32_t* p) {
    return *(const __attribute__((address_space(4))) int32_t*)p;
}

// The two values of x held by lanes i and i + 32 (i = lane & 31), in that order, in every
// lane: v_permlane32_swap exchanges the upper half of its first operand with the lower
// half of its second, with no trip through LDS.  Written as inline asm because the
// compiler's own folding of the builtin takes its two results for one value; the leading
// s_nop covers the wait a permlane needs after a VALU write of its operands.
__device__ __forceinline__ mfa_f32x2 mfa_halves(float x) {
    float lo = x, hi = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
    return mfa_f32x2{lo, hi};
}
// Sum and maximum of x over the lane pair (i, i + 32); every lane gets the same bits.
__device__ __forceinline__ float mfa_pair_sum(float x) {
    const mfa_f32x2 h = mfa_halves(x);
    return h[0] + h[1];
}
__device__ __forceinline__ float mfa_pair_max(float x) {
    const mfa_f32x2 h = mfa_halves(x);
    return fmaxf(h[0], h[1]);
}
