// Internal interface between the C ABI layer (mfa_api.cpp) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "mfa.h"

struct MfaFwdProblem {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    int32_t* tile_log;   // nullable: per-tile visit record
    int B, Hq, Hkv, Nq, Nk, D;
    float scale;
    int causal, left, right;
    int dtype;
    // packed variable-length sequences (NULL for the dense [B, H, N, D] layout): Nq, Nk
    // then hold max_seqlen_q, max_seqlen_k
    const int32_t* cu_seqlens_q;
    const int32_t* cu_seqlens_k;
    int total_q, total_k;
    // keys in a paged cache (with packed queries; NULL otherwise): Nk then holds the
    // block table's capacity max_pages * 16
    const int32_t* block_table;
    const int32_t* seq_lens_k;
    int num_pages, max_pages;
    // dense forward with modifiers / block mask (NULL otherwise)
    const mfa_fwd_ext_args* ext;
};

struct MfaDecodeProblem {
    const void* q;
    const void* k_pages;
    const void* v_pages;
    const int32_t* block_table;
    const int32_t* seq_lens;
    void* out;
    float* lse;
    int B, Hq, Hkv, D;
    int num_pages, max_pages_per_seq;
    float scale;
    int num_splits;      // resolved (> 0)
    int chunk_pages;     // pages per split
    void* workspace;
    int dtype;
    int nq;              // query tokens per sequence (1 for mfa_decode_paged)
    int multi;           // 1: the multi-token kernel (mfa_decode_paged_multi)
};

struct MfaBwdProblem {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    void* workspace;     // 2 * B * Hq * Nq floats
    int B, Hq, Hkv, Nq, Nk, D;
    float scale;
    int causal, left, right;
    int dtype;
};

// Compute units of the current device (cached per device).
int mfa_num_cus();

int mfa_fwd_bm();
int mfa_fwd_bn(int D);
int mfa_fwd_groups(long long q_tiles, int Hq, int num_cus);
int mfa_fwd_launch(const MfaFwdProblem& p, hipStream_t stream, mfa_dispatch_info* info);

int mfa_bwd_launch(const MfaBwdProblem& p, hipStream_t stream, mfa_dispatch_info* info);

// Pages per split of the decode kernels for nq new tokens per sequence.
int mfa_decode_chunk_pages(int max_pages_per_seq, int num_splits, int nq);
// Device address and size of the current device's fixed decode scratch (looked up once per
// device); MFA_ERR_HIP if the lookup fails.
int mfa_decode_scratch(void** ptr, size_t* bytes);
int mfa_decode_launch(const MfaDecodeProblem& p, hipStream_t stream, mfa_dispatch_info* info);
