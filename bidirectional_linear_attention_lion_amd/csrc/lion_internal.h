// lion_internal.h -- host-side interface between the C ABI and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace lion {

// Arguments common to the three forms, already validated by the ABI layer.
struct AttnArgs {
    const void *q, *k, *v;      // [B, H, L, d], bf16 or fp32
    const float *log_lambda;    // NULL (LIT), [H] (D), [B, H, L] (S)
    int kind;                   // 0 LIT, 1 D, 2 S
    bool causal;                // keys after the query masked out (the forward recurrence alone)
    const int *order;           // full form only, nullable: a second token order [L] (averaged masks)
    float eps;
    int B, H, L, d;
    bool in_bf16;               // element type of q, k, v
    bool fp32c;                 // compute in fp32: fp32 inputs, or bf16 inputs upcast exactly (LION_FP32_ARITH)
    void *y;                    // [B, H, L, d]
    bool out_bf16;              // element type of y
    float *den_out;             // nullable [B, H, L]
    int C;                      // chunk size (chunk form only)
    void *workspace;            // form-specific scratch (may be NULL)
    size_t workspace_bytes;
};

// What a form needs for given sizes, decided on the host without any HIP call.
struct Plan {
    bool ok;            // false: the sizes exceed what the kernels support (e.g. LDS per workgroup)
    size_t workspace;   // bytes of caller workspace the launch will use
};

constexpr size_t kLdsPerWorkgroup = 160 * 1024;   // gfx950 LDS available to one workgroup

// Arguments of the full form's backward pass, validated by the ABI layer (bf16 inputs).
struct BwdArgs {
    const void *q, *k, *v;      // [B, H, L, d] bf16
    const float *log_lambda;    // NULL (LIT), [H] (D), [B, H, L] (S)
    int kind;
    bool causal;
    int B, H, L, d;
    const void *y, *dy;         // [B, H, L, d] bf16
    const float *den;           // [B, H, L]: the forward's row sums + eps
    void *dq, *dk, *dv;         // [B, H, L, d]
    bool g_bf16;                // element type of dq, dk, dv
    float *dll;                 // NULL (LIT), [H] (D), [B, H, L] (S)
    int C;                      // chunk size (chunk form's backward only)
    void *workspace;
    size_t workspace_bytes;
};

// Arguments of the LION-S selectivity prologue, validated by the ABI layer.
struct SelArgs {
    const void *x, *w;          // [B, L, Dm], [H, Dm] bf16
    const float *bias;          // [H]
    int B, L, H, Dm;
    float *log_lambda;          // [B, H, L]
    float *key_scale;           // nullable [B, H, L]
    const void *k;              // nullable [B, H, L, d] bf16
    void *k_out;                // with k
    int d;
};

Plan plan_full(const AttnArgs &a);
Plan plan_selectivity(const SelArgs &a);
Plan plan_full_bwd(const BwdArgs &a);
Plan plan_chunk_bwd(const BwdArgs &a);
Plan plan_chunk_bwd_mfma(const BwdArgs &a);   // chunks of 64 and 128 (bf16 matrix cores)
Plan plan_chunk(const AttnArgs &a);
Plan plan_chunk2(const AttnArgs &a);
Plan plan_birnn(const AttnArgs &a);

// Each launcher enqueues its kernels on `stream` and returns hipSuccess or the launch error.
// Callers check the form's plan first.
hipError_t launch_full(const AttnArgs &a, hipStream_t stream);
hipError_t launch_full_bwd(const BwdArgs &a, hipStream_t stream);
hipError_t launch_chunk_bwd(const BwdArgs &a, hipStream_t stream);
hipError_t launch_chunk_bwd_mfma(const BwdArgs &a, hipStream_t stream);
// The full form's backward as one chunk of the chunkwise main kernel (d of 32 or 64, L <= 256; the
// full form's workspace).
bool single_chunk_bwd_ok(const BwdArgs &a);
hipError_t launch_single_chunk_bwd(const BwdArgs &a, hipStream_t stream);
// dlog(lambda) from the two halves of dA ([B, H, L] each): LION-S a reverse prefix sum per (batch,
// head), LION-D sum_t t dA_t per head over the batch.  kind is 1 (D) or 2 (S).
hipError_t launch_dll(int kind, float *da_row, float *da_col, float *dll, int B, int H, int L, hipStream_t stream);
// LION-D dlog(lambda) from per-(batch, head) token sums: part is fp32 [B, H, 4], two hi/lo pairs each.
hipError_t launch_dll_parts(const float *part, float *dll, int B, int H, hipStream_t stream);
hipError_t launch_selectivity(const SelArgs &a, hipStream_t stream);
hipError_t launch_chunk(const AttnArgs &a, hipStream_t stream);
hipError_t launch_chunk2(const AttnArgs &a, hipStream_t stream);
hipError_t launch_birnn(const AttnArgs &a, hipStream_t stream);

}  // namespace lion
