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
    float eps;
    int B, H, L, d;
    bool in_bf16;               // element type of q, k, v
    void *y;                    // [B, H, L, d]
    bool out_bf16;              // element type of y
    float *den_out;             // nullable [B, H, L]
    int C;                      // chunk size (chunk form only)
    void *workspace;            // form-specific scratch (may be NULL)
    size_t workspace_bytes;
};

// Each launcher enqueues its kernels on `stream` and returns hipSuccess or the launch error.
hipError_t launch_full(const AttnArgs &a, hipStream_t stream);
hipError_t launch_chunk(const AttnArgs &a, hipStream_t stream);
hipError_t launch_birnn(const AttnArgs &a, hipStream_t stream);

size_t chunk_workspace_bytes(int B, int H, int L, int d, int C);
size_t birnn_workspace_bytes(int B, int H, int L, int d);

}  // namespace lion
