// lion_device.h -- device-side building blocks shared by the LION attention kernels (gfx950).
//
// Matrix-core tiles: v_mfma_f32_16x16x32_bf16 (bf16 inputs) and v_mfma_f32_16x16x4_f32 (fp32
// inputs), both 16 x 16 fp32 outputs.  For a 64-lane wave, lane l = 16 g + r (r = l % 16,
// g = l / 16):
//   A operand: row r of A, the g-th group of K-slots     (8 bf16 values, or 1 fp32 value)
//   B operand: column r of B, the same g-th group of K-slots
//   D result : D[4 g + e][r], e = 0..3                   (4 fp32 values)
// The kernels only rely on A and B assigning K-slots to (g, element) the same way, so any
// consistent mapping of the contraction index onto (g, element) is exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lion {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaskLit = 0, kMaskD = 1, kMaskS = 2;

__device__ __forceinline__ float bf2f(__bf16 b) { return (float)b; }
__device__ __forceinline__ __bf16 f2bf(float f) { return (__bf16)f; }  // v_cvt_pk_bf16_f32, RNE

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// phi of one element, without the normalisation of LION-S:
//   LIT: elu(x) + 1 = x + 1 (x > 0), exp(x) (x <= 0);   D: x;   S: silu(x) = x / (1 + exp(-x)).
template <int KIND>
__device__ __forceinline__ float phi_pre(float x) {
    if constexpr (KIND == kMaskLit) {
        float e = fast_exp2(x * kLog2e);
        return x > 0.f ? x + 1.f : e;
    } else if constexpr (KIND == kMaskD) {
        return x;
    } else {
        return x * __builtin_amdgcn_rcpf(1.f + fast_exp2(-x * kLog2e));
    }
}

// Sum over the lanes of a group of `N` consecutive lanes (N a power of two <= 64).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = 1; m < N; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Scale factor of LION-S's L2 normalisation from a sum of squares (phi = 0 for a zero vector).
__device__ __forceinline__ float inv_norm(float ss) { return ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f; }

// Workgroup index -> tile index such that consecutive tiles run on the same XCD.  Workgroups are
// dispatched round-robin over the 8 XCDs; this gives XCD x the contiguous tile range
// [x * per + min(x, rem), ...) so tiles of one (batch, head) share an L2.
__device__ __forceinline__ int xcd_tile(int bid, int nblocks) {
    constexpr int kXcd = 8;
    const int x = bid % kXcd, idx = bid / kXcd;
    const int per = nblocks / kXcd, rem = nblocks % kXcd;
    return x * per + (x < rem ? x : rem) + idx;
}

// Value known to be the same in every lane of the wave, kept in a scalar register (so branches on it
// are scalar branches rather than exec-mask divergence).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uniform(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

}  // namespace lion
