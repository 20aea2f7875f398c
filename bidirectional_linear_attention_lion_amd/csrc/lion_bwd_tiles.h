// lion_bwd_tiles.h -- matrix-core fragments and per-row epilogues shared by the backward kernels of
// the full and the chunkwise form (gfx950).
//
// Staged operands are bf16 row tiles (RowTile<D, __bf16>, lion_stage.h) read in sub-blocks of kKB = 32
// rows, two 16-row halves.  rows_frag gives an operand whose contraction index is the channel; tr_frag
// one whose contraction index is the row (read transposed with ds_read_b64_tr_b16).  A product of two
// operands only needs both sides to map the contraction index onto (lane group g, element) the same
// way (lion_device.h).
#pragma once

#include "lion_device.h"
#include "lion_stage.h"

namespace lion {

constexpr int kKB = 32;   // rows per sub-block (two 16-row halves)

// Lane i (< 8) of the lane's 16-lane row (DPP row_newbcast; a multiply that uses it takes it as a DPP
// operand).  The separable mask's column factors travel this way: lane r < 8 of a row computes the
// factor of sub-block position 16 (r / 4) + 4 g + r % 4, the position slot 4 t + e of every lane of the
// row needs.
__device__ __forceinline__ float bwd_bcast16(float x, int i) {
    switch (i) {
#define LION_RB(I) \
    case I: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + I, 0xF, 0xF, false));
    LION_RB(0) LION_RB(1) LION_RB(2) LION_RB(3) LION_RB(4) LION_RB(5) LION_RB(6) LION_RB(7)
#undef LION_RB
    default: return x;
    }
}

// phi over the rows of a staged tile, in place; rows at or past `row_end` become zero rows.
template <int D, int KIND>
__device__ __forceinline__ void phi_stage(__bf16 *tile, int rows, int row_end, int tid, int nt) {
    using RT = RowTile<D, __bf16>;
    const int nslot = rows * RT::CPK;
    const int lane = tid & 63;
    const int first = (KIND == kMaskD) ? row_end * RT::CPK : 0;   // identity phi: only the padding
    for (int sl0 = first - first % 64; sl0 < nslot; sl0 += nt) {
        const int sl = sl0 + tid;
        if (sl - lane >= nslot) break;   // wave-uniform: nslot is a multiple of 64
        const bool mine = sl >= first && sl < nslot;
        const int row = sl / RT::CPK;
        __bf16 x[8];
        __builtin_memcpy(x, tile + (size_t)sl * 8, 16);
        float f[8], ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            f[e] = phi_pre<KIND>((float)x[e]);
            ss += f[e] * f[e];
        }
        float scl = row < row_end ? 1.f : 0.f;
        if constexpr (KIND == kMaskS) scl *= inv_norm(group_sum<RT::CPK>(ss));
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = f2bf(f[e] * scl);
        if (mine) __builtin_memcpy(tile + (size_t)sl * 8, x, 16);
    }
}

// B-operand fragments of one row (row index r of the wave's 16-row tile): fragment st of lane group g
// holds the eight channels 8 (4 st + g) .. + 7, phi applied (scaled by `ok`) or raw.
template <int D, int KIND, bool PHI>
__device__ __forceinline__ void row_frags(const __bf16 *row, bool ok, bf16x8 *out) {
    constexpr int NS = D / 32;
    float x[NS][8], ss = 0.f;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        const int g = (threadIdx.x & 63) >> 4;
        const bf16x8 raw = __builtin_bit_cast(bf16x8, ld16(row + 8 * (4 * st + g)));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[st][e] = PHI ? phi_pre<KIND>((float)raw[e]) : (float)raw[e];
            ss += x[st][e] * x[st][e];
        }
    }
    float sc = ok ? 1.f : 0.f;
    if constexpr (PHI && KIND == kMaskS) {
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        sc *= inv_norm(ss);
    }
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        bf16x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = f2bf(x[st][e] * sc);
        out[st] = f;
    }
}

// A-operand fragment of rows h*32 + {16 t + r} of a staged tile, channels 8 (4 st + g) .. + 7.
template <int D>
__device__ __forceinline__ bf16x8 rows_frag(const __bf16 *tile, int h, int t, int st, int r, int g) {
    using RT = RowTile<D, __bf16>;
    return *reinterpret_cast<const bf16x8 *>(tile + RT::off(h * kKB + 16 * t + r, 8 * (4 * st + g)));
}

// A-operand fragment of the transposed tile: lane (r, g) gets column 16 ct + r at rows h*32 + 4g + e
// and h*32 + 16 + 4g + e (see lion_stage.h).
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16 *tile, int h, int ct, int r, int g) {
    using RT = RowTile<D, __bf16>;
    const int row = h * kKB + 4 * g + (r >> 2), col = 16 * ct + 4 * (r & 3);
    const bf16x4 lo = read_tr_b16(tile + RT::off(row, col));
    const bf16x4 hi = read_tr_b16(tile + RT::off(row + 16, col));
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = lo[e];
        f[4 + e] = hi[e];
    }
    return f;
}

// The transposed Jacobian of phi at x (channels 16 ct + 4 g + e of one row, held by the four lanes of
// the row) applied to dphi: LIT elu+1 -> 1 or exp(x); D identity; S normalised silu,
// dx = silu'(x) (dphi - phi (phi.dphi)) / ||silu(x)||, silu'(x) = sig (1 + x (1 - sig)).
template <int D, int KIND>
__device__ __forceinline__ void phi_backward(const float (&x)[D / 16][4], f32x4 (&g4)[D / 16]) {
    if constexpr (KIND == kMaskLit) {
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!(x[ct][e] > 0.f)) g4[ct][e] *= fast_exp2(x[ct][e] * kLog2e);
    } else if constexpr (KIND == kMaskS) {
        float sig[D / 16][4], sv[D / 16][4], ss = 0.f;
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sig[ct][e] = __builtin_amdgcn_rcpf(1.f + fast_exp2(-x[ct][e] * kLog2e));
                sv[ct][e] = x[ct][e] * sig[ct][e];
                ss += sv[ct][e] * sv[ct][e];
            }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        const float inv = inv_norm(ss);
        float pg = 0.f;
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) pg += sv[ct][e] * inv * g4[ct][e];
        pg += __shfl_xor(pg, 16, 64);
        pg += __shfl_xor(pg, 32, 64);
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float ds = sig[ct][e] * (1.f + x[ct][e] * (1.f - sig[ct][e]));
                g4[ct][e] = ds * (g4[ct][e] - sv[ct][e] * inv * pg) * inv;
            }
    }
}

// Store four gradient values of row `row`, channels 16 ct + 4 g .. + 3.
__device__ __forceinline__ void store4(void *base, bool bf16, size_t off, f32x4 v) {
    if (bf16) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f2bf(v[e]);
        *reinterpret_cast<bf16x4 *>(reinterpret_cast<__bf16 *>(base) + off) = o;
    } else {
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(base) + off) = v;
    }
}

}  // namespace lion
