// lion_birnn.hip -- bidirectional RNN form of LION masked linear attention.
//
// "LION: A bidirectional framework that trains like a Transformer and infers like an RNN",
// reply "Concern 1" (Theorem 3.3 Eq. 20-24) and reply "1: Recurrence Form of Linear Attention":
//   forward  S^F_t = lambda_t S^F_{t-1} + phi(k_t) v_t^T,      z^F_t = lambda_t z^F_{t-1} + phi(k_t)
//   backward S^B_t = lambda_{t+1} S^B_{t+1} + phi(k_t) v_t^T,  z^B_t likewise
//   y_t = (q_t^T S^F_t + q_t^T S^B_t - (q_t.k_t) v_t) / (q_t^T z^F_t + q_t^T z^B_t - q_t.k_t + eps)
// with q, k after phi; the diagonal term appears in both recurrences and is counted once.  Only a
// vector y and a scalar c per token and direction are kept (the pages' O(Ld + L) memory).
//
// Work split: one workgroup per (batch, head, group of CW value columns) -- columns of y never interact,
// so groups need no communication -- with NR waves per direction.  A wave's lane is a value column c
// of the group (lane % CW) in one of 64 / CW row slices (lane / CW); the lane holds RW rows of that
// column of the d x d state in registers (RW = d CW / (64 NR)).  Per token and element the state update
// and the output dot product are one v_fmac_f32 each: k_i and q_i reach every lane through the DPP
// row_newbcast modifier (lane i of each 16-lane row broadcast to the row), folded into the
// instruction.  The decay is taken out of the per-element work by carrying S' = S / Lambda_t, Lambda_t
// the running product of the decays inside a 16-token block: S'_t = S'_{t-1} + (k_t / Lambda_t) v_t^T
// and q^T S_t = Lambda_t q^T S'_t; S' is brought back to scale at every block start, and within a block
// whenever Lambda would fall below 2^-60 (a decay of 0 simply resets the state).  The row-sum state z is
// kept once per 16-lane row (lane i holding z_i); q.z is a 16-lane DPP sum, taken for the whole block
// at its end.
//
// Tokens go in blocks of kT = 16 per direction.  A block's phi(q), phi(k), v, diagonal and scale
// factors are staged in LDS from rows loaded during the previous block; the recurrences write per-slice
// partials of y and q.z to LDS; then the partials are reduced: a token the other direction visited in
// an earlier block is finished with the partial parked then, a token whose other visit comes in a later
// block is parked (in the caller's workspace), and a token both directions visit within this block is
// finished directly.  The first visitor removes the diagonal, so it is counted once.
//
// Causal variant (keys after the query masked out): the forward recurrence alone, each token finished
// from its own forward partial, y_t = q_t^T S^F_t / (q_t^T z^F_t + eps) -- its diagonal term is
// counted once already, and nothing is parked.  The plain kernel then runs only the forward waves.
#include <type_traits>

#include "lion_device.h"
#include "lion_internal.h"

namespace lion {
namespace {

constexpr int kT = 16;   // tokens per block and direction

struct RnnParams {
    const void *q, *k, *v;
    const float *ll;
    float eps;
    int H, L;
    void *y;
    int out_bf16;
    float *den_out;
    float *park;   // [B*H][groups][L][CW+1]: one direction's partial (y, c) of each token
    int causal;    // forward direction only
};

// ---- DPP broadcast fused multiply-adds ---------------------------------------------------------------
// The DPP source (kb, qb) must not be written by a VALU instruction in the two instructions before a DPP
// read; each block starts with s_nop 1 since the compiler does not track hazards inside inline asm.
#define LION_BC_S(i) "v_fmac_f32_dpp %[s" #i "], %[kb], %[vj] row_newbcast:" #i " row_mask:0xf bank_mask:0xf\n\t"
#define LION_BC_Y(i, a) "v_fmac_f32_dpp %[" a "], %[qb], %[s" #i "] row_newbcast:" #i " row_mask:0xf bank_mask:0xf\n\t"

// S[i] += k_(row base + i) * vj for i < N, k broadcast from lane i of each 16-lane row of kb.
template <int N>
__device__ __forceinline__ void dpp_update(float *S, float kb, float vj);
template <>
__device__ __forceinline__ void dpp_update<16>(float *S, float kb, float vj) {
    asm volatile("s_nop 1\n\t" LION_BC_S(0) LION_BC_S(1) LION_BC_S(2) LION_BC_S(3) LION_BC_S(4) LION_BC_S(5)
                     LION_BC_S(6) LION_BC_S(7) LION_BC_S(8) LION_BC_S(9) LION_BC_S(10) LION_BC_S(11) LION_BC_S(12)
                         LION_BC_S(13) LION_BC_S(14) LION_BC_S(15)
                 : [s0] "+v"(S[0]), [s1] "+v"(S[1]), [s2] "+v"(S[2]), [s3] "+v"(S[3]), [s4] "+v"(S[4]),
                   [s5] "+v"(S[5]), [s6] "+v"(S[6]), [s7] "+v"(S[7]), [s8] "+v"(S[8]), [s9] "+v"(S[9]),
                   [s10] "+v"(S[10]), [s11] "+v"(S[11]), [s12] "+v"(S[12]), [s13] "+v"(S[13]), [s14] "+v"(S[14]),
                   [s15] "+v"(S[15])
                 : [kb] "v"(kb), [vj] "v"(vj));
}
template <>
__device__ __forceinline__ void dpp_update<8>(float *S, float kb, float vj) {
    asm volatile("s_nop 1\n\t" LION_BC_S(0) LION_BC_S(1) LION_BC_S(2) LION_BC_S(3) LION_BC_S(4) LION_BC_S(5)
                     LION_BC_S(6) LION_BC_S(7)
                 : [s0] "+v"(S[0]), [s1] "+v"(S[1]), [s2] "+v"(S[2]), [s3] "+v"(S[3]), [s4] "+v"(S[4]),
                   [s5] "+v"(S[5]), [s6] "+v"(S[6]), [s7] "+v"(S[7])
                 : [kb] "v"(kb), [vj] "v"(vj));
}
template <>
__device__ __forceinline__ void dpp_update<4>(float *S, float kb, float vj) {
    asm volatile("s_nop 1\n\t" LION_BC_S(0) LION_BC_S(1) LION_BC_S(2) LION_BC_S(3)
                 : [s0] "+v"(S[0]), [s1] "+v"(S[1]), [s2] "+v"(S[2]), [s3] "+v"(S[3])
                 : [kb] "v"(kb), [vj] "v"(vj));
}
template <>
__device__ __forceinline__ void dpp_update<2>(float *S, float kb, float vj) {
    asm volatile("s_nop 1\n\t" LION_BC_S(0) LION_BC_S(1)
                 : [s0] "+v"(S[0]), [s1] "+v"(S[1])
                 : [kb] "v"(kb), [vj] "v"(vj));
}

// y0 += q_i S[i] (even i), y1 += q_i S[i] (odd i) for i < N, q broadcast like k above.
template <int N>
__device__ __forceinline__ void dpp_dot(float &y0, float &y1, float qb, const float *S);
template <>
__device__ __forceinline__ void dpp_dot<16>(float &y0, float &y1, float qb, const float *S) {
    asm volatile("s_nop 1\n\t" LION_BC_Y(0, "y0") LION_BC_Y(1, "y1") LION_BC_Y(2, "y0") LION_BC_Y(3, "y1")
                     LION_BC_Y(4, "y0") LION_BC_Y(5, "y1") LION_BC_Y(6, "y0") LION_BC_Y(7, "y1") LION_BC_Y(8, "y0")
                         LION_BC_Y(9, "y1") LION_BC_Y(10, "y0") LION_BC_Y(11, "y1") LION_BC_Y(12, "y0")
                             LION_BC_Y(13, "y1") LION_BC_Y(14, "y0") LION_BC_Y(15, "y1")
                 : [y0] "+v"(y0), [y1] "+v"(y1)
                 : [qb] "v"(qb), [s0] "v"(S[0]), [s1] "v"(S[1]), [s2] "v"(S[2]), [s3] "v"(S[3]), [s4] "v"(S[4]),
                   [s5] "v"(S[5]), [s6] "v"(S[6]), [s7] "v"(S[7]), [s8] "v"(S[8]), [s9] "v"(S[9]), [s10] "v"(S[10]),
                   [s11] "v"(S[11]), [s12] "v"(S[12]), [s13] "v"(S[13]), [s14] "v"(S[14]), [s15] "v"(S[15]));
}
template <>
__device__ __forceinline__ void dpp_dot<8>(float &y0, float &y1, float qb, const float *S) {
    asm volatile("s_nop 1\n\t" LION_BC_Y(0, "y0") LION_BC_Y(1, "y1") LION_BC_Y(2, "y0") LION_BC_Y(3, "y1")
                     LION_BC_Y(4, "y0") LION_BC_Y(5, "y1") LION_BC_Y(6, "y0") LION_BC_Y(7, "y1")
                 : [y0] "+v"(y0), [y1] "+v"(y1)
                 : [qb] "v"(qb), [s0] "v"(S[0]), [s1] "v"(S[1]), [s2] "v"(S[2]), [s3] "v"(S[3]), [s4] "v"(S[4]),
                   [s5] "v"(S[5]), [s6] "v"(S[6]), [s7] "v"(S[7]));
}
template <>
__device__ __forceinline__ void dpp_dot<4>(float &y0, float &y1, float qb, const float *S) {
    asm volatile("s_nop 1\n\t" LION_BC_Y(0, "y0") LION_BC_Y(1, "y1") LION_BC_Y(2, "y0") LION_BC_Y(3, "y1")
                 : [y0] "+v"(y0), [y1] "+v"(y1)
                 : [qb] "v"(qb), [s0] "v"(S[0]), [s1] "v"(S[1]), [s2] "v"(S[2]), [s3] "v"(S[3]));
}
template <>
__device__ __forceinline__ void dpp_dot<2>(float &y0, float &y1, float qb, const float *S) {
    asm volatile("s_nop 1\n\t" LION_BC_Y(0, "y0") LION_BC_Y(1, "y1")
                 : [y0] "+v"(y0), [y1] "+v"(y1)
                 : [qb] "v"(qb), [s0] "v"(S[0]), [s1] "v"(S[1]));
}
// As dpp_dot, but y0 and y1 start at the first two products (no accumulator to clear).
#define LION_BC_Y0(i, a) "v_mul_f32_dpp %[" a "], %[qb], %[s" #i "] row_newbcast:" #i " row_mask:0xf bank_mask:0xf\n\t"
template <int N>
__device__ __forceinline__ void dpp_dot_first(float &y0, float &y1, float qb, const float *S);
template <>
__device__ __forceinline__ void dpp_dot_first<16>(float &y0, float &y1, float qb, const float *S) {
    asm volatile("s_nop 1\n\t" LION_BC_Y0(0, "y0") LION_BC_Y0(1, "y1") LION_BC_Y(2, "y0") LION_BC_Y(3, "y1")
                     LION_BC_Y(4, "y0") LION_BC_Y(5, "y1") LION_BC_Y(6, "y0") LION_BC_Y(7, "y1") LION_BC_Y(8, "y0")
                         LION_BC_Y(9, "y1") LION_BC_Y(10, "y0") LION_BC_Y(11, "y1") LION_BC_Y(12, "y0")
                             LION_BC_Y(13, "y1") LION_BC_Y(14, "y0") LION_BC_Y(15, "y1")
                 : [y0] "=&v"(y0), [y1] "=&v"(y1)
                 : [qb] "v"(qb), [s0] "v"(S[0]), [s1] "v"(S[1]), [s2] "v"(S[2]), [s3] "v"(S[3]), [s4] "v"(S[4]),
                   [s5] "v"(S[5]), [s6] "v"(S[6]), [s7] "v"(S[7]), [s8] "v"(S[8]), [s9] "v"(S[9]), [s10] "v"(S[10]),
                   [s11] "v"(S[11]), [s12] "v"(S[12]), [s13] "v"(S[13]), [s14] "v"(S[14]), [s15] "v"(S[15]));
}
template <>
__device__ __forceinline__ void dpp_dot_first<8>(float &y0, float &y1, float qb, const float *S) {
    asm volatile("s_nop 1\n\t" LION_BC_Y0(0, "y0") LION_BC_Y0(1, "y1") LION_BC_Y(2, "y0") LION_BC_Y(3, "y1")
                     LION_BC_Y(4, "y0") LION_BC_Y(5, "y1") LION_BC_Y(6, "y0") LION_BC_Y(7, "y1")
                 : [y0] "=&v"(y0), [y1] "=&v"(y1)
                 : [qb] "v"(qb), [s0] "v"(S[0]), [s1] "v"(S[1]), [s2] "v"(S[2]), [s3] "v"(S[3]), [s4] "v"(S[4]),
                   [s5] "v"(S[5]), [s6] "v"(S[6]), [s7] "v"(S[7]));
}
template <>
__device__ __forceinline__ void dpp_dot_first<4>(float &y0, float &y1, float qb, const float *S) {
    asm volatile("s_nop 1\n\t" LION_BC_Y0(0, "y0") LION_BC_Y0(1, "y1") LION_BC_Y(2, "y0") LION_BC_Y(3, "y1")
                 : [y0] "=&v"(y0), [y1] "=&v"(y1)
                 : [qb] "v"(qb), [s0] "v"(S[0]), [s1] "v"(S[1]), [s2] "v"(S[2]), [s3] "v"(S[3]));
}
template <>
__device__ __forceinline__ void dpp_dot_first<2>(float &y0, float &y1, float qb, const float *S) {
    asm volatile("s_nop 1\n\t" LION_BC_Y0(0, "y0") LION_BC_Y0(1, "y1")
                 : [y0] "=&v"(y0), [y1] "=&v"(y1)
                 : [qb] "v"(qb), [s0] "v"(S[0]), [s1] "v"(S[1]));
}
#undef LION_BC_Y0
#undef LION_BC_S
#undef LION_BC_Y

// Sum over the 16 lanes of each row (every lane receives its row's sum).
__device__ __forceinline__ float row16_sum(float x) {
    auto dpp = [](float v, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), decltype(ctrl)::value,
                                                                     0xF, 0xF, true));
    };
    x += dpp(x, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
    x += dpp(x, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
    x += dpp(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
    x += dpp(x, std::integral_constant<int, 0x140>{});   // row_mirror
    return x;
}


template <int D, int CW, int NR>
struct RnnShape {
    static constexpr int NS = 64 / CW;              // row slices per wave
    static constexpr int RW = D * CW / (64 * NR);   // state rows per lane
    static constexpr int RB = RW < 16 ? RW : 16;    // rows per DPP block
    static constexpr int KV = (RW + 15) / 16;       // DPP blocks per lane
    static constexpr int NG = D / CW;               // column groups
    static constexpr int NP = NR * NS;              // partials per column
};

template <int D, int KIND, int CW, int NR, bool BF16>
__global__ void __launch_bounds__(2 * NR * 64) __attribute__((amdgpu_waves_per_eu(3))) birnn_kernel(RnnParams p) {
    using T = std::conditional_t<BF16, __bf16, float>;
    using Sh = RnnShape<D, CW, NR>;
    constexpr int NS = Sh::NS, RW = Sh::RW, RB = Sh::RB, KV = Sh::KV, NG = Sh::NG, NP = Sh::NP;
    constexpr int NTD = NR * 64;              // threads per direction
    constexpr int TPT = D / 4;                // staging threads per token (4 channels each)
    constexpr int PAIRS = kT * TPT;
    constexpr int PPT = (PAIRS + NTD - 1) / NTD;
    constexpr int QKS = kT * D + 16;          // q/k staging floats (padded: lanes past a slice read on)
    constexpr int RITER = (kT * CW + NTD - 1) / NTD;
    constexpr float kRenorm = 8.673617379884035e-19f;   // 2^-60
    static_assert(RW >= 2 && RW <= 64 && RW % RB == 0, "rows per lane");

    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int dir = uniform(tid / NTD);       // 0 forward, 1 backward
    const int dt = tid % NTD;
    const int lane = tid & 63;
    const int rg = uniform(dt >> 6);          // wave within the direction
    const int c = lane % CW, sub = lane / CW;
    const int slice = rg * NS + sub;
    const int rb = slice * RW;                // first state row of this lane
    const int L = p.L;
    const int bid = blockIdx.x, bh = bid / NG, cg = bid % NG;
    const int col = cg * CW + c;
    const size_t base = (size_t)bh * L;

    // LDS: per direction [Qs][Ks][Vs][diag][ksc][ysc][mult], then Yp[2][kT][NP][CW] and Cp[2][kT][NP]
    constexpr int DIRF = 2 * QKS + kT * D + 4 * kT;
    float *stg = reinterpret_cast<float *>(smem) + dir * DIRF;
    float *Qs = stg, *Ks = Qs + QKS, *Vs = Ks + QKS, *sdiag = Vs + kT * D, *ksc = sdiag + kT, *ysc = ksc + kT,
          *mult = ysc + kT;
    float *Yp = reinterpret_cast<float *>(smem) + 2 * DIRF;
    float *Cp = Yp + 2 * kT * NP * CW;
    float *park = p.park + (size_t)bid * L * (CW + 1);

    const T *qg = reinterpret_cast<const T *>(p.q) + base * D;
    const T *kg = reinterpret_cast<const T *>(p.k) + base * D;
    const T *vg = reinterpret_cast<const T *>(p.v) + base * D;
    const float lg_head = (KIND == kMaskD) ? p.ll[bh % p.H] * kLog2e : 0.f;
    auto token_at = [&](int s) { return dir == 0 ? s : L - 1 - s; };
    // decay applied before adding the token visited at step s: lambda_t forward, lambda_{t+1} backward
    auto decay_at = [&](int s) -> float {
        if constexpr (KIND == kMaskLit) return 1.f;
        else if constexpr (KIND == kMaskD) return fast_exp2(lg_head);
        else {
            const int td = dir == 0 ? s : L - s;
            return (s < L && td < L) ? fast_exp2(p.ll[base + td] * kLog2e) : 1.f;
        }
    };
    const int nblk = (L + kT - 1) / kT;

    // ---- staging: raw rows loaded during the previous block, then phi, diagonal, scale factors -----
    using V4 = std::conditional_t<BF16, bf16x4, f32x4>;   // kept in the input type: no wait at load
    V4 raw[PPT][3];
    auto prefetch = [&](int b) {
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            const int pr = dt + NTD * u;
            const int tl = pr / TPT, c4 = (pr % TPT) * 4;
            const size_t off = (size_t)token_at(min(b * kT + tl, L - 1)) * D + c4;
            if (pr < PAIRS) {
                raw[u][0] = *reinterpret_cast<const V4 *>(qg + off);
                raw[u][1] = *reinterpret_cast<const V4 *>(kg + off);
                raw[u][2] = *reinterpret_cast<const V4 *>(vg + off);
            }
        }
    };
    auto stage = [&](int b) {
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            const int pr0 = NTD * u;
            if (pr0 + dt - lane >= PAIRS) break;   // whole wave past the end (PAIRS is a multiple of 64)
            const int pr = pr0 + dt;
            const int tl = pr / TPT, c4 = (pr % TPT) * 4;
            const int s = b * kT + tl;
            const bool valid = s < L;
            float xq[4], xk[4], sq = 0.f, sk = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xq[e] = phi_pre<KIND>((float)raw[u][0][e]);
                xk[e] = phi_pre<KIND>((float)raw[u][1][e]);
                sq += xq[e] * xq[e];
                sk += xk[e] * xk[e];
            }
            float fq = valid ? 1.f : 0.f, fk = fq;
            if constexpr (KIND == kMaskS) {
                fq *= inv_norm(group_sum<TPT>(sq));
                fk *= inv_norm(group_sum<TPT>(sk));
            }
            float dg = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xq[e] *= fq;
                xk[e] *= fk;
                Qs[tl * D + c4 + e] = xq[e];
                Ks[tl * D + c4 + e] = xk[e];
                Vs[tl * D + c4 + e] = (float)raw[u][2][e];
                dg += xq[e] * xk[e];
            }
            dg = group_sum<TPT>(dg);
            if (c4 == 0) {
                sdiag[tl] = dg;
                if constexpr (KIND != kMaskLit) {
                    // replay the block's scale sequence up to this token (every leader derives the same)
                    float lam = 1.f, mu = 1.f;
                    for (int u2 = 0; u2 <= tl; ++u2) {
                        const float l2 = lam * decay_at(b * kT + u2);
                        if (l2 < kRenorm) {
                            mu = l2;
                            lam = 1.f;
                        } else {
                            mu = 1.f;
                            lam = l2;
                        }
                    }
                    ksc[tl] = 1.f / lam;
                    ysc[tl] = lam;
                    mult[tl] = mu;
                }
            }
        }
    };

    // ---- state: S'[i] = rows rb + i of column col; z' per 16-lane row (lane i%16 of block m: row 16m+i) --
    float S[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) S[i] = 0.f;
    float z[KV], zmask[KV];
#pragma unroll
    for (int m = 0; m < KV; ++m) {
        z[m] = 0.f;
        zmask[m] = 16 * m + (lane & 15) < RW ? 1.f : 0.f;
    }
    float lam_end = 1.f;   // scale of S' at the end of the previous block

    prefetch(0);
    stage(0);
    // the 16 floats after the last token's q and k rows, which lanes past the last slice read (and mask
    // out by multiplying with zero), must hold finite values: zeros
    if (dt < 32) stg[(dt < 16 ? 0 : QKS) + kT * D + (dt & 15)] = 0.f;
    __syncthreads();

    for (int b = 0; b < nblk; ++b) {
        const int s0 = b * kT;
        const int nsteps = min(kT, L - s0);
        // the next block's rows load while this block's recurrence runs (staged after the reduction).
        // The previous reduction's stores are drained first: with stores still counted alongside the
        // loads, the compiler would otherwise wait for the loads too before reusing a store's registers.
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        if (b + 1 < nblk) prefetch(b + 1);

        // ---- recurrence over the block's tokens ------------------------------------------------------
        if constexpr (KIND != kMaskLit) {
#pragma unroll
            for (int i = 0; i < RW; ++i) S[i] *= lam_end;
#pragma unroll
            for (int m = 0; m < KV; ++m) z[m] *= lam_end;
        }
        // per-token scalars of the block, one register each (lane t holds token t's value); the tokens
        // where the state is renormalised, as a scalar bit mask
        const float kscv = KIND != kMaskLit ? ksc[lane & 15] : 1.f;
        const float multv = KIND != kMaskLit ? mult[lane & 15] : 1.f;
        const unsigned rmask = KIND != kMaskLit ? (unsigned)(__ballot(multv != 1.f) & 0xFFFFu) : 0u;
        auto lane_val = [](float v, int i) {
            return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), i));
        };
        // this lane's k, q (rows rb + 16m + lane % 16) and v of token tl; loaded one token ahead
        struct Tok {
            float kb[KV], qb[KV], vj;
        };
        auto load_tok = [&](int tl) {
            Tok x;
            const float *qrow = Qs + tl * D + rb + (lane & 15);
            const float *krow = Ks + tl * D + rb + (lane & 15);
#pragma unroll
            for (int m = 0; m < KV; ++m) {
                x.kb[m] = krow[16 * m];
                x.qb[m] = qrow[16 * m];
            }
            x.vj = Vs[tl * D + col];
            return x;
        };
        float cpv[kT];
        Tok cur = load_tok(0);
#pragma unroll
        for (int tl = 0; tl < kT; ++tl) {
            cpv[tl] = 0.f;
            if (tl >= nsteps) continue;
            // (unconditional: the staging buffer always holds kT rows; rows past the block are unused)
            Tok nxt;
            if (tl + 1 < kT) nxt = load_tok(tl + 1);
            float ks = 1.f;
            if constexpr (KIND != kMaskLit) {
                ks = lane_val(kscv, tl);
                if (rmask & (1u << tl)) {
                    const float mu = lane_val(multv, tl);
#pragma unroll
                    for (int i = 0; i < RW; ++i) S[i] *= mu;
#pragma unroll
                    for (int m = 0; m < KV; ++m) z[m] *= mu;
                }
            }
            float y0 = 0.f, y1 = 0.f, cp = 0.f;
#pragma unroll
            for (int m = 0; m < KV; ++m) {
                const float kb = cur.kb[m] * ks, qb = cur.qb[m];
                dpp_update<RB>(S + RB * m, kb, cur.vj);
                dpp_dot<RB>(y0, y1, qb, S + RB * m);
                z[m] += kb;
                cp += zmask[m] * qb * z[m];
            }
            // unscaled partials (q^T S' and q.z' of this slice); the scale and the diagonal are applied
            // once per token in the reduction
            cpv[tl] = cp;
            Yp[((dir * kT + tl) * NP + slice) * CW + c] = y0 + y1;
            if (tl + 1 < kT) cur = nxt;
        }
        if constexpr (KIND != kMaskLit) lam_end = ysc[nsteps - 1];
        // q.z partials of the block: 16 independent row sums, written by the first lane of each slice
#pragma unroll
        for (int tl = 0; tl < kT; ++tl) cpv[tl] = row16_sum(cpv[tl]);
        if (c == 0) {
#pragma unroll
            for (int tl = 0; tl < kT; ++tl) Cp[(dir * kT + tl) * NP + slice] = cpv[tl];
        }
        __syncthreads();

        // ---- reduce the partials: park, finish with a parked partial, or finish both directions ------
        // (the parked partials this block needs are loaded first, all at once)
        float pky[RITER], pkc[RITER];
#pragma unroll
        for (int it = 0; it < RITER; ++it) {
            const int idx = dt + NTD * it;
            pky[it] = pkc[it] = 0.f;
            if (idx < nsteps * CW) {
                const int tl = idx / CW, c2 = idx % CW;
                const int s = s0 + tl;
                if (!p.causal && L - 1 - s < s0) {
                    const size_t row = (size_t)token_at(s) * (CW + 1);
                    pky[it] = park[row + c2];
                    pkc[it] = park[row + CW];
                }
            }
        }
#pragma unroll
        for (int it = 0; it < RITER; ++it) {
            const int idx = dt + NTD * it;
            if (idx >= nsteps * CW) break;
            const int tl = idx / CW, c2 = idx % CW;
            const int s = s0 + tl, sp = L - 1 - s;
            const int t = token_at(s);
            float y = 0.f, cs = 0.f;
#pragma unroll
            for (int g = 0; g < NP; ++g) {
                y += Yp[((dir * kT + tl) * NP + g) * CW + c2];
                cs += Cp[(dir * kT + tl) * NP + g];
            }
            if constexpr (KIND != kMaskLit) {
                const float ys = ysc[tl];
                y *= ys;
                cs *= ys;
            }
            float yo, co, dg = 0.f;
            if (p.causal) {
                yo = co = 0.f;                            // the forward visit alone
            } else if (sp >= s0 + nsteps) {
                park[(size_t)t * (CW + 1) + c2] = y;
                if (c2 == 0) park[(size_t)t * (CW + 1) + CW] = cs;
                continue;
            } else if (sp < s0) {
                yo = pky[it];
                co = pkc[it];
            } else {
                if (dir == 1) continue;
                const int tp = sp - s0;
                yo = 0.f;
                co = 0.f;
#pragma unroll
                for (int g = 0; g < NP; ++g) {
                    yo += Yp[((kT + tp) * NP + g) * CW + c2];
                    co += Cp[(kT + tp) * NP + g];
                }
                if constexpr (KIND != kMaskLit) {
                    const float ys = ysc[DIRF + tp];   // the backward direction's scale of that token
                    yo *= ys;
                    co *= ys;
                }
            }
            // both visits included the diagonal term: remove it once
            if (!p.causal) dg = sdiag[tl];
            const float div = cs + co - dg + p.eps;
            const float out = (y + yo - dg * Vs[tl * D + cg * CW + c2]) / div;
            const size_t o = (base + t) * D + cg * CW + c2;
            if (p.out_bf16)
                reinterpret_cast<__bf16 *>(p.y)[o] = f2bf(out);
            else
                reinterpret_cast<float *>(p.y)[o] = out;
            if (p.den_out && cg == 0 && c2 == 0) p.den_out[base + t] = div;
        }
        // staging overwrites the rows, diagonal and scales the reduction reads (its own direction's and,
        // for tokens both directions visit in this block, the other direction's scales): every wave must
        // be done reducing first
        __syncthreads();
        if (b + 1 < nblk) stage(b + 1);
        __syncthreads();
    }
}

// ---- pipelined variant --------------------------------------------------------------------------------
// For grids of at most one workgroup per CU.  kHelp more waves take the per-block work off the
// recurrence waves, which then run nothing per token but the DPP products and the store of their
// partial: while they run block b, the helpers reduce block b-1 (park, finish, store), stage block b+1
// (phi, diagonal, k already divided by its scale Lambda_t, from rows loaded one block earlier), carry the
// row-sum states z of both directions through block b (one helper wave per direction, lane i holding
// z_i) and derive the scale factors of block b+2 (one helper wave).  One barrier per block separates the
// roles and the recurrence waves never touch global memory.  Staging is triple-buffered (b+1 is written
// while b is read and b-1 is still needed by its reduction), partials double-buffered, scale factors in
// a ring of four blocks (b-1 reduced, b running, b+1 staged, b+2 written).
constexpr int kHelp = 8;

template <int D, int CW, int NR>
struct PipeLayout {
    using Sh = RnnShape<D, CW, NR>;
    static constexpr int QKS = kT * D + 16;              // q or k rows of a block, then 16 zero floats
    static constexpr int DIRF = 2 * QKS + kT * D + kT;   // q, k / Lambda, v, diagonal of one direction
    static constexpr int YP = 2 * kT * Sh::NP * CW;      // per-slice partials q^T S' of a block
    static constexpr int PSZ = YP + 2 * kT;              // then q . z' per token and direction
    static constexpr int RING = 3 * 2 * kT;              // [k scale, y scale, multiplier][direction][token]
    static constexpr int ZST = 68;                       // row stride of the q . z transposition
    // offsets in floats: partials first, so a token's partial is an immediate offset from a per-block base
    static constexpr int PART = 0;
    static constexpr int STG = PART + 2 * PSZ;
    static constexpr int RNG = STG + 6 * DIRF;
    static constexpr int ZT = RNG + 4 * RING;
    static constexpr int TOTAL = ZT + 2 * kT * ZST;
};

template <int D, int CW, int NR>
constexpr size_t rnn_pipe_lds() {
    return (size_t)PipeLayout<D, CW, NR>::TOTAL * 4;
}

template <int D, int KIND, int CW, int NR, bool BF16>
__global__ void __launch_bounds__((2 * NR + kHelp) * 64) birnn_pipe_kernel(RnnParams p) {
    using T = std::conditional_t<BF16, __bf16, float>;
    using Sh = RnnShape<D, CW, NR>;
    using Ly = PipeLayout<D, CW, NR>;
    constexpr int NS = Sh::NS, RW = Sh::RW, RB = Sh::RB, KV = Sh::KV, NG = Sh::NG, NP = Sh::NP;
    constexpr int NTD = NR * 64;               // recurrence threads per direction
    constexpr int NRT = 2 * NTD;               // recurrence threads
    constexpr int NHT = kHelp * 64;            // helper threads
    constexpr int TPT = D / 4;                 // staging threads per token (4 channels each)
    constexpr int PAIRS = 2 * kT * TPT;        // staging units of a block, both directions
    constexpr int PPT = (PAIRS + NHT - 1) / NHT;
    constexpr int QKS = Ly::QKS, DIRF = Ly::DIRF, PSZ = Ly::PSZ, YP = Ly::YP;
    constexpr int RITEMS = 2 * kT * CW;        // reduction units of a block, both directions
    constexpr int RITER = (RITEMS + NHT - 1) / NHT;
    constexpr float kRenorm = 8.673617379884035e-19f;   // 2^-60
    static_assert(RW >= 2 && RW <= 64 && RW % RB == 0, "rows per lane");
    static_assert(PAIRS % 64 == 0, "staging units per wave");
    static_assert(kHelp >= 3, "two z waves and at least one reducing wave");
    // state update on the matrix cores (see the recurrence waves), not for fp32 inputs with 16 or more
    // rows per lane (registers)
    constexpr bool kMatrixUpdate = RW % 4 == 0 && (BF16 || RW < 16);

    extern __shared__ __align__(16) unsigned char smem[];
    float *S0 = reinterpret_cast<float *>(smem);
    auto part_of = [&](int b) { return S0 + Ly::PART + (b & 1) * PSZ; };
    auto stg_of = [&](int b, int d) { return S0 + Ly::STG + ((b % 3) * 2 + d) * DIRF; };
    auto ring_of = [&](int b) { return S0 + Ly::RNG + (b & 3) * Ly::RING; };

    const int tid = threadIdx.x, lane = tid & 63;
    const bool helper = uniform(tid) >= NRT;
    const int L = p.L;
    const int bid = blockIdx.x, bh = bid / NG, cg = bid % NG;
    const size_t base = (size_t)bh * L;
    float *park = p.park + (size_t)bid * L * (CW + 1);
    const int nblk = (L + kT - 1) / kT;

    if (helper) {
        // ================= helper waves =================================================================
        // Their work per block is the longer path (the recurrence waves wait at the barrier), so they
        // take the issue slots first where both are ready.
        __builtin_amdgcn_s_setprio(1);
        const int ht = tid - NRT;
        const int hw = uniform(ht >> 6);
        const T *qg = reinterpret_cast<const T *>(p.q) + base * D;
        const T *kg = reinterpret_cast<const T *>(p.k) + base * D;
        const T *vg = reinterpret_cast<const T *>(p.v) + base * D;
        const float lg_head = (KIND == kMaskD) ? p.ll[bh % p.H] * kLog2e : 0.f;
        auto token_at = [&](int d, int s) { return d == 0 ? s : L - 1 - s; };

        // Scale factors of block b, both directions (lanes 0-15 forward, 16-31 backward; the upper half
        // of the wave repeats them).  Inside a block the running product Lambda of the decays starts at 1;
        // where it would fall below 2^-60 the state is multiplied by that product instead and Lambda
        // restarts at 1.  Per token: 1 / Lambda (k scale), Lambda (y scale), the multiplier (1 if none).
        auto scales = [&](int b) {
            const int d = (lane >> 4) & 1, tl = lane & 15;
            const int s = b * kT + tl;
            float lg = 0.f;   // log2 of the decay applied at this step
            if (s < L && !(p.causal && d == 1)) {
                if constexpr (KIND == kMaskD) lg = lg_head;
                else lg = (d == 0 || s > 0) ? p.ll[base + (d == 0 ? s : L - s)] * kLog2e : 0.f;
            }
            // Usual case: the block's running product stays above 2^-59 in both directions, so no
            // multiplier is needed and Lambda_t = 2^(prefix sum of the log decays), summed within each
            // 16-lane row by four DPP row shifts.
            auto shr = [](float x, auto ctrl) {   // row_shr by ctrl - 0x110 lanes, 0 shifted in
                return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                             decltype(ctrl)::value, 0xF, 0xF, false));
            };
            float ps = lg;
            ps += shr(ps, std::integral_constant<int, 0x111>{});
            ps += shr(ps, std::integral_constant<int, 0x112>{});
            ps += shr(ps, std::integral_constant<int, 0x114>{});
            ps += shr(ps, std::integral_constant<int, 0x118>{});
            if (!__any(lane < 32 && ps < -59.f)) {
                if (lane < 32) {
                    float *rg = ring_of(b);
                    rg[d * kT + tl] = fast_exp2(-ps);
                    rg[(2 + d) * kT + tl] = fast_exp2(ps);
                    rg[(4 + d) * kT + tl] = 1.f;
                }
                return;
            }
            // otherwise the products step by step, restarting where they would fall below 2^-60
            const float dec = fast_exp2(lg);
            float lam = 1.f, ys = 1.f, mu_t = 1.f;
#pragma unroll
            for (int u = 0; u < kT; ++u) {
                const int i0 = __builtin_amdgcn_readlane(__builtin_bit_cast(int, dec), u);
                const int i1 = __builtin_amdgcn_readlane(__builtin_bit_cast(int, dec), kT + u);
                const float l2 = lam * __builtin_bit_cast(float, d == 0 ? i0 : i1);
                const bool rn = l2 < kRenorm;
                const float mu = rn ? l2 : 1.f;
                lam = rn ? 1.f : l2;
                if (u == tl) {
                    ys = lam;
                    mu_t = mu;
                }
            }
            if (lane < 32) {
                float *rg = ring_of(b);
                rg[d * kT + tl] = 1.f / ys;
                rg[(2 + d) * kT + tl] = ys;
                rg[(4 + d) * kT + tl] = mu_t;
            }
        };

        using V4 = std::conditional_t<BF16, bf16x4, f32x4>;
        V4 raw[PPT][3];
        auto prefetch = [&](int b) {
#pragma unroll
            for (int u = 0; u < PPT; ++u) {
                const int pr = ht + NHT * u;
                const int d = pr / (kT * TPT), tl = (pr % (kT * TPT)) / TPT, c4 = (pr % TPT) * 4;
                const size_t off = (size_t)token_at(d, min(b * kT + tl, L - 1)) * D + c4;
                if (pr < PAIRS && !(p.causal && d == 1)) {
                    raw[u][0] = *reinterpret_cast<const V4 *>(qg + off);
                    raw[u][1] = *reinterpret_cast<const V4 *>(kg + off);
                    raw[u][2] = *reinterpret_cast<const V4 *>(vg + off);
                }
            }
        };
        auto tok_sum = [](float x) {
            if constexpr (TPT == 16) return row16_sum(x);
            else return group_sum<TPT>(x);
        };
        auto stage = [&](int b) {
#pragma unroll
            for (int u = 0; u < PPT; ++u) {
                const int pr0 = NHT * u;
                if (pr0 + ht - lane >= PAIRS) break;   // whole wave past the end
                const int pr = pr0 + ht;
                const int d = pr / (kT * TPT), tl = (pr % (kT * TPT)) / TPT, c4 = (pr % TPT) * 4;
                if (p.causal && d == 1) break;        // wave-uniform: kT * TPT is a multiple of 64
                float *st = stg_of(b, d);
                float *Qs = st, *Ks = Qs + QKS, *Vs = Ks + QKS, *sdiag = Vs + kT * D;
                const int s = b * kT + tl;
                const bool valid = s < L;
                f32x4 xq, xk, xv;
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xq[e] = phi_pre<KIND>((float)raw[u][0][e]);
                    xk[e] = phi_pre<KIND>((float)raw[u][1][e]);
                    xv[e] = (float)raw[u][2][e];
                    sq += xq[e] * xq[e];
                    sk += xk[e] * xk[e];
                }
                float fq = valid ? 1.f : 0.f, fk = fq;
                if constexpr (KIND == kMaskS) {
                    fq *= inv_norm(tok_sum(sq));
                    fk *= inv_norm(tok_sum(sk));
                }
                const float ks = KIND != kMaskLit ? ring_of(b)[d * kT + tl] : 1.f;
                float dg = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xq[e] *= fq;
                    xk[e] *= fk;
                    dg += xq[e] * xk[e];
                    xk[e] *= ks;
                }
                *reinterpret_cast<f32x4 *>(Qs + tl * D + c4) = xq;
                *reinterpret_cast<f32x4 *>(Ks + tl * D + c4) = xk;
                *reinterpret_cast<f32x4 *>(Vs + tl * D + c4) = xv;
                dg = tok_sum(dg);
                if (c4 == 0) sdiag[tl] = dg;
            }
        };

        // Row-sum state of one direction through block b (helper wave d): z' = z' m_t + k_t / Lambda_t per
        // token, lane i holding z'_i (and z'_(i+64) for d = 128); the 16 products q_t . z'_t are summed
        // over the lanes by a transposition through LDS and written beside the block's partials.
        constexpr int ZR = D > 64 ? D / 64 : 1;
        float zr[ZR], zlam = 1.f;
#pragma unroll
        for (int j = 0; j < ZR; ++j) zr[j] = 0.f;
        auto zsum = [&](int b, int d) {
            const int s0 = b * kT, nsteps = min(kT, L - s0);
            const float *st = stg_of(b, d);
            const float *Qs = st, *Ks = Qs + QKS;
            const float *mult = ring_of(b) + (4 + d) * kT;
            float *zt = S0 + Ly::ZT + d * kT * Ly::ZST;
            if constexpr (KIND != kMaskLit) {
#pragma unroll
                for (int j = 0; j < ZR; ++j) zr[j] *= zlam;
            }
            // Every token of the block, with no branch between them, and the products kept in registers
            // until all are done: the loads of all tokens can be in flight together.  Tokens past the end
            // are staged with k = q = 0 and multiplier 1, so they leave z' as it is.
            // The block's loads (or a part at a time) issued before any use (the compiler
            // otherwise waits for each token's loads in turn).
            constexpr int kH = !BF16 ? kT / 4 : RW >= 16 ? kT / 2 : kT;   // (fewer at a time where registers are short)
            float xs[kT];
#pragma unroll
            for (int h = 0; h < kT / kH; ++h) {
                float kz[kH][ZR], qz[kH][ZR], mz[kH];
#pragma unroll
                for (int u = 0; u < kH; ++u) {
                    const int tl = h * kH + u;
                    mz[u] = KIND != kMaskLit ? mult[tl] : 1.f;
#pragma unroll
                    for (int j = 0; j < ZR; ++j) {
                        const int r = min(lane + 64 * j, D - 1);
                        kz[u][j] = Ks[tl * D + r];
                        qz[u][j] = Qs[tl * D + r];
                    }
                }
                asm volatile("" ::: "memory");   // keep the loads above
#pragma unroll
                for (int u = 0; u < kH; ++u) {
                    float x = 0.f;
#pragma unroll
                    for (int j = 0; j < ZR; ++j) {
                        if (lane + 64 * j < D) {
                            zr[j] = fmaf(zr[j], mz[u], kz[u][j]);
                            x = fmaf(qz[u][j], zr[j], x);
                        }
                    }
                    xs[h * kH + u] = x;
                }
            }
#pragma unroll
            for (int tl = 0; tl < kT; ++tl) zt[tl * Ly::ZST + lane] = xs[tl];
            // the same wave reads what its lanes wrote: LDS keeps a wave's accesses in order
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");
            const int t = lane >> 2, part = lane & 3;
            const f32x4 *src = reinterpret_cast<const f32x4 *>(zt + t * Ly::ZST + part * 16);
            float v = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 a = src[j];
                v += (a[0] + a[1]) + (a[2] + a[3]);
            }
            // sum over the 4 lanes of a token (DPP quad permutations: no LDS round trip)
            auto qp = [](float x, auto ctrl) {
                return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                             decltype(ctrl)::value, 0xF, 0xF, true));
            };
            v += qp(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
            v += qp(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
            if (part == 0) part_of(b)[YP + d * kT + t] = v;
            if constexpr (KIND != kMaskLit) zlam = ring_of(b)[(2 + d) * kT + nsteps - 1];
            asm volatile("" ::: "memory");
        };

        // parked partials block b's reduction needs: those parked at least two iterations before the
        // reduction (partner step < s0 - kT) are loaded an iteration ahead, the rest when reduced
        float pky[RITER], pkc[RITER];
        auto prefetch_park = [&](int b, bool ahead) {
            const int s0 = b * kT, nsteps = min(kT, L - s0);
#pragma unroll
            for (int it = 0; it < RITER; ++it) {
                const int idx = ht + NHT * it;
                const int d = idx / (kT * CW), tl = (idx % (kT * CW)) / CW, c2 = idx % CW;
                if (idx < RITEMS && tl < nsteps && !p.causal) {
                    const int s = s0 + tl, sp = L - 1 - s;
                    if (ahead ? sp < s0 - kT : (sp < s0 && sp >= s0 - kT)) {
                        const size_t row = (size_t)token_at(d, s) * (CW + 1);
                        pky[it] = park[row + c2];
                        pkc[it] = park[row + CW];
                    }
                }
            }
        };
        auto reduce = [&](int b) {
            const int s0 = b * kT, nsteps = min(kT, L - s0);
            const float *Yp = part_of(b), *Cp = Yp + YP;
            const float *ysc = ring_of(b) + 2 * kT;   // [direction][token]
            prefetch_park(b, false);
            // Every item's LDS operands first (indices past the end clamped: read, never used), then the
            // arithmetic, so the block's reduction waits for LDS once rather than once per partial.
            // items loaded together (registers: one at a time for fp32 inputs with four or more items)
            constexpr int kPair = (RITER < 2 || (!BF16 && RITER > 2)) ? 1 : 2;
#pragma unroll
            for (int i0 = 0; i0 < RITER; i0 += kPair) {
            float pp[kPair][NP], csl[kPair], scl[kPair], dgl[kPair], vl[kPair];
#pragma unroll
            for (int j = 0; j < kPair; ++j) {
                const int it = i0 + j;
                const int ic = min(ht + NHT * it, RITEMS - 1);
                const int d = ic / (kT * CW), tl = (ic % (kT * CW)) / CW, c2 = ic % CW;
#pragma unroll
                for (int g = 0; g < NP; ++g) pp[j][g] = Yp[((d * kT + tl) * NP + g) * CW + c2];
                csl[j] = Cp[d * kT + tl];
                scl[j] = KIND != kMaskLit ? ysc[d * kT + tl] : 1.f;
                const float *Vs = stg_of(b, d) + 2 * QKS;
                dgl[j] = Vs[kT * D + tl];
                vl[j] = Vs[tl * D + cg * CW + c2];
            }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int j = 0; j < kPair; ++j) {
                const int it = i0 + j;
                const int idx = ht + NHT * it;
                const int d = idx / (kT * CW), tl = (idx % (kT * CW)) / CW, c2 = idx % CW;
                if (idx >= RITEMS || tl >= nsteps || (p.causal && d == 1)) continue;
                const int s = s0 + tl, sp = L - 1 - s;
                const int t = token_at(d, s);
                float ps[NP];
#pragma unroll
                for (int g = 0; g < NP; ++g) ps[g] = pp[j][g];
#pragma unroll
                for (int w = 1; w < NP; w <<= 1)
#pragma unroll
                    for (int g = 0; g + w < NP; g += 2 * w) ps[g] += ps[g + w];
                float y = ps[0] * scl[j], cs = csl[j] * scl[j];
                float yo, co;
                if (p.causal) {
                    yo = co = 0.f;                        // the forward visit alone
                } else if (sp >= s0 + nsteps) {
                    park[(size_t)t * (CW + 1) + c2] = y;
                    if (c2 == 0) park[(size_t)t * (CW + 1) + CW] = cs;
                    continue;
                } else if (sp < s0) {
                    yo = pky[it];
                    co = pkc[it];
                } else {
                    if (d == 1) continue;
                    const int tp = sp - s0;
                    yo = 0.f;
#pragma unroll
                    for (int g = 0; g < NP; ++g) yo += Yp[((kT + tp) * NP + g) * CW + c2];
                    co = Cp[kT + tp];
                    if constexpr (KIND != kMaskLit) {
                        yo *= ysc[kT + tp];   // backward scale of that token
                        co *= ysc[kT + tp];
                    }
                }
                // q . z' of both visits includes the diagonal term q_t . k_t: remove it once.  With the
                // update on the matrix cores the partials q^T S' leave (q_t . k_t) v_t out: add it once;
                // otherwise both visits include it: remove it once
                const float dg = dgl[j];
                const float dgc = p.causal ? 0.f : dg;
                const float dgy = kMatrixUpdate ? dg : -dgc;
                const float div = cs + co - dgc + p.eps;
                const float out = (y + yo + dgy * vl[j]) * __builtin_amdgcn_rcpf(div);
                const size_t o = (base + t) * D + cg * CW + c2;
                if (p.out_bf16)
                    reinterpret_cast<__bf16 *>(p.y)[o] = f2bf(out);
                else
                    reinterpret_cast<float *>(p.y)[o] = out;
                if (p.den_out && cg == 0 && c2 == 0) p.den_out[base + t] = div;
            }
            }
        };

        // all helper waves stage and reduce; waves 0 and 1 also carry the row-sum states, the last one the
        // scale factors (each on a SIMD of its own)
        const bool scale_wave = KIND != kMaskLit && hw == kHelp - 1;
        if (scale_wave) {
            scales(0);
            if (1 < nblk) scales(1);
        }
        __syncthreads();   // scale factors of blocks 0 and 1
        prefetch(0);
        stage(0);
        if (1 < nblk) prefetch(1);
        // zeros after the last token's q and k rows of every staging buffer (read, never used, by lanes
        // past the last row slice)
        if (ht < 6 * 32) S0[Ly::STG + (ht / 32) * DIRF + (ht % 32 < 16 ? 0 : QKS) + kT * D + (ht & 15)] = 0.f;
        __syncthreads();
        for (int it = 0; it <= nblk; ++it) {
            if (it >= 1) reduce(it - 1);
            if (it + 1 < nblk) {
                stage(it + 1);
                if (it + 2 < nblk) prefetch(it + 2);
            }
            if (it < nblk && hw < 2 && !(p.causal && hw == 1)) zsum(it, hw);
            if (scale_wave && it + 2 < nblk) scales(it + 2);
            if (it < nblk) prefetch_park(it, true);
            __syncthreads();
        }
        return;
    }

    // ================= recurrence waves ================================================================
    const int dir = uniform(tid / NTD);        // 0 forward, 1 backward
    const int dt = tid % NTD;
    const int rg = uniform(dt >> 6);
    const int c = lane % CW, sub = lane / CW;
    const int slice = rg * NS + sub;
    const int rb = slice * RW;
    const int col = cg * CW + c;

    // State rows rb .. rb+RW-1 of column col, as RW/4 vectors: with a multiple of 4 rows per lane the
    // update S' += (k / Lambda) v^T runs on the matrix cores, v_mfma_f32_4x4x1f32 being 16 independent
    // 4 x 4 outer products per wave (output register r of lane l is row r of the 4-lane group's block:
    // the k of that row comes from lane 4 (l / 4) + r, the v from lane l itself).  The state is then
    // double-buffered: token t's product writes one copy while its dot product q^T S reads the other,
    // S'_(t-1), written a token earlier, so the vector units never wait for the matrix cores; the
    // diagonal term (q_t . k_t) v_t this leaves out is added in the reduction.  Otherwise (2 rows per
    // lane, or fp32 inputs with 16 or more) the update is DPP FMAs in place and the dot product reads S'_t.
    constexpr bool kMU = kMatrixUpdate;
    constexpr int NM = (RW + 3) / 4;
    f32x4 Sa[NM], Sb[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) Sa[m] = Sb[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lam_end = 1.f;
    __syncthreads();   // scale factors of blocks 0 and 1
    __syncthreads();   // block 0 staged
    const bool active = !(p.causal && dir == 1);
    for (int it = 0; it <= nblk; ++it) {
        if (it < nblk && active) {
            const int b = it, s0 = b * kT, nsteps = min(kT, L - s0);
            const float *st = stg_of(b, dir);
            const float *Qs = st, *Ks = Qs + QKS, *Vs = Ks + QKS;
            const float *ysc = ring_of(b) + (2 + dir) * kT, *mult = ysc + 2 * kT;
            float *yp = part_of(b) + (dir * kT * NP + slice) * CW + c;
            if constexpr (KIND != kMaskLit) {
#pragma unroll
                for (int m = 0; m < NM; ++m) Sa[m] *= lam_end;
            }
            const float multv = KIND != kMaskLit ? mult[lane & 15] : 1.f;
            const unsigned rmask = KIND != kMaskLit ? (unsigned)(__ballot(multv != 1.f) & 0xFFFFu) : 0u;
            struct Tok {
                float ka[kMU ? NM : 1], kb[KV], qb[KV], vj;
            };
            auto load_tok = [&](int tl) {
                Tok x;
                const float *qrow = Qs + tl * D + rb + (lane & 15);
                const float *krow = Ks + tl * D + rb + (lane & 15);
#pragma unroll
                for (int m = 0; m < KV; ++m) {
                    if constexpr (!kMU) x.kb[m] = krow[16 * m];
                    x.qb[m] = qrow[16 * m];
                }
                if constexpr (kMU) {
#pragma unroll
                    for (int m = 0; m < NM; ++m) x.ka[m] = Ks[tl * D + rb + 4 * m + (lane & 3)];
                }
                x.vj = Vs[tl * D + col];
                return x;
            };
            // one token: rs holds S'_(t-1) on entry; the update goes to ws (the other copy) with the
            // matrix cores, or to rs itself with DPP FMAs
            auto step = [&](int tl, const Tok &x, f32x4 (&rs)[NM], f32x4 (&ws)[NM]) {
                if (KIND != kMaskLit && (rmask & (1u << tl))) {
                    const float mu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, multv), tl));
#pragma unroll
                    for (int m = 0; m < NM; ++m) rs[m] *= mu;
                }
                float y0, y1;
                if constexpr (kMU) {
#pragma unroll
                    for (int m = 0; m < NM; ++m) {
                        ws[m] = __builtin_amdgcn_mfma_f32_4x4x1f32(x.ka[m], x.vj, rs[m], 0, 0, 0);
                        // issue this token's product before its dot product (an empty asm statement
                        // taking its result keeps the compiler from moving it below the asm dot): the
                        // dot then reads rs, written by the product issued a whole token earlier, far
                        // more than the 4 wait states a vector read of that result needs
                        asm volatile("" ::"v"(ws[m]));
                    }
                    float sr[RW];
#pragma unroll
                    for (int i = 0; i < RW; ++i) sr[i] = rs[i / 4][i % 4];
                    dpp_dot_first<RB>(y0, y1, x.qb[0], sr);
#pragma unroll
                    for (int m = 1; m < KV; ++m) dpp_dot<RB>(y0, y1, x.qb[m], sr + RB * m);
                } else {
                    float sr[RW];
#pragma unroll
                    for (int i = 0; i < RW; ++i) sr[i] = rs[i / 4][i % 4];
                    dpp_update<RB>(sr, x.kb[0], x.vj);
                    dpp_dot_first<RB>(y0, y1, x.qb[0], sr);
#pragma unroll
                    for (int m = 1; m < KV; ++m) {
                        dpp_update<RB>(sr + RB * m, x.kb[m], x.vj);
                        dpp_dot<RB>(y0, y1, x.qb[m], sr + RB * m);
                    }
#pragma unroll
                    for (int i = 0; i < RW; ++i) rs[i / 4][i % 4] = sr[i];
                }
                yp[tl * NP * CW] = y0 + y1;
            };
            // every token of the block, past the end included: those are staged with k = q = 0 and
            // multiplier 1, so they leave the state as it is, and their partials are never read
            // a token's operands are loaded one token ahead (measured: deeper is slower)
            constexpr int kAhead = 1;
            Tok tk[kAhead + 1];
#pragma unroll
            for (int u = 0; u < kAhead; ++u) tk[u] = load_tok(u);
#pragma unroll
            for (int tl = 0; tl < kT; ++tl) {
                if (tl + kAhead < kT) tk[(tl + kAhead) % (kAhead + 1)] = load_tok(tl + kAhead);
                const Tok &cur = tk[tl % (kAhead + 1)];
                if (!kMU || (tl & 1) == 0)
                    step(tl, cur, Sa, Sb);
                else
                    step(tl, cur, Sb, Sa);
            }
            // kT is even: after the block the state is in Sa again
            if constexpr (KIND != kMaskLit) lam_end = ysc[nsteps - 1];
        }
        __syncthreads();
    }
}

template <int D, int CW, int NR>
constexpr size_t rnn_lds() {
    using Sh = RnnShape<D, CW, NR>;
    const size_t dirf = 2 * ((size_t)kT * D + 16) + (size_t)kT * D + 4 * kT;
    return (2 * dirf + 2 * (size_t)kT * Sh::NP * CW + 2 * (size_t)kT * Sh::NP) * 4;
}

// Work splits (column group width, waves per direction) per head dimension, from the fewest waves
// (least per-token overhead) to the most; the first giving at least 1.5 waves per SIMD is used, or 3
// per SIMD for splits with 32 state rows per lane (their register count allows no more than 3).
// Measured at d = 64: B64 H12 L197 runs best on 64 x 2, B32 H16 L512 and B64 H3 L197 on 64 x 4,
// B8 H12 L4097 on 32 x 4.
struct RnnSplit {
    int cw, nr;
};
constexpr RnnSplit kSplit16[] = {{16, 1}, {16, 2}};
constexpr RnnSplit kSplit32[] = {{32, 2}, {32, 4}, {16, 4}};
constexpr RnnSplit kSplit64[] = {{64, 2}, {64, 4}, {32, 4}, {16, 4}};
constexpr RnnSplit kSplit128[] = {{64, 4}, {32, 4}, {16, 4}};

// The causal variant (one recurrence) takes the same split: measured faster than counting its waves
// alone (which picks narrower groups, e.g. a grid past one workgroup per CU for B8 H12 L4097, where the
// pipelined variant no longer applies: 922 us against 505 us).
template <int D>
int rnn_split(int B, int H) {
    const RnnSplit *sp = D == 16 ? kSplit16 : D == 32 ? kSplit32 : D == 64 ? kSplit64 : kSplit128;
    const int n = D == 16 ? 2 : D == 32 ? 3 : D == 64 ? 4 : 3;
    for (int i = 0; i < n; ++i) {
        const int rw = D * sp[i].cw / (64 * sp[i].nr);
        if ((long)B * H * (D / sp[i].cw) * 2 * sp[i].nr >= (rw >= 32 ? 3072 : 1536)) return i;
    }
    return n - 1;
}

template <int D, int KIND, int CW, int NR, bool BF16>
hipError_t launch_split(const AttnArgs &a, hipStream_t stream) {
    RnnParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.ll = a.log_lambda;
    p.eps = a.eps;
    p.H = a.H;
    p.L = a.L;
    p.y = a.y;
    p.out_bf16 = a.out_bf16 ? 1 : 0;
    p.den_out = a.den_out;
    p.park = reinterpret_cast<float *>(a.workspace);
    p.causal = a.causal ? 1 : 0;
    const unsigned grid = (unsigned)(a.B * a.H * (D / CW));
    constexpr size_t plds = rnn_pipe_lds<D, CW, NR>();
    if constexpr (plds <= kLdsPerWorkgroup) {
        if (grid <= 256) {   // one workgroup per CU: the pipelined variant
            if (plds > 64 * 1024)
                (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&birnn_pipe_kernel<D, KIND, CW, NR, BF16>),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)plds);
            hipLaunchKernelGGL((birnn_pipe_kernel<D, KIND, CW, NR, BF16>), dim3(grid), dim3((2 * NR + kHelp) * 64), plds,
                               stream, p);
            return hipGetLastError();
        }
    }
    constexpr size_t lds = rnn_lds<D, CW, NR>();
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&birnn_kernel<D, KIND, CW, NR, BF16>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    // causal: the forward waves alone (threads of the backward direction would have nothing to do)
    hipLaunchKernelGGL((birnn_kernel<D, KIND, CW, NR, BF16>), dim3(grid), dim3((a.causal ? 1 : 2) * NR * 64), lds,
                       stream, p);
    return hipGetLastError();
}

template <int D, int KIND, bool BF16>
hipError_t launch_t(const AttnArgs &a, hipStream_t stream) {
    const int i = rnn_split<D>(a.B, a.H);
    if constexpr (D == 16) {
        return i == 0 ? launch_split<16, KIND, 16, 1, BF16>(a, stream) : launch_split<16, KIND, 16, 2, BF16>(a, stream);
    } else if constexpr (D == 32) {
        if (i == 0) return launch_split<32, KIND, 32, 2, BF16>(a, stream);
        if (i == 1) return launch_split<32, KIND, 32, 4, BF16>(a, stream);
        return launch_split<32, KIND, 16, 4, BF16>(a, stream);
    } else if constexpr (D == 64) {
        if (i == 0) return launch_split<64, KIND, 64, 2, BF16>(a, stream);
        if (i == 1) return launch_split<64, KIND, 64, 4, BF16>(a, stream);
        if (i == 2) return launch_split<64, KIND, 32, 4, BF16>(a, stream);
        return launch_split<64, KIND, 16, 4, BF16>(a, stream);
    } else {
        if (i == 0) return launch_split<128, KIND, 64, 4, BF16>(a, stream);
        if (i == 1) return launch_split<128, KIND, 32, 4, BF16>(a, stream);
        return launch_split<128, KIND, 16, 4, BF16>(a, stream);
    }
}

template <int D, bool BF16>
hipError_t dispatch_kind(const AttnArgs &a, hipStream_t stream) {
    switch (a.kind) {
    case kMaskLit: return launch_t<D, kMaskLit, BF16>(a, stream);
    case kMaskD: return launch_t<D, kMaskD, BF16>(a, stream);
    default: return launch_t<D, kMaskS, BF16>(a, stream);
    }
}

template <bool BF16>
hipError_t dispatch_d(const AttnArgs &a, hipStream_t stream) {
    switch (a.d) {
    case 16: return dispatch_kind<16, BF16>(a, stream);
    case 32: return dispatch_kind<32, BF16>(a, stream);
    case 64: return dispatch_kind<64, BF16>(a, stream);
    default: return dispatch_kind<128, BF16>(a, stream);
    }
}

template <int D>
size_t workspace_t(const AttnArgs &a) {
    if (a.causal) return 0;   // nothing parked
    const RnnSplit sp =
        (D == 16 ? kSplit16 : D == 32 ? kSplit32 : D == 64 ? kSplit64 : kSplit128)[rnn_split<D>(a.B, a.H)];
    return (size_t)a.B * a.H * (D / sp.cw) * a.L * (sp.cw + 1) * 4;
}

}  // namespace

Plan plan_birnn(const AttnArgs &a) {
    Plan p;
    p.ok = rnn_lds<128, 64, 4>() <= kLdsPerWorkgroup;
    switch (a.d) {
    case 16: p.workspace = workspace_t<16>(a); break;
    case 32: p.workspace = workspace_t<32>(a); break;
    case 64: p.workspace = workspace_t<64>(a); break;
    default: p.workspace = workspace_t<128>(a); break;
    }
    return p;
}

hipError_t launch_birnn(const AttnArgs &a, hipStream_t stream) {
    return a.in_bf16 ? dispatch_d<true>(a, stream) : dispatch_d<false>(a, stream);
}

}  // namespace lion
