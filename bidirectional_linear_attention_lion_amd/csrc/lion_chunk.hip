// lion_chunk.hip -- chunkwise form of LION bidirectional masked linear attention.
//
// Chunking is how the pages parallelise LION inference when memory is short ("LION: A
// bidirectional framework that trains like a Transformer and infers like an RNN", reply
// "4: Practicality of Recurrent Inference"; blog "LION Part IV - Results", "LION Chunk").  The
// pages print no chunk equations; the ones used here follow from the mask M_ij = exp(-|A_i - A_j|)
// (A = prefix sums of log(lambda)).  For chunk c = tokens s_c .. e_c and [v, 1] the value row with
// the row-sum column appended:
//   F_c = exp(A_{e_c} - A_{e_{c-1}}) F_{c-1} + sum_{j in c} exp(A_{e_c} - A_j) phi(k_j) [v_j, 1]^T
//   G_c = exp(A_{e_c} - A_{e_{c-1}}) G_{c+1} + sum_{j in c} exp(A_j - A_{e_{c-1}}) phi(k_j) [v_j, 1]^T
//   out_i = sum_{j in c} M_ij (phi(q_i).phi(k_j)) [v_j, 1]
//           + exp(A_i - A_{e_{c-1}}) phi(q_i)^T F_{c-1} + exp(A_{e_c} - A_i) phi(q_i)^T G_{c+1}
//   y_i = out_i[:d] / (out_i[d] + eps)
// Every exponent is <= 0.
//
// One workgroup (8 waves) per (batch, head) sweeps the chunks twice, keeping the d x (d+1)
// states on chip:
//   backward pass, c = n-1 .. 1: park G_{c+1} (bf16 d x d plus the fp32 row-sum column), then fold
//     chunk c into G;
//   forward pass,  c = 0 .. n-1: intra-chunk masked attention on matrix cores (as in the full form),
//     plus F_{c-1} and the parked G_{c+1} applied to the decayed queries, then fold chunk c into F.
// Chunk states live in fp32 matrix-core accumulators spread over the 8 waves.  The fold multiplies
// the weighted values (w_j v_j)^T by phi(K); the row-sum column rides along as two extra rows of
// that operand holding w_j split into a bf16 high part and the bf16 rounding of the remainder, so
// the row-sum state -- whose rounding error a nearly cancelling denominator amplifies -- keeps
// about 2^-17 relative accuracy although the tiles are bf16.  Parked backward states stay in LDS
// when they fit, else in the caller's workspace.
#include <type_traits>

#include "lion_device.h"
#include "lion_internal.h"
#include "lion_mask.h"

namespace lion {
namespace {

constexpr int kKB = 32;                // tokens per staged sub-block
constexpr int kNW = 8;                 // waves per workgroup
constexpr int kNT = kNW * 64;
constexpr int kGLdsMax = 64 * 1024;    // parked backward states kept in LDS up to this many bytes

struct ChunkParams {
    const void *q, *k, *v;
    const float *ll;
    float eps;
    int H, L, C;
    void *y;
    int out_bf16;
    float *den_out;
    unsigned char *ws;   // parked states in global memory, or null when they live in LDS
};

template <int D, bool BF16>
struct ChunkCfg {
    using T = std::conditional_t<BF16, __bf16, float>;
    static constexpr int VEC = 16 / (int)sizeof(T);
    static constexpr int CPK = D / VEC;
    static constexpr int CPL = D / 4;
    static constexpr int NS = BF16 ? (CPL + 7) / 8 : CPL;
    static constexpr int KROW = D + (BF16 ? 8 : 4);      // row-major phi(K) sub-block pitch
    static constexpr int TROW = kKB + (BF16 ? 8 : 4);    // transposed (token-contiguous) pitch
    static constexpr int VR = D + 16;                     // weighted V^T rows: D values, w_hi, w_lo, zeros
    static constexpr int SROW = D + (BF16 ? 8 : 4);      // state copy pitch (rows = value channel)
    static constexpr int NCT = D / 16 + 1;                // state tiles along the value(+1) axis
    static constexpr int NDT = D / 16;                    // state tiles along the key-channel axis
    static constexpr int MAXT = (NCT * NDT + kNW - 1) / kNW;   // state tiles per wave
    static constexpr int QT = D == 128 ? 1 : 2;           // query tiles per wave: C <= 16 * kNW * QT
    using QFrag = std::conditional_t<BF16, bf16x8, float>;
    static constexpr size_t GSLOT = (size_t)D * D * sizeof(T) + (size_t)D * 4;   // one parked state
};

template <int D, bool BF16>
__host__ __device__ size_t lds_fixed_bytes(int L) {
    using C = ChunkCfg<D, BF16>;
    using T = typename C::T;
    const int Lpad = ((L + kKB - 1) / kKB) * kKB;
    size_t b = (size_t)Lpad * 4 + kNT * 8;                 // exponent table + scan scratch
    b += (size_t)kKB * C::KROW * sizeof(T);                // Ks
    b += (size_t)D * C::TROW * sizeof(T);                  // Vt (plain, for P V)
    b += (size_t)C::VR * C::TROW * sizeof(T);              // Vw (weighted, plus the two weight rows)
    b += (size_t)D * C::TROW * sizeof(T);                  // Kt
    b += (size_t)D * C::SROW * sizeof(T) + (size_t)D * 4;   // current F copy and its row-sum column
    return (b + 15) & ~(size_t)15;
}

// Parked backward states go to LDS when they are small and fit beside the fixed carve-up.
template <int D, bool BF16>
bool park_in_lds(int L, int Cc) {
    const size_t park = (size_t)((L + Cc - 1) / Cc) * ChunkCfg<D, BF16>::GSLOT;
    return park <= (size_t)kGLdsMax && lds_fixed_bytes<D, BF16>(L) + park <= kLdsPerWorkgroup;
}

template <int D, int KIND, bool BF16>
__global__ void __launch_bounds__(kNT) chunk_kernel(ChunkParams p) {
    using Cf = ChunkCfg<D, BF16>;
    using T = typename Cf::T;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int L = p.L, Cc = p.C;
    const int n = (L + Cc - 1) / Cc;
    const int Lpad = ((L + kKB - 1) / kKB) * kKB;
    const int bh = blockIdx.x;
    const size_t base = (size_t)bh * L;

    // ---- LDS carve-up ---------------------------------------------------------------------------------
    unsigned char *sp = smem;
    float *E = reinterpret_cast<float *>(sp);
    sp += (size_t)Lpad * 4;
    double *scan_sh = reinterpret_cast<double *>(sp);
    sp += kNT * 8;
    T *Ks = reinterpret_cast<T *>(sp);
    sp += (size_t)kKB * Cf::KROW * sizeof(T);
    T *Vt = reinterpret_cast<T *>(sp);
    sp += (size_t)D * Cf::TROW * sizeof(T);
    T *Vw = reinterpret_cast<T *>(sp);
    sp += (size_t)Cf::VR * Cf::TROW * sizeof(T);
    T *Kt = reinterpret_cast<T *>(sp);
    sp += (size_t)D * Cf::TROW * sizeof(T);
    T *Fs = reinterpret_cast<T *>(sp);
    sp += (size_t)D * Cf::SROW * sizeof(T);
    float *Fz = reinterpret_cast<float *>(sp);
    sp = smem + lds_fixed_bytes<D, BF16>(L);
    unsigned char *park = p.ws ? p.ws + (size_t)bh * n * Cf::GSLOT : sp;

    const T *qg = reinterpret_cast<const T *>(p.q) + base * D;
    const T *kg = reinterpret_cast<const T *>(p.k) + base * D;
    const T *vg = reinterpret_cast<const T *>(p.v) + base * D;

    if constexpr (KIND != kMaskLit) build_exponents<KIND>(E, scan_sh, p.ll, bh, p.H, L, Lpad, 0, tid, kNT);
    auto Ex = [&](int t) -> float {
        if constexpr (KIND == kMaskLit) return 0.f;
        else return E[t];
    };

    f32x4 st[Cf::MAXT];

    // Stage, for the tokens [j0, j0 + 32) that lie in [cs, ce]: phi(K) row-major (if attend),
    // phi(K)^T, V^T, and the weighted (w_j v_j)^T with the weight split w_hi + w_lo below it.
    auto stage = [&](int j0, int cs, int ce, bool attend, bool fwd_weights) {
        const int total = kKB * Cf::CPK;
        const float eref = fwd_weights ? Ex(ce) : Ex(cs > 0 ? cs - 1 : 0);
        for (int c0 = 0; c0 < total; c0 += kNT) {
            const int c = c0 + tid;
            const bool active = c < total;
            const int kl = c / Cf::CPK, cc = (c % Cf::CPK) * Cf::VEC;
            const int j = j0 + kl;
            const bool valid = active && j >= cs && j <= ce;
            float xk[Cf::VEC], xv[Cf::VEC];
            if (valid) {
                const T *ks = kg + (size_t)j * D + cc;
                const T *vs = vg + (size_t)j * D + cc;
#pragma unroll
                for (int e = 0; e < Cf::VEC; ++e) {
                    xk[e] = (float)ks[e];
                    xv[e] = (float)vs[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < Cf::VEC; ++e) xk[e] = xv[e] = 0.f;
            }
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < Cf::VEC; ++e) {
                xk[e] = phi_pre<KIND>(xk[e]);
                ss += xk[e] * xk[e];
            }
            if constexpr (KIND == kMaskS) {
                const float sc = inv_norm(group_sum<Cf::CPK>(ss));
#pragma unroll
                for (int e = 0; e < Cf::VEC; ++e) xk[e] *= sc;
            }
            // fold weight: forward exp(A_{e_c} - A_j), backward exp(A_j - A_{e_{c-1}}); both <= 1
            float w = 1.f;
            if constexpr (KIND != kMaskLit) {
                if (valid) w = fast_exp2(fwd_weights ? eref - Ex(j) : Ex(j) - eref);
            }
            if (active) {
                if (!valid) w = 0.f;
#pragma unroll
                for (int e = 0; e < Cf::VEC; ++e) {
                    const float kv = valid ? xk[e] : 0.f;
                    if (attend) {
                        Ks[kl * Cf::KROW + cc + e] = (T)kv;
                        Vt[(cc + e) * Cf::TROW + kl] = (T)xv[e];
                    }
                    Kt[(cc + e) * Cf::TROW + kl] = (T)kv;
                    Vw[(cc + e) * Cf::TROW + kl] = (T)(w * xv[e]);
                }
                if (cc == 0) {
                    const T whi = (T)w;
                    Vw[D * Cf::TROW + kl] = whi;
                    Vw[(D + 1) * Cf::TROW + kl] = (T)(w - (float)whi);
#pragma unroll
                    for (int z = 2; z < 16; ++z) Vw[(D + z) * Cf::TROW + kl] = (T)0.f;
                }
            }
        }
    };

    // st += Vw (sub-block) x phi(K) (sub-block) for this wave's state tiles
    auto fold = [&]() {
#pragma unroll
        for (int u = 0; u < Cf::MAXT; ++u) {
            const int tt = wave + kNW * u;
            if (tt >= Cf::NCT * Cf::NDT) break;
            const int ct = tt / Cf::NDT, nt = tt % Cf::NDT;
            const T *va = Vw + (16 * ct + r) * Cf::TROW + 4 * g;
            const T *kb = Kt + (16 * nt + r) * Cf::TROW + 4 * g;
            if constexpr (BF16) {
                bf16x8 a, b;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[e] = va[e];
                    a[4 + e] = va[16 + e];
                    b[e] = kb[e];
                    b[4 + e] = kb[16 + e];
                }
                st[u] = mfma_bf16(a, b, st[u]);
            } else {
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                    for (int e = 0; e < 4; ++e) st[u] = mfma_f32(va[16 * t2 + e], kb[16 * t2 + e], st[u]);
            }
        }
    };

    auto scale_state = [&](float a) {
#pragma unroll
        for (int u = 0; u < Cf::MAXT; ++u) st[u] *= a;
    };

    // write this wave's state tiles into a state copy (rows = value channel, cols = key channel)
    auto write_state = [&](T *dst, float *dz) {
#pragma unroll
        for (int u = 0; u < Cf::MAXT; ++u) {
            const int tt = wave + kNW * u;
            if (tt >= Cf::NCT * Cf::NDT) break;
            const int ct = tt / Cf::NDT, nt = tt % Cf::NDT;
            if (ct < D / 16) {
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(16 * ct + 4 * g + e) * Cf::SROW + 16 * nt + r] = (T)st[u][e];
            } else if (g == 0) {
                dz[16 * nt + r] = st[u][0] + st[u][1];   // row-sum state = w_hi part + w_lo part
            }
        }
    };

    auto zero_state = [&]() {
#pragma unroll
        for (int u = 0; u < Cf::MAXT; ++u) st[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // ================= backward pass: park G_{c+1} for c = n-1 .. 0, fold chunk c for c >= 1 ==========
    zero_state();
    for (int c = n - 1; c >= 0; --c) {
        const int cs = c * Cc, ce = min(cs + Cc, L) - 1;
        // park G_{c+1} (zero for the last chunk)
        {
            T *gs = reinterpret_cast<T *>(park + (size_t)c * Cf::GSLOT);
            float *gz = reinterpret_cast<float *>(park + (size_t)c * Cf::GSLOT + (size_t)D * D * sizeof(T));
#pragma unroll
            for (int u = 0; u < Cf::MAXT; ++u) {
                const int tt = wave + kNW * u;
                if (tt >= Cf::NCT * Cf::NDT) break;
                const int ct = tt / Cf::NDT, nt = tt % Cf::NDT;
                if (ct < D / 16) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) gs[(16 * ct + 4 * g + e) * D + 16 * nt + r] = (T)st[u][e];
                } else if (g == 0) {
                    gz[16 * nt + r] = st[u][0] + st[u][1];
                }
            }
        }
        if (c == 0) break;
        // G_c = exp(A_{e_c} - A_{e_{c-1}}) G_{c+1} + sum_j exp(A_j - A_{e_{c-1}}) k_j [v_j, 1]^T
        if constexpr (KIND != kMaskLit) scale_state(fast_exp2(Ex(ce) - Ex(cs - 1)));
        for (int j0 = cs - (cs % kKB); j0 <= ce; j0 += kKB) {
            __syncthreads();
            stage(j0, cs, ce, false, false);
            __syncthreads();
            fold();
        }
    }
    if (p.ws) __threadfence();
    __syncthreads();

    // ================= forward pass ======================================================================
    const int tiles_per_chunk = (Cc + 15) / 16;
    zero_state();
    for (int c = 0; c < n; ++c) {
        const int cs = c * Cc, ce = min(cs + Cc, L) - 1;
        const bool has_f = c > 0, has_g = c < n - 1;
        // current F_{c-1} (this wave's tiles -> LDS copy); G_{c+1} is read from its parking slot
        __syncthreads();
        if (has_f) write_state(Fs, Fz);
        const T *Gs = reinterpret_cast<const T *>(park + (size_t)c * Cf::GSLOT);
        const float *Gz = reinterpret_cast<const float *>(park + (size_t)c * Cf::GSLOT + (size_t)D * D * sizeof(T));
        // fold weights for F_c; the state registers are rescaled now, the LDS copy keeps F_{c-1}
        if (has_f && KIND != kMaskLit) scale_state(fast_exp2(Ex(ce) - Ex(cs - 1)));

        // ---- query fragments of this wave's tiles in chunk c ----------------------------------------
        typename Cf::QFrag qf[Cf::QT][Cf::NS];
        float Ei[Cf::QT];
        int ntl = 0;
#pragma unroll
        for (int qt = 0; qt < Cf::QT; ++qt) {
            const int tl = wave + kNW * qt;
            const int i = cs + tl * 16 + r;
            const bool tile_ok = tl < tiles_per_chunk;
            if (tile_ok) ntl = qt + 1;
            const bool ok = tile_ok && i <= ce;
            float xq[Cf::CPL];
            float ssq = 0.f;
#pragma unroll
            for (int cc = 0; cc < Cf::CPL; ++cc) {
                float x = ok ? (float)qg[(size_t)i * D + g * Cf::CPL + cc] : 0.f;
                x = phi_pre<KIND>(x);
                xq[cc] = x;
                ssq += x * x;
            }
            if constexpr (KIND == kMaskS) {
                ssq += __shfl_xor(ssq, 16, 64);
                ssq += __shfl_xor(ssq, 32, 64);
                const float sc = inv_norm(ssq);
#pragma unroll
                for (int cc = 0; cc < Cf::CPL; ++cc) xq[cc] *= sc;
            }
            if (!ok) {
#pragma unroll
                for (int cc = 0; cc < Cf::CPL; ++cc) xq[cc] = 0.f;
            }
            if constexpr (BF16) {
#pragma unroll
                for (int s = 0; s < Cf::NS; ++s) {
                    bf16x8 f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] = (8 * s + e < Cf::CPL) ? f2bf(xq[8 * s + e]) : f2bf(0.f);
                    qf[qt][s] = f;
                }
            } else {
#pragma unroll
                for (int s = 0; s < Cf::NS; ++s) qf[qt][s] = xq[s];
            }
            Ei[qt] = Ex(ok ? i : cs);
        }

        f32x4 acc[Cf::QT][D / 16];
        float den[Cf::QT];
#pragma unroll
        for (int qt = 0; qt < Cf::QT; ++qt) {
            den[qt] = 0.f;
#pragma unroll
            for (int ct = 0; ct < D / 16; ++ct) acc[qt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        // ---- intra-chunk attention and the fold of chunk c into F -------------------------------------
        for (int j0 = cs - (cs % kKB); j0 <= ce; j0 += kKB) {
            __syncthreads();
            stage(j0, cs, ce, true, true);
            __syncthreads();
            if (c < n - 1) fold();
            if (ntl == 0) continue;
            typename Cf::QFrag kf[2][Cf::NS];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const T *src = Ks + (16 * t + r) * Cf::KROW + g * Cf::CPL;
                if constexpr (BF16) {
#pragma unroll
                    for (int s = 0; s < Cf::NS; ++s) {
                        bf16x8 f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) f[e] = (8 * s + e < Cf::CPL) ? src[8 * s + e] : f2bf(0.f);
                        kf[t][s] = f;
                    }
                } else {
#pragma unroll
                    for (int s = 0; s < Cf::NS; ++s) kf[t][s] = src[s];
                }
            }
            float Ej[2][4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = min(j0 + 16 * t + 4 * g + e, L - 1);
                    Ej[t][e] = Ex(j);
                }
#pragma unroll
            for (int qt = 0; qt < Cf::QT; ++qt) {
                if (qt >= ntl) break;
                f32x4 sa[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    sa[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < Cf::NS; ++s) {
                        if constexpr (BF16)
                            sa[t] = mfma_bf16(kf[t][s], qf[qt][s], sa[t]);
                        else
                            sa[t] = mfma_f32(kf[t][s], qf[qt][s], sa[t]);
                    }
                }
                float pv[2][4];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float m = 1.f;
                        if constexpr (KIND != kMaskLit) m = fast_exp2(-__builtin_fabsf(Ei[qt] - Ej[t][e]));
                        const float pe = sa[t][e] * m;
                        den[qt] += pe;
                        pv[t][e] = pe;
                    }
                if constexpr (BF16) {
                    bf16x8 pf;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pf[e] = f2bf(pv[0][e]);
                        pf[4 + e] = f2bf(pv[1][e]);
                    }
#pragma unroll
                    for (int ct = 0; ct < D / 16; ++ct) {
                        const T *vs = Vt + (16 * ct + r) * Cf::TROW + 4 * g;
                        bf16x8 vf;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            vf[e] = vs[e];
                            vf[4 + e] = vs[16 + e];
                        }
                        acc[qt][ct] = mfma_bf16(vf, pf, acc[qt][ct]);
                    }
                } else {
#pragma unroll
                    for (int ct = 0; ct < D / 16; ++ct) {
                        const T *vs = Vt + (16 * ct + r) * Cf::TROW + 4 * g;
#pragma unroll
                        for (int t = 0; t < 2; ++t)
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[qt][ct] = mfma_f32(vs[16 * t + e], pv[t][e], acc[qt][ct]);
                    }
                }
            }
        }

        // ---- inter-chunk terms: F_{c-1} and G_{c+1} applied to the decayed queries ---------------------
        if (ntl > 0 && (has_f || has_g)) {
#pragma unroll
            for (int which = 0; which < 2; ++which) {
                const bool use = which == 0 ? has_f : has_g;
                if (!use) continue;
                const T *Ss = which == 0 ? Fs : Gs;
                const float *Sz = which == 0 ? Fz : Gz;
                const int pitch = which == 0 ? Cf::SROW : D;
#pragma unroll
                for (int qt = 0; qt < Cf::QT; ++qt) {
                    if (qt >= ntl) break;
                    // decay from the chunk boundary to the query: exp(A_i - A_{e_{c-1}}) or exp(A_{e_c} - A_i)
                    float dq = 1.f;
                    if constexpr (KIND != kMaskLit)
                        dq = which == 0 ? fast_exp2(Ei[qt] - Ex(cs - 1)) : fast_exp2(Ex(ce) - Ei[qt]);
                    // the same rounded phi(q) the intra-chunk scores use
                    float zdot = 0.f;
                    typename Cf::QFrag qd[Cf::NS];
                    if constexpr (BF16) {
#pragma unroll
                        for (int s = 0; s < Cf::NS; ++s) {
                            bf16x8 f;
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const float x = (8 * s + e < Cf::CPL) ? (float)qf[qt][s][e] : 0.f;
                                if (8 * s + e < Cf::CPL) zdot += x * Sz[g * Cf::CPL + 8 * s + e];
                                f[e] = f2bf(dq * x);
                            }
                            qd[s] = f;
                        }
                    } else {
#pragma unroll
                        for (int s = 0; s < Cf::NS; ++s) {
                            zdot += qf[qt][s] * Sz[g * Cf::CPL + s];
                            qd[s] = dq * qf[qt][s];
                        }
                    }
                    den[qt] += dq * zdot;
#pragma unroll
                    for (int ct = 0; ct < D / 16; ++ct) {
                        const T *src = Ss + (16 * ct + r) * pitch + g * Cf::CPL;
#pragma unroll
                        for (int s = 0; s < Cf::NS; ++s) {
                            if constexpr (BF16) {
                                bf16x8 a;
#pragma unroll
                                for (int e = 0; e < 8; ++e) a[e] = (8 * s + e < Cf::CPL) ? src[8 * s + e] : f2bf(0.f);
                                acc[qt][ct] = mfma_bf16(a, qd[s], acc[qt][ct]);
                            } else {
                                acc[qt][ct] = mfma_f32(src[s], qd[s], acc[qt][ct]);
                            }
                        }
                    }
                }
            }
        }

        // ---- epilogue ----------------------------------------------------------------------------------
#pragma unroll
        for (int qt = 0; qt < Cf::QT; ++qt) {
            if (qt >= ntl) break;
            float dsum = den[qt];
            dsum += __shfl_xor(dsum, 16, 64);
            dsum += __shfl_xor(dsum, 32, 64);
            const float div = dsum + p.eps;
            const int i = cs + (wave + kNW * qt) * 16 + r;
            if (i <= ce) {
                const float inv = 1.f / div;
                const size_t row = base + i;
                if (p.out_bf16) {
                    __bf16 *yo = reinterpret_cast<__bf16 *>(p.y) + row * D;
#pragma unroll
                    for (int ct = 0; ct < D / 16; ++ct) {
                        bf16x4 o;
#pragma unroll
                        for (int e = 0; e < 4; ++e) o[e] = f2bf(acc[qt][ct][e] * inv);
                        *reinterpret_cast<bf16x4 *>(yo + 16 * ct + 4 * g) = o;
                    }
                } else {
                    float *yo = reinterpret_cast<float *>(p.y) + row * D;
#pragma unroll
                    for (int ct = 0; ct < D / 16; ++ct) {
                        f32x4 o;
#pragma unroll
                        for (int e = 0; e < 4; ++e) o[e] = acc[qt][ct][e] * inv;
                        *reinterpret_cast<f32x4 *>(yo + 16 * ct + 4 * g) = o;
                    }
                }
                if (p.den_out && g == 0) p.den_out[row] = div;
            }
        }
    }
}

template <int D, int KIND, bool BF16>
hipError_t launch_t(const AttnArgs &a, hipStream_t stream) {
    ChunkParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.ll = a.log_lambda;
    p.eps = a.eps;
    p.H = a.H;
    p.L = a.L;
    p.C = a.C;
    p.y = a.y;
    p.out_bf16 = a.out_bf16 ? 1 : 0;
    p.den_out = a.den_out;
    const bool in_lds = park_in_lds<D, BF16>(a.L, a.C);
    p.ws = in_lds ? nullptr : reinterpret_cast<unsigned char *>(a.workspace);
    size_t lds = lds_fixed_bytes<D, BF16>(a.L);
    if (in_lds) lds += (size_t)((a.L + a.C - 1) / a.C) * ChunkCfg<D, BF16>::GSLOT;
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_kernel<D, KIND, BF16>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((chunk_kernel<D, KIND, BF16>), dim3(a.B * a.H), dim3(kNT), lds, stream, p);
    return hipGetLastError();
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

template <int D, bool BF16>
Plan plan_t(const AttnArgs &a) {
    Plan p;
    p.ok = lds_fixed_bytes<D, BF16>(a.L) <= kLdsPerWorkgroup;
    p.workspace = park_in_lds<D, BF16>(a.L, a.C)
                      ? 0
                      : (size_t)a.B * a.H * ((a.L + a.C - 1) / a.C) * ChunkCfg<D, BF16>::GSLOT;
    return p;
}

}  // namespace

Plan plan_chunk(const AttnArgs &a) {
    switch (a.d) {
    case 16: return a.in_bf16 ? plan_t<16, true>(a) : plan_t<16, false>(a);
    case 32: return a.in_bf16 ? plan_t<32, true>(a) : plan_t<32, false>(a);
    case 64: return a.in_bf16 ? plan_t<64, true>(a) : plan_t<64, false>(a);
    default: return a.in_bf16 ? plan_t<128, true>(a) : plan_t<128, false>(a);
    }
}

hipError_t launch_chunk(const AttnArgs &a, hipStream_t stream) {
    return a.in_bf16 ? dispatch_d<true>(a, stream) : dispatch_d<false>(a, stream);
}

}  // namespace lion
