// lion_full.hip -- full (attention) form of LION bidirectional masked linear attention.
//
// Y = SCALE(phi(Q) phi(K)^T (.) M) V, the form LION trains with ("LION: A bidirectional framework
// that trains like a Transformer and infers like an RNN", reply "Concern 1", Theorem 3.3 Eq. 25).
// The L x L score matrix is never materialised: each workgroup owns a run of 16-row query tiles
// of one (batch, head) and streams the keys in blocks of 32 through LDS.  Per block and query
// tile a wave forms S^T = phi(K) phi(Q)^T with matrix-core tiles, applies the mask in registers,
// accumulates the fp32 row sums, and feeds the masked scores back as the B operand of
// O^T = V^T P^T without leaving registers.
//
// Mask: M_ij = exp(-|A_i - A_j|) with A the prefix sums of log(lambda) (the cumsum mask of the
// pages' "P3: LION-S uses cumsum" reply), kept as a per-position exponent table E (base 2) in LDS:
//   LIT: no mask;  D: E_t = (t - t_ref) log2(lambda_h);  S: E_t = (A_t - A_ref) log2(e) from an fp64
//   prefix scan, so no fp32 cancellation builds up along long sequences.
// Only non-positive exponents are exponentiated (exp2(-|E_i - E_j|)).
#include <type_traits>

#include "lion_device.h"
#include "lion_internal.h"
#include "lion_mask.h"

namespace lion {
namespace {

constexpr int kKB = 32;  // keys per staged block (two 16-key halves of S^T)

struct FullParams {
    const void *q, *k, *v;
    const float *ll;
    float eps;
    int H, L;
    void *y;
    int out_bf16;
    float *den_out;
    int nsb;           // workgroups per (batch, head)
    int tiles_per_wg;  // 16-row query tiles per workgroup
    int nblocks;       // grid size
};

template <int D, bool BF16>
struct FullCfg {
    using T = std::conditional_t<BF16, __bf16, float>;
    static constexpr int VEC = 16 / (int)sizeof(T);        // elements per 16-byte chunk
    static constexpr int CPK = D / VEC;                     // chunks per key row
    static constexpr int CPL = D / 4;                       // channels owned by each lane group
    static constexpr int NS = BF16 ? (CPL + 7) / 8 : CPL;   // score MFMA steps
    static constexpr int KROW = D + (BF16 ? 8 : 4);         // K tile row pitch (elements)
    static constexpr int VROW = kKB + (BF16 ? 8 : 4);       // V^T tile row pitch (elements)
    using QFrag = std::conditional_t<BF16, bf16x8, float>;
};

template <int D, int KIND, int QT, bool BF16>
__global__ void __launch_bounds__(512) full_kernel(FullParams p) {
    using C = FullCfg<D, BF16>;
    using T = typename C::T;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int L = p.L;
    const int nkb = (L + kKB - 1) / kKB;
    const int Lpad = nkb * kKB;
    const int ntiles = (L + 15) / 16;

    const int tile = xcd_tile(blockIdx.x, p.nblocks);
    const int bh = tile / p.nsb;
    const int sb = tile % p.nsb;
    const int tile0 = sb * p.tiles_per_wg;                  // first query tile of this workgroup
    const int wtile0 = tile0 + wave * QT;                    // first query tile of this wave

    // LDS carve-up: [E table][fp64 scan scratch][K tile][V^T tile]
    float *E = reinterpret_cast<float *>(smem);
    double *scan_sh = reinterpret_cast<double *>(smem + (KIND == kMaskLit ? 0 : Lpad * 4));
    unsigned char *tiles = smem + (KIND == kMaskLit ? 0 : Lpad * 4 + (KIND == kMaskS ? nt * 8 : 0));
    T *Ks = reinterpret_cast<T *>(tiles);
    T *Vt = Ks + kKB * C::KROW;

    const size_t base = (size_t)bh * L;  // row offset of this (batch, head)
    const T *qg = reinterpret_cast<const T *>(p.q) + base * D;
    const T *kg = reinterpret_cast<const T *>(p.k) + base * D;
    const T *vg = reinterpret_cast<const T *>(p.v) + base * D;

    if constexpr (KIND != kMaskLit)
        build_exponents<KIND>(E, scan_sh, p.ll, bh, p.H, L, Lpad, min(tile0 * 16, L - 1), tid, nt);

    // ---- query fragments: phi(q) for this wave's tiles (B operand of S^T = K Q^T) -------------
    typename C::QFrag qf[QT][C::NS];
    float Ei[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int i = (wtile0 + qt) * 16 + r;
        float x[C::CPL];
        if (i < L && wtile0 + qt < ntiles) {
            const T *src = qg + (size_t)i * D + g * C::CPL;
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) x[c] = (float)src[c];
        } else {
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) x[c] = 0.f;
        }
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < C::CPL; ++c) {
            x[c] = phi_pre<KIND>(x[c]);
            ss += x[c] * x[c];
        }
        if constexpr (KIND == kMaskS) {
            ss += __shfl_xor(ss, 16, 64);
            ss += __shfl_xor(ss, 32, 64);
            const float sc = inv_norm(ss);
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) x[c] *= sc;
        }
        if (!(i < L)) {
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) x[c] = 0.f;
        }
        if constexpr (BF16) {
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                bf16x8 f;
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = (8 * s + e < C::CPL) ? f2bf(x[8 * s + e]) : f2bf(0.f);
                qf[qt][s] = f;
            }
        } else {
#pragma unroll
            for (int s = 0; s < C::NS; ++s) qf[qt][s] = x[s];
        }
        Ei[qt] = 0.f;
        if constexpr (KIND != kMaskLit) Ei[qt] = E[min(i, L - 1)];
    }

    f32x4 acc_o[QT][D / 16];
    float den[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        den[qt] = 0.f;
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct) acc_o[qt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int wave_tiles = max(0, min(QT, ntiles - wtile0));

    for (int kb = 0; kb < nkb; ++kb) {
        // ---- stage phi(K) (row-major) and V^T for keys kb*32 .. kb*32+31 -------------------------
        const int total = kKB * C::CPK;
        for (int c0 = 0; c0 < total; c0 += nt) {
            const int c = c0 + tid;
            const bool active = c < total;
            const int kl = c / C::CPK, cc = (c % C::CPK) * C::VEC;
            const int j = kb * kKB + kl;
            float xk[C::VEC], xv[C::VEC];
            if (active && j < L) {
                const T *ks = kg + (size_t)j * D + cc;
                const T *vs = vg + (size_t)j * D + cc;
#pragma unroll
                for (int e = 0; e < C::VEC; ++e) {
                    xk[e] = (float)ks[e];
                    xv[e] = (float)vs[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < C::VEC; ++e) xk[e] = xv[e] = 0.f;
            }
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < C::VEC; ++e) {
                xk[e] = phi_pre<KIND>(xk[e]);
                ss += xk[e] * xk[e];
            }
            if constexpr (KIND == kMaskS) {
                ss = group_sum<C::CPK>(ss);
                const float sc = inv_norm(ss);
#pragma unroll
                for (int e = 0; e < C::VEC; ++e) xk[e] *= sc;
            }
            if (active) {
                const bool valid = j < L;
#pragma unroll
                for (int e = 0; e < C::VEC; ++e) {
                    Ks[kl * C::KROW + cc + e] = (T)(valid ? xk[e] : 0.f);
                    Vt[(cc + e) * C::VROW + kl] = (T)xv[e];
                }
            }
        }
        __syncthreads();

        if (wave_tiles > 0) {
            // K fragments (A operand of S^T): row 16t + r, channels of lane group g
            typename C::QFrag kf[2][C::NS];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const T *src = Ks + (16 * t + r) * C::KROW + g * C::CPL;
                if constexpr (BF16) {
#pragma unroll
                    for (int s = 0; s < C::NS; ++s) {
                        bf16x8 f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) f[e] = (8 * s + e < C::CPL) ? src[8 * s + e] : f2bf(0.f);
                        kf[t][s] = f;
                    }
                } else {
#pragma unroll
                    for (int s = 0; s < C::NS; ++s) kf[t][s] = src[s];
                }
            }
            // mask exponents of the 8 keys this lane touches: 16t + 4g + e
            float Ej[2][4];
            if constexpr (KIND != kMaskLit) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) Ej[t][e] = E[kb * kKB + 16 * t + 4 * g + e];
            }
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                if (qt >= wave_tiles) break;
                f32x4 s_acc[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    s_acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < C::NS; ++s) {
                        if constexpr (BF16)
                            s_acc[t] = mfma_bf16(kf[t][s], qf[qt][s], s_acc[t]);
                        else
                            s_acc[t] = mfma_f32(kf[t][s], qf[qt][s], s_acc[t]);
                    }
                }
                // s_acc[t][e] = S[query r][key 16t + 4g + e]; mask, row-sum, feed to P V
                float pv[2][4];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float m = 1.f;
                        if constexpr (KIND != kMaskLit) m = fast_exp2(-__builtin_fabsf(Ei[qt] - Ej[t][e]));
                        const float pe = s_acc[t][e] * m;
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
                        const T *vs = Vt + (16 * ct + r) * C::VROW + 4 * g;
                        bf16x8 vf;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            vf[e] = vs[e];
                            vf[4 + e] = vs[16 + e];
                        }
                        acc_o[qt][ct] = mfma_bf16(vf, pf, acc_o[qt][ct]);
                    }
                } else {
#pragma unroll
                    for (int ct = 0; ct < D / 16; ++ct) {
                        const T *vs = Vt + (16 * ct + r) * C::VROW + 4 * g;
#pragma unroll
                        for (int t = 0; t < 2; ++t)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                acc_o[qt][ct] = mfma_f32(vs[16 * t + e], pv[t][e], acc_o[qt][ct]);
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue: full row sums, divide, store -------------------------------------------------
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        if (qt >= wave_tiles) break;
        float dsum = den[qt];
        dsum += __shfl_xor(dsum, 16, 64);
        dsum += __shfl_xor(dsum, 32, 64);
        const float div = dsum + p.eps;
        const int i = (wtile0 + qt) * 16 + r;
        if (i < L) {
            const float inv = 1.f / div;
            const size_t row = base + i;
            if (p.out_bf16) {
                __bf16 *yo = reinterpret_cast<__bf16 *>(p.y) + row * D;
#pragma unroll
                for (int ct = 0; ct < D / 16; ++ct) {
                    bf16x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = f2bf(acc_o[qt][ct][e] * inv);
                    *reinterpret_cast<bf16x4 *>(yo + 16 * ct + 4 * g) = o;
                }
            } else {
                float *yo = reinterpret_cast<float *>(p.y) + row * D;
#pragma unroll
                for (int ct = 0; ct < D / 16; ++ct) {
                    f32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = acc_o[qt][ct][e] * inv;
                    *reinterpret_cast<f32x4 *>(yo + 16 * ct + 4 * g) = o;
                }
            }
            if (p.den_out && g == 0) p.den_out[row] = div;
        }
    }
}

// Launch shape of the full form: query tiles per wave, waves per workgroup, workgroups per
// (batch, head), and the LDS the kernel asks for.
struct FullShape {
    int qt, nw, nsb;
    size_t lds;
};

FullShape full_shape(const AttnArgs &a) {
    const int ntiles = (a.L + 15) / 16;
    const long bhs = (long)a.B * a.H;
    int qt = 1;
    if (a.in_bf16) {
        // largest tile count per wave that still gives >= 2 waves per SIMD (256 CUs x 4 SIMDs)
        const int cand[3] = {a.d == 128 ? 2 : 4, 2, 1};
        for (int c : cand) {
            qt = c;
            if (bhs * ((ntiles + c - 1) / c) >= 2048) break;
        }
    }
    const int wtiles = (ntiles + qt - 1) / qt;      // waves needed per (batch, head)
    FullShape sh;
    sh.qt = qt;
    sh.nw = wtiles < 8 ? wtiles : 8;
    sh.nsb = (ntiles + sh.nw * qt - 1) / (sh.nw * qt);
    const size_t esz = a.in_bf16 ? 2 : 4;
    const int Lpad = ((a.L + kKB - 1) / kKB) * kKB;
    size_t lds = (size_t)(kKB * (a.d + (a.in_bf16 ? 8 : 4)) + a.d * (kKB + (a.in_bf16 ? 8 : 4))) * esz;
    if (a.kind != kMaskLit) lds += (size_t)Lpad * 4;
    if (a.kind == kMaskS) lds += (size_t)sh.nw * 64 * 8;
    sh.lds = lds;
    return sh;
}

template <int D, int KIND, int QT, bool BF16>
hipError_t launch_full_t(const AttnArgs &a, hipStream_t stream, const FullShape &sh) {
    FullParams p;
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
    p.nsb = sh.nsb;
    p.tiles_per_wg = sh.nw * QT;
    p.nblocks = a.B * a.H * sh.nsb;
    if (sh.lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&full_kernel<D, KIND, QT, BF16>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh.lds);
    hipLaunchKernelGGL((full_kernel<D, KIND, QT, BF16>), dim3(p.nblocks), dim3(sh.nw * 64), sh.lds, stream, p);
    return hipGetLastError();
}

template <int D, int KIND, bool BF16>
hipError_t dispatch_qt(const AttnArgs &a, hipStream_t stream) {
    const FullShape sh = full_shape(a);
    if constexpr (BF16) {
        if constexpr (D != 128)
            if (sh.qt == 4) return launch_full_t<D, KIND, 4, BF16>(a, stream, sh);
        if (sh.qt == 2) return launch_full_t<D, KIND, 2, BF16>(a, stream, sh);
    }
    return launch_full_t<D, KIND, 1, BF16>(a, stream, sh);
}

template <int D, bool BF16>
hipError_t dispatch_kind(const AttnArgs &a, hipStream_t stream) {
    switch (a.kind) {
    case kMaskLit: return dispatch_qt<D, kMaskLit, BF16>(a, stream);
    case kMaskD: return dispatch_qt<D, kMaskD, BF16>(a, stream);
    default: return dispatch_qt<D, kMaskS, BF16>(a, stream);
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

}  // namespace

Plan plan_full(const AttnArgs &a) {
    Plan p;
    p.ok = full_shape(a).lds <= kLdsPerWorkgroup;
    p.workspace = 0;
    return p;
}

hipError_t launch_full(const AttnArgs &a, hipStream_t stream) {
    return a.in_bf16 ? dispatch_d<true>(a, stream) : dispatch_d<false>(a, stream);
}

}  // namespace lion
