// lion_full.hip -- full (attention) form of LION bidirectional masked linear attention.
//
// Y = SCALE(phi(Q) phi(K)^T (.) M) V, the form LION trains with ("LION: A bidirectional framework
// that trains like a Transformer and infers like an RNN", reply "Concern 1", Theorem 3.3 Eq. 25).
// The L x L score matrix is never materialised.  A workgroup owns a run of 16-row query tiles of one
// (batch, head); each wave owns up to QT consecutive tiles.  Keys and values pass through LDS as
// row-major tiles loaded straight from global memory, and V^T fragments are read from the row-major
// value rows with ds_read_b64_tr_b16.  Two kernels:
//   - resident (bf16, d >= 32, keys and values of the whole sequence within 64 KiB of LDS and at most
//     448 rows, grids of at most 256 workgroups): one compute wave per query tile plus a loader wave
//     that issues every key/value load of the workgroup at the start, in rounds; the compute waves
//     work on each round of keys as soon as it has landed, so matrix-core work overlaps the loads;
//   - streaming (everything else): the sequence as one stage, or double-buffered stages whose loads
//     are in flight while the waves compute on the previous one.
// phi is applied to the staged keys in place (or on the way into LDS).  Per 32-key sub-block and
// query tile a wave forms S^T = phi(K) phi(Q)^T on matrix cores, applies the mask in registers,
// accumulates fp32 row sums, and feeds the masked scores back as the B operand of O^T = V^T P^T
// (the D layout of the first product is the B layout of the second, so P never leaves registers).
//
// Mask (see lion_mask.h): M_ij = exp2(-|E_i - E_j|).  A sub-block whose keys all lie after a wave's
// last query row r uses the separable form M_ij = exp2(E_r - E_i) * exp2(E_j - E_r) (both factors
// <= 1): the row factor is computed once per query row, the column factor once per key and shared
// by all the wave's tiles, so a score costs two multiplies instead of an exponential.  Keys wholly
// before the first row r0 use exp2(E_i - E_r0) * exp2(E_r0 - E_j) likewise.  Only sub-blocks that
// overlap the wave's rows pay one exponential per score.
//
// Two token orders (patch-reordered LION-D / LION-S: the pages average the masks of two patch orders,
// reply "P2: Comparison against vision SSMs", item 1): M = (M_b + M_c) / 2 with M_c the same mask along a
// second order of the tokens.  Its exponents are a second table F_t = prefix sum of log(lambda) along that
// order, at token t's position in it, so (M_c)_ij = exp2(-|F_i - F_j|); every score then pays two
// exponentials (F is not monotone along the tokens' own order, so no separable shortcut applies).
#include <algorithm>
#include <type_traits>

#include "lion_device.h"
#include "lion_internal.h"
#include "lion_mask.h"
#include "lion_stage.h"

namespace lion {
namespace {

constexpr int kKB = 32;                       // keys per sub-block (two 16-key halves of S^T)
constexpr size_t kStageBytes = 64 * 1024;     // K + V bytes of one stage (a double buffer halves it)
constexpr long kResidentMaxGrid = 256;        // resident kernel: at most one workgroup per CU

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
    int sk;            // keys per stage (multiple of 32)
    int nbuf;          // 1: the whole sequence is one stage; 2: double-buffered stages
    int causal;        // keys after the query masked out
    const int *order;  // two-order variant: the tokens listed in the second order [L]
};

// Second-order exponent table F[t] = log2 of the decay product along `order` up to token t's position
// (LION-S: an fp64 scan of log(lambda) gathered in that order; LION-D: position * log2(lambda_h));
// entries past L - 1 are 0.  Order entries are clamped to [0, L) (the caller guarantees a permutation).
template <int KIND>
__device__ void build_order_exponents(float *F, double *scan_sh, const float *ll, const int *order, int bh, int H,
                                      int L, int Lpad, int tid, int nt) {
    for (int t = L + tid; t < Lpad; t += nt) F[t] = 0.f;
    if constexpr (KIND == kMaskD) {
        const float lg = ll[bh % H] * kLog2e;
        for (int p = tid; p < L; p += nt) F[min(max(order[p], 0), L - 1)] = (float)p * lg;
        __syncthreads();
    } else if constexpr (KIND == kMaskS) {
        const float *row = ll + (size_t)bh * L;
        const int seg = (L + nt - 1) / nt;
        const int p0 = tid * seg, p1 = min(p0 + seg, L);
        double s = 0.0;
        for (int p = p0; p < p1; ++p) s += (double)row[min(max(order[p], 0), L - 1)];
        double a = block_excl_scan(s, scan_sh, tid, nt);
        for (int p = p0; p < p1; ++p) {
            const int t = min(max(order[p], 0), L - 1);
            a += (double)row[t];
            F[t] = (float)(a * 1.4426950408889634);
        }
        __syncthreads();
    }
}

template <int D, bool BF16>
struct FullCfg {
    using T = std::conditional_t<BF16, __bf16, float>;
    using RT = RowTile<D, T>;
    static constexpr int CPL = D / 4;                       // channels owned by each lane group
    static constexpr int NS = BF16 ? (CPL + 7) / 8 : CPL;   // score MFMA steps
    using QFrag = std::conditional_t<BF16, bf16x8, float>;
};

// Registers of one wave: phi(q) fragments of its query tiles (B operand of S^T = K Q^T), their mask
// exponents and separable-mask row factors, the output accumulators and the fp32 row sums.
template <int D, int QT, bool BF16>
struct FullWave {
    using C = FullCfg<D, BF16>;
    typename C::QFrag qf[QT][C::NS];
    float Ei[QT], Fi[QT], rowf_b[QT], rowf_a[QT];
    f32x4 acc_o[QT][D / 16];
    float den[QT];
};

// Raw query elements of the wave's tiles (row (wtile0 + qt) * 16 + r, the channels of lane group g):
// loads only, consumed later by query_frags so that other loads can be issued in between.
template <int D, int QT, bool BF16, typename T = typename FullCfg<D, BF16>::T, int CPL = FullCfg<D, BF16>::CPL>
__device__ __forceinline__ void load_query(T (&xr)[QT][CPL], const T *qg, int wtile0, int wave_tiles, int L, int r,
                                           int g) {
    using C = FullCfg<D, BF16>;
    using RT = typename C::RT;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int i = (wtile0 + qt) * 16 + r;
        const bool ok = i < L && qt < wave_tiles;
        const T *row = qg + (size_t)(ok ? i : 0) * D;
        if constexpr (BF16 && C::CPL >= 8) {
            // fragment st of lane group g: the eight channels of 16-byte chunk 4 st + g
#pragma unroll
            for (int st = 0; st < C::NS; ++st) {
                const u32x4 raw = ld16(row + 8 * (4 * st + g));
                __builtin_memcpy(&xr[qt][8 * st], &raw, 16);
            }
        } else if constexpr (C::CPL * sizeof(T) % 16 == 0) {
            const T *src = row + g * C::CPL;
#pragma unroll
            for (int c = 0; c < C::CPL; c += RT::VEC) {
                const u32x4 raw = ld16(src + c);
                __builtin_memcpy(&xr[qt][c], &raw, 16);
            }
        } else {
            const T *src = row + g * C::CPL;
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) xr[qt][c] = src[c];
        }
    }
}

// phi(q) fragments from the raw elements (rows past L or past the wave's tiles become zero).
template <int D, int KIND, int QT, bool BF16, typename T = typename FullCfg<D, BF16>::T,
          int CPL = FullCfg<D, BF16>::CPL>
__device__ __forceinline__ void query_frags(FullWave<D, QT, BF16> &w, const T (&xr)[QT][CPL], int wtile0,
                                            int wave_tiles, int L, int r) {
    using C = FullCfg<D, BF16>;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int i = (wtile0 + qt) * 16 + r;
        const bool ok = i < L && qt < wave_tiles;
        float x[C::CPL];
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < C::CPL; ++c) {
            x[c] = phi_pre<KIND>((float)xr[qt][c]);
            ss += x[c] * x[c];
        }
        float sc = ok ? 1.f : 0.f;
        if constexpr (KIND == kMaskS) {
            ss += __shfl_xor(ss, 16, 64);
            ss += __shfl_xor(ss, 32, 64);
            sc *= inv_norm(ss);
        }
        if constexpr (BF16) {
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                bf16x8 f;
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = (8 * s + e < C::CPL) ? f2bf(x[8 * s + e] * sc) : f2bf(0.f);
                w.qf[qt][s] = f;
            }
        } else {
#pragma unroll
            for (int s = 0; s < C::NS; ++s) w.qf[qt][s] = x[s] * sc;
        }
    }
}

// Mask exponents of the wave's rows, the row factors of the separable mask (keys before the wave's
// first row r0: exp2(E_i - E_r0); keys after its last row rl: exp2(E_rl - E_i)), zeroed accumulators.
template <int D, int KIND, int QT, bool BF16, bool TWO>
__device__ __forceinline__ void wave_rows_init(FullWave<D, QT, BF16> &w, const float *E, const float *F, int wtile0,
                                               int L, int r, float e_first, float e_last) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int i = (wtile0 + qt) * 16 + r;
        w.Ei[qt] = w.Fi[qt] = 0.f;
        if constexpr (KIND != kMaskLit) w.Ei[qt] = E[min(i, L - 1)];
        if constexpr (TWO) w.Fi[qt] = F[min(i, L - 1)];
        w.rowf_b[qt] = w.rowf_a[qt] = 1.f;
        if constexpr (KIND != kMaskLit) {
            w.rowf_b[qt] = fast_exp2(w.Ei[qt] - e_first);
            w.rowf_a[qt] = fast_exp2(e_last - w.Ei[qt]);
        }
        w.den[qt] = 0.f;
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct) w.acc_o[qt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// Region of a 32-key sub-block starting at key j0 relative to the wave's rows rw0 .. rwl
// (wave-uniform): 0 = overlap (one exponential per score), 1 = every key before every row, 2 = every
// key after every row (separable mask).
template <int KIND, bool TWO>
__device__ __forceinline__ int subblock_region(int j0, int rw0, int rwl, bool causal) {
    if (TWO || (KIND == kMaskLit && !causal)) return 0;
    if (j0 + kKB - 1 < rw0) return 1;
    if (j0 > rwl) return 2;
    return 0;
}

// One 32-key sub-block (rows hk .. hk + 31 of the staged tiles, keys j0 .. j0 + 31) for the wave's
// query tiles: S^T = phi(K) phi(Q)^T on matrix cores, the mask in registers, fp32 row sums, then
// O^T += V^T P^T with the masked scores as the B operand.
template <int D, int KIND, int QT, bool BF16, bool TWO, typename T = typename FullCfg<D, BF16>::T>
__device__ __forceinline__ void full_subblock(FullWave<D, QT, BF16> &w, const T *kbuf, const T *vbuf, int hk, int j0,
                                              const float *E, const float *F, int region, float e_first,
                                              float e_last, int wtile0, int wave_tiles, bool causal, int r, int g) {
    using C = FullCfg<D, BF16>;
    using RT = typename C::RT;
    // K fragments (A operand of S^T): key row 16t + r of the sub-block, channels of group g
    auto kelem = [&](int t, int col) { return kbuf + RT::off(hk + 16 * t + r, col); };
    bf16x8 kf[2][BF16 ? C::NS : 1];
    if constexpr (BF16) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int st = 0; st < C::NS; ++st) {
                if constexpr (C::CPL >= 8) {
                    kf[t][st] = *reinterpret_cast<const bf16x8 *>(kelem(t, 8 * (4 * st + g)));
                } else {
                    const bf16x4 h4 = *reinterpret_cast<const bf16x4 *>(kelem(t, g * C::CPL));
                    bf16x8 f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        f[e] = h4[e];
                        f[4 + e] = f2bf(0.f);
                    }
                    kf[t][st] = f;
                }
            }
    }
    // per-key mask data of the 8 keys this lane touches, j0 + 16t + 4g + e: the exponent in the
    // overlap region, the column factor elsewhere
    float mk[2][4], fk[2][4];
    if constexpr (TWO) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const f32x4 f4 = *reinterpret_cast<const f32x4 *>(F + j0 + 16 * t + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) fk[t][e] = f4[e];
        }
    }
    if constexpr (KIND != kMaskLit) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const f32x4 e4 = *reinterpret_cast<const f32x4 *>(E + j0 + 16 * t + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mk[t][e] = region == 0 ? e4[e] : fast_exp2(region == 1 ? e_first - e4[e] : e4[e] - e_last);
        }
    }
    // V^T fragments (A operand of O^T += V^T P^T): keys j0 + 4g + e and j0 + 16 + 4g + e of
    // value channel 16 ct + r, read transposed from the row-major value tile
    bf16x8 vfr[BF16 ? D / 16 : 1];
    if constexpr (BF16) {
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct) {
            const int row = hk + 4 * g + (r >> 2), col = 16 * ct + 4 * (r & 3);
            const bf16x4 lo = read_tr_b16(vbuf + RT::off(row, col));
            const bf16x4 hi = read_tr_b16(vbuf + RT::off(row + 16, col));
            bf16x8 f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = lo[e];
                f[4 + e] = hi[e];
            }
            vfr[ct] = f;
        }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        if (qt >= wave_tiles) break;
        f32x4 sacc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < C::NS; ++st) {
                if constexpr (BF16)
                    sacc[t] = mfma_bf16(kf[t][st], w.qf[qt][st], sacc[t]);
                else
                    sacc[t] = mfma_f32(*kelem(t, g * C::CPL + st), w.qf[qt][st], sacc[t]);
            }
        }
        // sacc[t][e] = S[query r][key j0 + 16t + 4g + e]; mask it (region is wave-uniform)
        float pv[2][4];
        if constexpr (KIND == kMaskLit) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) pv[t][e] = sacc[t][e];
        } else if (region == 0) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pv[t][e] = TWO ? sacc[t][e] * (0.5f * (fast_exp2(-__builtin_fabsf(w.Ei[qt] - mk[t][e])) +
                                                           fast_exp2(-__builtin_fabsf(w.Fi[qt] - fk[t][e]))))
                                   : sacc[t][e] * fast_exp2(-__builtin_fabsf(w.Ei[qt] - mk[t][e]));
        } else {
            const float rowf = region == 1 ? w.rowf_b[qt] : w.rowf_a[qt];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) pv[t][e] = (sacc[t][e] * rowf) * mk[t][e];
        }
        if (causal && region == 0) {
            // keys after this lane's query row are masked out
            const int i = (wtile0 + qt) * 16 + r;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j0 + 16 * t + 4 * g + e > i) pv[t][e] = 0.f;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) w.den[qt] += pv[t][e];
        if constexpr (BF16) {
            bf16x8 pf;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pf[e] = f2bf(pv[0][e]);
                pf[4 + e] = f2bf(pv[1][e]);
            }
#pragma unroll
            for (int ct = 0; ct < D / 16; ++ct) w.acc_o[qt][ct] = mfma_bf16(vfr[ct], pf, w.acc_o[qt][ct]);
        } else {
#pragma unroll
            for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w.acc_o[qt][ct] = mfma_f32(vbuf[RT::off(hk + 16 * t + 4 * g + e, 16 * ct + r)],
                                                 pv[t][e], w.acc_o[qt][ct]);
        }
    }
}

// Epilogue: the full row sums (over the four lane groups), one divide per row, store.
template <int D, int QT, bool BF16>
__device__ __forceinline__ void full_epilogue(FullWave<D, QT, BF16> &w, const FullParams &p, size_t base, int wtile0,
                                              int wave_tiles, int L, int r, int g) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        if (qt >= wave_tiles) break;
        float dsum = w.den[qt];
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
                    for (int e = 0; e < 4; ++e) o[e] = f2bf(w.acc_o[qt][ct][e] * inv);
                    *reinterpret_cast<bf16x4 *>(yo + 16 * ct + 4 * g) = o;
                }
            } else {
                float *yo = reinterpret_cast<float *>(p.y) + row * D;
#pragma unroll
                for (int ct = 0; ct < D / 16; ++ct) {
                    f32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = w.acc_o[qt][ct][e] * inv;
                    *reinterpret_cast<f32x4 *>(yo + 16 * ct + 4 * g) = o;
                }
            }
            if (p.den_out && g == 0) p.den_out[row] = div;
        }
    }
}

// Streaming kernel: any length, fp32 or bf16, one or two token orders.  Keys and values pass through
// LDS as one stage or as double-buffered stages.  It keeps the sub-block arithmetic of the helpers above
// written out in place: built from the helpers it compiled to fewer registers but measured 6-7% slower
// (B64 H12 L197 D, 36.3 vs 33.8 us on one box).
// Lane i of the lane's 16-lane row (DPP row_newbcast; the multiply that uses it takes it as a DPP operand).
__device__ __forceinline__ float row_bcast(float x, int i) {
    switch (i) {
#define LION_RB(I) \
    case I: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + I, 0xF, 0xF, false));
    LION_RB(0) LION_RB(1) LION_RB(2) LION_RB(3) LION_RB(4) LION_RB(5) LION_RB(6) LION_RB(7)
#undef LION_RB
    default: return x;
    }
}

template <int D, int KIND, int QT, bool BF16, bool TWO, bool INB = BF16>
__global__ void __launch_bounds__(512) full_kernel(FullParams p) {
    using C = FullCfg<D, BF16>;
    using T = typename C::T;                               // compute and LDS type
    using TI = std::conditional_t<INB, __bf16, T>;        // input type (bf16 inputs of fp32 arithmetic)
    using RT = typename C::RT;
    static_assert(!BF16 || INB, "bf16 arithmetic takes bf16 inputs");
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, nt = blockDim.x, nw = nt >> 6;
    const int lane = tid & 63, wave = uniform(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int L = p.L, SK = p.sk;
    const int nst = (L + SK - 1) / SK;
    const int Lpad = nst * SK;
    const int ntiles = (L + 15) / 16;

    const int tile = xcd_tile(blockIdx.x, p.nblocks);
    const int bh = tile / p.nsb;
    // causal: workgroups of later rows (more keys) are dispatched first, so the light ones form the tail
    const int sb = p.causal ? p.nsb - 1 - tile % p.nsb : tile % p.nsb;
    const int tile0 = sb * p.tiles_per_wg;                  // first query tile of this workgroup
    const int wtile0 = tile0 + wave * QT;                    // first query tile of this wave
    const int wave_tiles = max(0, min(QT, ntiles - wtile0));

    // LDS: [K stage buffers][V stage buffers][E table][fp64 scan scratch]
    T *Kb = reinterpret_cast<T *>(smem);
    T *Vb = Kb + (size_t)p.nbuf * SK * D;
    float *E = reinterpret_cast<float *>(Vb + (size_t)p.nbuf * SK * D);
    float *F = E + Lpad;                                    // second-order exponents (TWO)
    double *scan_sh = reinterpret_cast<double *>(E + (KIND == kMaskLit ? 0 : (TWO ? 2 : 1) * Lpad));

    const size_t base = (size_t)bh * L;
    const TI *qg = reinterpret_cast<const TI *>(p.q) + base * D;
    const TI *kg = reinterpret_cast<const TI *>(p.k) + base * D;
    const TI *vg = reinterpret_cast<const TI *>(p.v) + base * D;
    // rows of keys or values into a stage buffer: direct loads, or (bf16 inputs of fp32 arithmetic)
    // converted through registers
    auto stage = [&](T *tile, const TI *src, int row0) {
        if constexpr (!BF16 && INB)
            stage_rows_cvt<D>(tile, src, row0, SK, L, tid, nt);
        else
            stage_rows<D, T>(tile, src, row0, SK, L, wave, nw, lane);
    };

    // stage 0 in flight while the prologue runs.  When the whole sequence is one stage (and its key
    // chunks fit 4 per thread), keys come through registers and phi is applied on the way into LDS.
    const bool kreg = BF16 && p.nbuf == 1 && SK * RT::CPK <= 4 * nt;
    u32x4 kx[4];
    stage(Vb, vg, 0);
    if (kreg) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c16 = min(tid + u * nt, SK * RT::CPK - 1);
            kx[u] = ld16(kg + (size_t)min(c16 / RT::CPK, L - 1) * D + (c16 % RT::CPK) * RT::VEC);
        }
    } else {
        stage(Kb, kg, 0);
    }

    if constexpr (KIND != kMaskLit)
        build_exponents<KIND>(E, scan_sh, p.ll, bh, p.H, L, Lpad, min(tile0 * 16, L - 1), tid, nt);
    if constexpr (TWO) build_order_exponents<KIND>(F, scan_sh, p.ll, p.order, bh, p.H, L, Lpad, tid, nt);

    // ---- query fragments: phi(q) of this wave's tiles (B operand of S^T = K Q^T) -----------------
    typename C::QFrag qf[QT][C::NS];
    float Ei[QT], Fi[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int i = (wtile0 + qt) * 16 + r;
        const bool ok = i < L && qt < wave_tiles;
        float x[C::CPL];
        const TI *row = qg + (size_t)(ok ? i : 0) * D;
        if constexpr (!BF16 && INB) {
            const TI *src = row + g * C::CPL;
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) x[c] = (float)src[c];
        } else if constexpr (BF16 && C::CPL >= 8) {
            // fragment st of lane group g: the eight channels of 16-byte chunk 4 st + g
#pragma unroll
            for (int st = 0; st < C::NS; ++st) {
                T tmp[8];
                const u32x4 raw = ld16(row + 8 * (4 * st + g));
                __builtin_memcpy(tmp, &raw, 16);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[8 * st + e] = (float)tmp[e];
            }
        } else if constexpr (C::CPL * sizeof(T) % 16 == 0) {
            const T *src = row + g * C::CPL;
#pragma unroll
            for (int c = 0; c < C::CPL; c += RT::VEC) {
                T tmp[RT::VEC];
                const u32x4 raw = ld16(src + c);
                __builtin_memcpy(tmp, &raw, 16);
#pragma unroll
                for (int e = 0; e < RT::VEC; ++e) x[c + e] = (float)tmp[e];
            }
        } else {
            const T *src = row + g * C::CPL;
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) x[c] = (float)src[c];
        }
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < C::CPL; ++c) {
            x[c] = phi_pre<KIND>(x[c]);
            ss += x[c] * x[c];
        }
        float sc = ok ? 1.f : 0.f;
        if constexpr (KIND == kMaskS) {
            ss += __shfl_xor(ss, 16, 64);
            ss += __shfl_xor(ss, 32, 64);
            sc *= inv_norm(ss);
        }
        if constexpr (BF16) {
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                bf16x8 f;
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = (8 * s + e < C::CPL) ? f2bf(x[8 * s + e] * sc) : f2bf(0.f);
                qf[qt][s] = f;
            }
        } else {
#pragma unroll
            for (int s = 0; s < C::NS; ++s) qf[qt][s] = x[s] * sc;
        }
        Ei[qt] = Fi[qt] = 0.f;
        if constexpr (KIND != kMaskLit) Ei[qt] = E[min(i, L - 1)];
        if constexpr (TWO) Fi[qt] = F[min(i, L - 1)];
    }

    // rows of this wave and the row factors of the separable mask (keys before / after the rows)
    const int rw0 = wtile0 * 16;
    const int rwl = min((wtile0 + wave_tiles) * 16, L) - 1;
    float e_first = 0.f, e_last = 0.f;
    if constexpr (KIND != kMaskLit) {
        if (wave_tiles > 0) {
            e_first = uniform(E[rw0]);
            e_last = uniform(E[rwl]);
        }
    }
    float rowf_b[QT], rowf_a[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        rowf_b[qt] = rowf_a[qt] = 1.f;
        if constexpr (KIND != kMaskLit) {
            rowf_b[qt] = fast_exp2(Ei[qt] - e_first);
            rowf_a[qt] = fast_exp2(e_last - Ei[qt]);
        }
    }

    f32x4 acc_o[QT][D / 16];
    float den[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        den[qt] = 0.f;
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct) acc_o[qt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    if (kreg) {
        // phi on the keys held in registers (rows at or past L written as zeros); the single stage is
        // then complete after one barrier
        wait_vm_all();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c16 = tid + u * nt, row = c16 / RT::CPK;
            T x[RT::VEC];
            __builtin_memcpy(x, &kx[u], 16);
            float f[RT::VEC], ss = 0.f;
#pragma unroll
            for (int e = 0; e < RT::VEC; ++e) {
                f[e] = phi_pre<KIND>((float)x[e]);
                ss += f[e] * f[e];
            }
            float scl = row < L ? 1.f : 0.f;
            if constexpr (KIND == kMaskS) scl *= inv_norm(group_sum<RT::CPK>(ss));
#pragma unroll
            for (int e = 0; e < RT::VEC; ++e) x[e] = (T)(f[e] * scl);
            if (c16 < SK * RT::CPK) __builtin_memcpy(Kb + RT::off(row, (c16 % RT::CPK) * RT::VEC), x, 16);
        }
        __syncthreads();
    }

    // causal: stages wholly after the workgroup's last query row are never needed
    const int nst_used = p.causal ? min(nst, (min((tile0 + p.tiles_per_wg) * 16, L) - 1) / SK + 1) : nst;
    for (int s = 0; s < nst_used; ++s) {
        const int buf = p.nbuf == 1 ? 0 : (s & 1);
        T *kbuf = Kb + (size_t)buf * SK * D;
        const T *vbuf = Vb + (size_t)buf * SK * D;
        if (!kreg) {
        wait_vm_all();
        __syncthreads();                                     // stage s is in LDS; buffer s+1 is free
        if (s + 1 < nst_used) {
            const int nb = (s + 1) & 1;
            stage(Kb + (size_t)nb * SK * D, kg, (s + 1) * SK);
            stage(Vb + (size_t)nb * SK * D, vg, (s + 1) * SK);
        }
        // phi over the staged keys (in place); keys at or past L become zero rows
        {
            const int row_end = min(SK, L - s * SK);         // rows of real keys in this stage
            const int nslot = SK * RT::CPK;
            const int first = (KIND == kMaskD) ? row_end * RT::CPK : 0;   // identity phi: only padding
            for (int sl0 = first - first % 64; sl0 < nslot; sl0 += nt) {
                const int sl = sl0 + tid;
                if (sl - lane >= nslot) break;                // wave-uniform: nslot is a multiple of 64
                const bool mine = sl >= first && sl < nslot;
                const int row = sl / RT::CPK;
                T x[RT::VEC];
                __builtin_memcpy(x, kbuf + (size_t)sl * RT::VEC, 16);
                float f[RT::VEC], ss = 0.f;
#pragma unroll
                for (int e = 0; e < RT::VEC; ++e) {
                    f[e] = phi_pre<KIND>((float)x[e]);
                    ss += f[e] * f[e];
                }
                float scl = row < row_end ? 1.f : 0.f;
                if constexpr (KIND == kMaskS) scl *= inv_norm(group_sum<RT::CPK>(ss));
#pragma unroll
                for (int e = 0; e < RT::VEC; ++e) x[e] = (T)(f[e] * scl);
                if (mine) __builtin_memcpy(kbuf + (size_t)sl * RT::VEC, x, 16);
            }
        }
        __syncthreads();
        }
        if (wave_tiles == 0) continue;

        for (int h = 0; h < SK / kKB; ++h) {
            const int j0 = s * SK + h * kKB;
            if (j0 >= L) break;
            if (p.causal && j0 > rwl) break;                   // causal: no later keys
            // region of this sub-block relative to the wave's rows (wave-uniform)
            int region = 0;                                    // overlap: per-score exponentials
            if (!TWO && (KIND != kMaskLit || p.causal)) {
                if (j0 + kKB - 1 < rw0) region = 1;            // every key before every row
                else if (j0 > rwl) region = 2;                  // every key after every row
            }
            // K fragments (A operand of S^T): key row 16t + r of the sub-block, channels of group g
            auto kelem = [&](int t, int col) { return kbuf + RT::off(h * kKB + 16 * t + r, col); };
            bf16x8 kf[2][BF16 ? C::NS : 1];
            if constexpr (BF16) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int st = 0; st < C::NS; ++st) {
                        if constexpr (C::CPL >= 8) {
                            kf[t][st] = *reinterpret_cast<const bf16x8 *>(kelem(t, 8 * (4 * st + g)));
                        } else {
                            const bf16x4 h4 = *reinterpret_cast<const bf16x4 *>(kelem(t, g * C::CPL));
                            bf16x8 f;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                f[e] = h4[e];
                                f[4 + e] = f2bf(0.f);
                            }
                            kf[t][st] = f;
                        }
                    }
            }
            // per-key mask data of the 8 keys this lane touches, j0 + 16t + 4g + e: the exponents in the
            // overlap region.  Elsewhere the column factor of a key is the same for the 16 lanes of a row
            // (one lane group g): lane r < 8 of the row computes that of key j0 + 16 (r / 4) + 4g + r % 4,
            // and the mask multiply takes it from that lane with a DPP row broadcast.
            float mk[2][4], fk[2][4], mkl = 1.f;
            if constexpr (TWO) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const f32x4 f4 = *reinterpret_cast<const f32x4 *>(F + j0 + 16 * t + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) fk[t][e] = f4[e];
                }
            }
            if constexpr (KIND != kMaskLit) {
                if (region == 0) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const f32x4 e4 = *reinterpret_cast<const f32x4 *>(E + j0 + 16 * t + 4 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e) mk[t][e] = e4[e];
                    }
                } else {
                    const float ej = E[j0 + 16 * ((r >> 2) & 1) + 4 * g + (r & 3)];
                    mkl = fast_exp2(region == 1 ? e_first - ej : ej - e_last);
                }
            }
            // V^T fragments (A operand of O^T += V^T P^T): keys j0 + 4g + e and j0 + 16 + 4g + e of
            // value channel 16 ct + r, read transposed from the row-major value tile
            bf16x8 vfr[BF16 ? D / 16 : 1];
            if constexpr (BF16) {
#pragma unroll
                for (int ct = 0; ct < D / 16; ++ct) {
                    const int row = h * kKB + 4 * g + (r >> 2), col = 16 * ct + 4 * (r & 3);
                    const bf16x4 lo = read_tr_b16(vbuf + RT::off(row, col));
                    const bf16x4 hi = read_tr_b16(vbuf + RT::off(row + 16, col));
                    bf16x8 f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        f[e] = lo[e];
                        f[4 + e] = hi[e];
                    }
                    vfr[ct] = f;
                }
            }
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                if (qt >= wave_tiles) break;
                f32x4 sacc[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < C::NS; ++st) {
                        if constexpr (BF16)
                            sacc[t] = mfma_bf16(kf[t][st], qf[qt][st], sacc[t]);
                        else
                            sacc[t] = mfma_f32(*kelem(t, g * C::CPL + st), qf[qt][st], sacc[t]);
                    }
                }
                // sacc[t][e] = S[query r][key j0 + 16t + 4g + e]; mask it (region is wave-uniform)
                float pv[2][4];
                if constexpr (KIND == kMaskLit) {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e) pv[t][e] = sacc[t][e];
                } else if (region == 0) {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            pv[t][e] = TWO ? sacc[t][e] * (0.5f * (fast_exp2(-__builtin_fabsf(Ei[qt] - mk[t][e])) +
                                                                   fast_exp2(-__builtin_fabsf(Fi[qt] - fk[t][e]))))
                                           : sacc[t][e] * fast_exp2(-__builtin_fabsf(Ei[qt] - mk[t][e]));
                } else {
                    const float rowf = region == 1 ? rowf_b[qt] : rowf_a[qt];
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e) pv[t][e] = row_bcast(mkl, 4 * t + e) * (sacc[t][e] * rowf);
                }
                if (p.causal && region == 0) {
                    // keys after this lane's query row are masked out
                    const int i = (wtile0 + qt) * 16 + r;
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (j0 + 16 * t + 4 * g + e > i) pv[t][e] = 0.f;
                }
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) den[qt] += pv[t][e];
                if constexpr (BF16) {
                    bf16x8 pf;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pf[e] = f2bf(pv[0][e]);
                        pf[4 + e] = f2bf(pv[1][e]);
                    }
#pragma unroll
                    for (int ct = 0; ct < D / 16; ++ct) acc_o[qt][ct] = mfma_bf16(vfr[ct], pf, acc_o[qt][ct]);
                } else {
#pragma unroll
                    for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
                        for (int t = 0; t < 2; ++t)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                acc_o[qt][ct] = mfma_f32(vbuf[RT::off(h * kKB + 16 * t + 4 * g + e, 16 * ct + r)],
                                                         pv[t][e], acc_o[qt][ct]);
                }
            }
        }
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

// Workgroup barrier that waits for this wave's LDS operations only.  (__syncthreads() also carries a
// workgroup release fence, which waits for every direct global->LDS load still in flight -- exactly
// the loads the resident kernel keeps in flight across its barriers.)  Direct loads a consumer reads
// are waited for explicitly by the wave that issued them before it reaches the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 16-byte LDS read and write for the loader wave, in inline assembly (the read waits for itself in the
// same block).  The compiler treats every LDS access that follows a direct global->LDS load as
// dependent on it and would wait for all of the loader's rounds; these accesses touch only a round
// the loader has already waited for.
__device__ __forceinline__ u32x4 lds_read16(const void *p) {
    u32x4 v;
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
    return v;
}
__device__ __forceinline__ void lds_write16(void *p, u32x4 v) {
    const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)p;
    asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(v) : "memory");
}

// phi in place over one 16-byte key chunk (slot) of the resident tile: rows at or past L become zero.
// The chunk is read and written through the loader-safe accessors above.  LION-S's norm sums the
// squares over the chunks of one row, which sit in consecutive lanes.
template <int D, int KIND>
__device__ __forceinline__ void phi_chunk(__bf16 *Kb, int slot, int L) {
    using RT = RowTile<D, __bf16>;
    const int row = slot / RT::CPK;
    const u32x4 raw = lds_read16(Kb + (size_t)slot * RT::VEC);
    __bf16 x[RT::VEC];
    __builtin_memcpy(x, &raw, 16);
    float f[RT::VEC], ss = 0.f;
#pragma unroll
    for (int e = 0; e < RT::VEC; ++e) {
        f[e] = phi_pre<KIND>((float)x[e]);
        ss += f[e] * f[e];
    }
    float scl = row < L ? 1.f : 0.f;
    if constexpr (KIND == kMaskS) scl *= inv_norm(group_sum<RT::CPK>(ss));
#pragma unroll
    for (int e = 0; e < RT::VEC; ++e) x[e] = (__bf16)(f[e] * scl);
    u32x4 out;
    __builtin_memcpy(&out, x, 16);
    lds_write16(Kb + (size_t)slot * RT::VEC, out);
}

// s_waitcnt vmcnt(16 * rounds_after): the loader wave's round rd is complete when at most the 16 loads of
// each later round are outstanding.
__device__ __forceinline__ void wait_loader_round(int rounds_after) {
    switch (rounds_after) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;          // vmcnt(0)
    case 1: __builtin_amdgcn_s_waitcnt(0x0F70 | 0x4000); break; // vmcnt(16)
    case 2: __builtin_amdgcn_s_waitcnt(0x0F70 | 0x8000); break; // vmcnt(32)
    default: __builtin_amdgcn_s_waitcnt(0x0F70 | 0xC000); break; // vmcnt(48)
    }
}

// Resident kernel: bf16, d >= 32, keys and values of the whole (batch, head) held in LDS.  Seven
// compute waves own the query tiles; the eighth wave is the loader.  At the start the loader issues
// every key and value load of the workgroup (four rounds of 8 KiB of keys and 8 KiB of values; loads
// past the sequence go to a 1 KiB sink, so every round is the same 16 loads), while the compute waves
// load only their own query rows.  Then, round by round, the loader waits for its round and releases
// it with a barrier; all eight waves apply phi to its keys in place (one 16-byte chunk per lane, rows
// at or past L zeroed; LION-D only zeroes the padding, in the loader) and the compute waves run the
// round's sub-blocks while later rounds are still in flight.  The load counter is per wave, so the
// compute waves never wait for key/value traffic they do not use yet.
template <int D, int KIND, int QT>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : 4))) full_resident_kernel(FullParams p) {
    using C = FullCfg<D, true>;
    using T = __bf16;
    using RT = typename C::RT;
    constexpr int kRounds = 4;                               // rounds of loads
    constexpr int kRPI = 64 / RT::CPK;                       // rows per 1 KiB load
    constexpr int kRR = 8 * kRPI;                            // rows per round (eight loads of keys)
    static_assert(kRR % kKB == 0, "rounds hold whole sub-blocks");
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = uniform(tid >> 6);
    const int nt = blockDim.x;
    const int ncw = (nt >> 6) - 1;                           // compute waves (the last wave loads)
    const bool loader = wave == ncw;
    const int r = lane & 15, g = lane >> 4;
    const int L = p.L;
    const int Lr = ((L + kKB - 1) / kKB) * kKB;              // rows staged (<= 448, <= kRounds * kRR)
    const int ntiles = (L + 15) / 16;

    const int tile = xcd_tile(blockIdx.x, p.nblocks);
    const int bh = tile / p.nsb;
    const int sb = p.causal ? p.nsb - 1 - tile % p.nsb : tile % p.nsb;
    const int tile0 = sb * p.tiles_per_wg;
    const int tile_end = min(tile0 + p.tiles_per_wg, ntiles);
    const int wtile0 = tile0 + wave * QT;
    const int wave_tiles = loader ? 0 : max(0, min(QT, tile_end - wtile0));

    // LDS: [K rows][V rows][1 KiB sink][E table][fp64 prefix sums]
    T *Kb = reinterpret_cast<T *>(smem);
    T *Vb = Kb + (size_t)Lr * D;
    T *sink = Vb + (size_t)Lr * D;
    float *E = reinterpret_cast<float *>(sink + 512);
    double *A = reinterpret_cast<double *>(E + Lr);          // LION-S: A_t for t < L, then 16 wave totals

    const size_t base = (size_t)bh * L;
    const T *qg = reinterpret_cast<const T *>(p.q) + base * D;
    const T *kg = reinterpret_cast<const T *>(p.k) + base * D;
    const T *vg = reinterpret_cast<const T *>(p.v) + base * D;

    const int t_ref = min(tile0 * 16, L - 1);
    const int keys_used = p.causal ? min(L, tile_end * 16) : L;   // keys any row of the workgroup sees
    const int nr_used = (keys_used + kRR - 1) / kRR;
    // The loader and the compute waves take separate paths with the same barriers (one for the LION-D
    // table, three for LION-S's; per round one for LION-D, two otherwise), so no wait of one path lands
    // on the other.
    if (loader) {
#pragma unroll
        for (int rd = 0; rd < kRounds; ++rd)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = rd * 8 + j;                    // 1 KiB load index within the tile
                const int slot = i * 64 + lane;
                const int row = slot / RT::CPK;
                const int c = (slot % RT::CPK) ^ RT::swz(row);
                const size_t goff = (size_t)min(row, L - 1) * D + c * RT::VEC;
                const bool real = i * kRPI < Lr;
                load_lds16(real ? Vb + (size_t)i * 64 * RT::VEC : sink, vg + goff);
                load_lds16(real ? Kb + (size_t)i * 64 * RT::VEC : sink, kg + goff);
            }
        if constexpr (KIND == kMaskD) lds_barrier();
        if constexpr (KIND == kMaskS) {
            lds_barrier();
            lds_barrier();
            lds_barrier();
        }
        for (int rd = 0; rd < nr_used; ++rd) {
            wait_loader_round(kRounds - 1 - rd);
            if constexpr (KIND == kMaskD) {
                // identity phi: the padding rows (copies of row L - 1) are zeroed
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = rd * 8 + j;
                    if (i * kRPI >= Lr) break;
                    if ((i + 1) * kRPI <= L) continue;
                    const int slot = i * 64 + lane;
                    if (slot / RT::CPK >= L) lds_write16(Kb + (size_t)slot * RT::VEC, u32x4{0u, 0u, 0u, 0u});
                }
                lds_barrier();                                  // round rd is ready
            } else {
                lds_barrier();                                  // round rd has landed
                for (int sl = tid; sl < 512; sl += nt) {        // this lane's share of the phi pass
                    const int slot = rd * 512 + sl;
                    if (slot / RT::CPK < Lr) phi_chunk<D, KIND>(Kb, slot, L);
                }
                lds_barrier();                                  // round rd is ready
            }
        }
        wait_vm_all();   // no load into LDS outlives the workgroup (unused rounds, the sink)
        return;
    }

    // ---- compute waves: query rows, mask exponents relative to the workgroup's first row -------------
    T xr[QT][C::CPL];
    load_query<D, QT, true>(xr, qg, wtile0, wave_tiles, L, r, g);
    float llv = 0.f;
    if constexpr (KIND == kMaskS) llv = p.ll[base + min(tid, L - 1)];   // token tid's log(lambda)
    if constexpr (KIND == kMaskD) {
        const float lg = p.ll[bh % p.H] * kLog2e;
        if (tid < Lr) E[tid] = (float)(min(tid, L - 1) - t_ref) * lg;
        lds_barrier();
    } else if constexpr (KIND == kMaskS) {
        // A_t = sum of log(lambda) over tokens 0..t in fp64: a scan within each compute wave, then the
        // totals of the earlier waves; rows past L take E[L - 1]
        double a = tid < L ? (double)llv : 0.0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double t = __shfl_up(a, o, 64);
            if (lane >= o) a += t;
        }
        if (lane == 63) A[448 + wave] = a;
        lds_barrier();
        for (int w2 = 0; w2 < wave; ++w2) a += A[448 + w2];
        if (tid < L) A[tid] = a;
        lds_barrier();
        if (tid < Lr) E[tid] = (float)((A[min(tid, L - 1)] - A[t_ref]) * 1.4426950408889634);
        lds_barrier();
    }

    const int rw0 = wtile0 * 16;
    const int rwl = min((wtile0 + wave_tiles) * 16, L) - 1;
    float e_first = 0.f, e_last = 0.f;
    if constexpr (KIND != kMaskLit) {
        if (wave_tiles > 0) {
            e_first = uniform(E[rw0]);
            e_last = uniform(E[rwl]);
        }
    }
    FullWave<D, QT, true> w;
    query_frags<D, KIND, QT, true>(w, xr, wtile0, wave_tiles, L, r);
    wave_rows_init<D, KIND, QT, true, false>(w, E, nullptr, wtile0, L, r, e_first, e_last);

    // ---- rounds: compute on round rd once the loader has released it ----------------------------------
    for (int rd = 0; rd < nr_used; ++rd) {
        lds_barrier();
        if constexpr (KIND != kMaskD) {
            for (int sl = tid; sl < 512; sl += nt) {
                const int slot = rd * 512 + sl;
                if (slot / RT::CPK < Lr) phi_chunk<D, KIND>(Kb, slot, L);
            }
            lds_barrier();
        }
        if (wave_tiles == 0) continue;
#pragma unroll
        for (int h = 0; h < kRR / kKB; ++h) {
            const int j0 = rd * kRR + h * kKB;
            if (j0 >= L) break;
            if (p.causal && j0 > rwl) break;
            const int region = subblock_region<KIND, false>(j0, rw0, rwl, p.causal);
            full_subblock<D, KIND, QT, true, false>(w, Kb, Vb, j0, j0, E, nullptr, region, e_first, e_last, wtile0,
                                                   wave_tiles, p.causal, r, g);
        }
    }
    full_epilogue<D, QT, true>(w, p, base, wtile0, wave_tiles, L, r, g);
}

// Launch shape of the full form: which kernel, query tiles per wave, waves per workgroup, workgroups
// per (batch, head), query tiles per workgroup, keys per stage (resident: the padded sequence), stage
// buffers, and the LDS the kernel asks for.
struct FullShape {
    bool resident;
    int qt, nw, nsb, tiles_per_wg, sk, nbuf;
    size_t lds;
};

FullShape full_shape(const AttnArgs &a) {
    const bool two = a.order != nullptr && a.kind != kMaskLit;
    const int ntiles = (a.L + 15) / 16;
    const long bhs = (long)a.B * a.H;
    const bool bf16c = !a.fp32c;                     // bf16 arithmetic
    const size_t esz = bf16c ? 2 : 4;                // staged K and V elements
    const size_t per_key = 2 * (size_t)a.d * esz;   // K and V bytes of one key
    const int lr = ((a.L + kKB - 1) / kKB) * kKB;
    FullShape sh;
    // resident kernel: one workgroup per (batch, head) (two past 15 query tiles) when the whole grid is
    // on the chip at once; larger grids overlap workgroups' loads with others' compute in the streaming
    // kernel (measured: B64 H3 L197 10.7 vs 12.1 us; B64 H12 L197 37.7 vs 33.5 us)
    const int nsb_res = (ntiles + 14) / 15;
    sh.resident = bf16c && a.d >= 32 && !two && (size_t)lr * per_key <= kStageBytes && lr <= 448 &&
                  bhs * nsb_res <= kResidentMaxGrid;
    if (sh.resident) {
        // one compute wave per query tile plus the loader; the compute waves also cover the staged rows
        // (the LION-S scan and the exponent table take one row per compute lane)
        sh.qt = 1;
        sh.tiles_per_wg = (ntiles + nsb_res - 1) / nsb_res;
        sh.nsb = (ntiles + sh.tiles_per_wg - 1) / sh.tiles_per_wg;
        sh.nw = std::max(sh.tiles_per_wg, (lr + 63) / 64) + 1;
        sh.sk = lr;
        sh.nbuf = 1;
        size_t lds = (size_t)lr * per_key + 1024;
        if (a.kind != kMaskLit) lds += (size_t)lr * 4;
        if (a.kind == kMaskS) lds += (448 + 16) * 8;
        sh.lds = lds;
        return sh;
    }
    int qt = 1;
    if (bf16c) {
        // largest tile count per wave that still gives >= 2 waves per SIMD (256 CUs x 4 SIMDs)
        const int cand[3] = {a.d == 128 ? 1 : 4, 2, 1};
        for (int c : cand) {
            qt = c;
            if (bhs * ((ntiles + c - 1) / c) >= 2048) break;
        }
    }
    const int wtiles = (ntiles + qt - 1) / qt;      // waves with query tiles per (batch, head)
    sh.qt = qt;
    sh.nw = wtiles >= 6 ? 8 : 4;
    sh.nsb = (ntiles + sh.nw * qt - 1) / (sh.nw * qt);
    sh.tiles_per_wg = sh.nw * qt;
    auto lds_of = [&](int sk, int nbuf) {
        const int Lpad = ((a.L + sk - 1) / sk) * sk;
        size_t lds = (size_t)nbuf * sk * per_key;
        if (a.kind != kMaskLit) lds += (size_t)Lpad * 4 * (two ? 2 : 1);
        if (a.kind == kMaskS) lds += (size_t)sh.nw * 64 * 8;
        return lds;
    };
    if ((size_t)lr * per_key <= kStageBytes) {
        sh.sk = lr;                                  // the whole sequence is one stage
        sh.nbuf = 1;
    } else {
        sh.sk = (int)(kStageBytes / 2 / per_key);     // double-buffered stages
        sh.nbuf = 2;
        // long sequences: stages twice that size where the LDS holds them (half the workgroup
        // barriers; B8 H12 L4097: 609 -> 581 us)
        if (a.L >= 1024 && lds_of(2 * sh.sk, 2) <= kLdsPerWorkgroup) sh.sk *= 2;
    }
    sh.lds = lds_of(sh.sk, sh.nbuf);
    return sh;
}

FullParams full_params(const AttnArgs &a, const FullShape &sh) {
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
    p.tiles_per_wg = sh.tiles_per_wg;
    p.nblocks = a.B * a.H * sh.nsb;
    p.sk = sh.sk;
    p.nbuf = sh.nbuf;
    p.causal = a.causal ? 1 : 0;
    p.order = a.order;
    return p;
}

template <typename K>
hipError_t launch_kernel(K kernel, const FullParams &p, const FullShape &sh, hipStream_t stream) {
    if (sh.lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)sh.lds);
    hipLaunchKernelGGL(kernel, dim3(p.nblocks), dim3(sh.nw * 64), sh.lds, stream, p);
    return hipGetLastError();
}

template <int D, int KIND, int QT, bool BF16, bool TWO, bool INB>
hipError_t launch_full_t(const AttnArgs &a, hipStream_t stream, const FullShape &sh) {
    const FullParams p = full_params(a, sh);
    if constexpr (BF16 && !TWO && D >= 32 && QT == 1) {
        if (sh.resident) return launch_kernel(&full_resident_kernel<D, KIND, QT>, p, sh, stream);
    }
    return launch_kernel(&full_kernel<D, KIND, QT, BF16, TWO, INB>, p, sh, stream);
}

template <int D, int KIND, bool BF16, bool TWO, bool INB>
hipError_t dispatch_qt2(const AttnArgs &a, hipStream_t stream) {
    const FullShape sh = full_shape(a);
    if constexpr (BF16) {
        if constexpr (D != 128) {
            if (sh.qt == 4) return launch_full_t<D, KIND, 4, BF16, TWO, INB>(a, stream, sh);
            if (sh.qt == 2) return launch_full_t<D, KIND, 2, BF16, TWO, INB>(a, stream, sh);
        }
    }
    return launch_full_t<D, KIND, 1, BF16, TWO, INB>(a, stream, sh);
}

// the two-order variant exists for the kinds with a decay (LIT's mask is all ones in any order), in
// the input type's own arithmetic
template <int D, int KIND, bool BF16, bool INB>
hipError_t dispatch_qt(const AttnArgs &a, hipStream_t stream) {
    if constexpr (KIND != kMaskLit && BF16 == INB) {
        if (a.order) return dispatch_qt2<D, KIND, BF16, true, INB>(a, stream);
    }
    return dispatch_qt2<D, KIND, BF16, false, INB>(a, stream);
}

template <int D, bool BF16, bool INB>
hipError_t dispatch_kind(const AttnArgs &a, hipStream_t stream) {
    switch (a.kind) {
    case kMaskLit: return dispatch_qt<D, kMaskLit, BF16, INB>(a, stream);
    case kMaskD: return dispatch_qt<D, kMaskD, BF16, INB>(a, stream);
    default: return dispatch_qt<D, kMaskS, BF16, INB>(a, stream);
    }
}

// BF16: bf16 arithmetic; INB: bf16 inputs (with BF16 false: upcast exactly for fp32 arithmetic)
template <bool BF16, bool INB>
hipError_t dispatch_d(const AttnArgs &a, hipStream_t stream) {
    switch (a.d) {
    case 16: return dispatch_kind<16, BF16, INB>(a, stream);
    case 32: return dispatch_kind<32, BF16, INB>(a, stream);
    case 64: return dispatch_kind<64, BF16, INB>(a, stream);
    default: return dispatch_kind<128, BF16, INB>(a, stream);
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
    if (!a.fp32c) return dispatch_d<true, true>(a, stream);
    return a.in_bf16 ? dispatch_d<false, true>(a, stream) : dispatch_d<false, false>(a, stream);
}

}  // namespace lion
