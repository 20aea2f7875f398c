// lion_full_bwd.hip -- backward pass of the full (attention) form of LION.
//
// LION trains with the attention form ("LION: A bidirectional framework that trains like a Transformer
// and infers like an RNN", OpenReview abstract; reply "Concern 1", Theorem 3.3 Eq. 25).  For
//   s_ij = phi(q_i).phi(k_j),  p_ij = M_ij s_ij,  den_i = sum_j p_ij + eps,  y_i = sum_j p_ij v_j / den_i
// and an incoming gradient dy, the chain rule gives (delta_i = dy_i.y_i / den_i)
//   dp_ij = (dy_i.v_j) / den_i - delta_i
//   dv_j  = sum_i (p_ij / den_i) dy_i
//   dphi(q_i) = sum_j M_ij dp_ij phi(k_j),   dphi(k_j) = sum_i M_ij dp_ij phi(q_i)
//   dq, dk  = the Jacobian of phi (transposed) applied to those
// and, through M_ij = exp(A_max(i,j) - A_min(i,j)) with A the prefix sums of log(lambda),
//   dA_t = sum over pairs with max(i,j) = t of w_ij - sum over pairs with min(i,j) = t of w_ij,
//   w_ij = dp_ij p_ij,   dlog(lambda_u) = sum_{t >= u} dA_t   (u >= 1; lambda_0 never enters).
//
// Three launches, none of which forms an L x L matrix:
//   dq:   a wave per one or two 16-query tiles streams the keys and values (LDS stages, as in the forward kernel):
//         S^T = phi(K) phi(Q)^T and (dy v^T)^T = V dY^T on matrix cores, the masked dS^T in registers,
//         then dphi(Q)^T += phi(K)^T dS^T (the D layout of the first products is the B layout of this
//         one, as in the forward).  It also writes delta and the row half of dA.
//   dk/dv: a wave per one or two 16-key tiles streams phi(Q) and dY the same way: S and dY V^T with keys as the
//         column index, then dV^T += dY^T (P / den) and dphi(K)^T += phi(Q)^T dS, and the column half
//         of dA.
//   dlog(lambda): LION-S a reverse prefix sum of dA per (batch, head); LION-D sum_t t dA_t over every
//         batch entry of a head (per-(batch, head) sums first, then a head's batch entries).
// In both gradient kernels a sub-block that lies wholly on one side of a wave's rows forms the mask as
// a row factor times a column factor (both at most 1) instead of one exponential per score, as the
// forward does.
// Causal variant: M_ij = 0 for j > i (a constant), so those pairs are skipped or zeroed.
// A sequence of at most 256 tokens with d <= 64 takes another route (launch_full_bwd): it is one chunk
// of the chunkwise backward's main kernel (lion_chunk_bwd_mfma.hip), which stages the whole sequence
// once and forms both sides' products there, with no states.
#include <type_traits>

#include "lion_device.h"
#include "lion_internal.h"
#include "lion_mask.h"
#include "lion_stage.h"
#include "lion_bwd_tiles.h"

namespace lion {
namespace {

constexpr size_t kStageBytes = 64 * 1024;     // bytes of the two streamed operands per stage

struct BwdParams {
    const __bf16 *q, *k, *v;
    const float *ll;
    int H, L;
    const __bf16 *y, *dy;
    const float *den;          // the forward's divisors (row sum + eps)
    void *dq, *dk, *dv;
    int g_bf16;                // gradients stored as bf16 (else fp32)
    float *delta, *da_row, *da_col;   // workspace, [B*H*L] each
    float *dll;
    int nsb;                   // workgroups per (batch, head)
    int nblocks;               // grid size
    int sk;                    // rows per stage (multiple of 32)
    int nbuf;                  // 1: the whole sequence is one stage; 2: double-buffered stages
    int causal;
};

// ================================ dq ==================================================================
// TT query tiles per wave: the key/value fragments a sub-block reads from LDS serve all of them.
template <int D, int KIND, int TT>
__global__ void __launch_bounds__(512) bwd_dq_kernel(BwdParams p) {
    using T = __bf16;
    constexpr int NS = D / 32, NCT = D / 16;
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
    // causal: workgroups of later rows (more keys) first
    const int sb = p.causal ? p.nsb - 1 - tile % p.nsb : tile % p.nsb;
    const int wt0 = (sb * nw + wave) * TT;         // this wave's first query tile
    const bool active = wt0 < ntiles;

    T *Kb = reinterpret_cast<T *>(smem);
    T *Vb = Kb + (size_t)p.nbuf * SK * D;
    float *E = reinterpret_cast<float *>(Vb + (size_t)p.nbuf * SK * D);
    double *scan_sh = reinterpret_cast<double *>(E + (KIND == kMaskLit ? 0 : Lpad));

    const size_t base = (size_t)bh * L;
    const T *kg = p.k + base * D;
    const T *vg = p.v + base * D;
    stage_rows<D, T>(Kb, kg, 0, SK, L, wave, nw, lane);
    stage_rows<D, T>(Vb, vg, 0, SK, L, wave, nw, lane);
    if constexpr (KIND != kMaskLit)
        build_exponents<KIND>(E, scan_sh, p.ll, bh, p.H, L, Lpad, min(sb * nw * TT * 16, L - 1), tid, nt);

    // this lane's query row i of each tile: phi(q), dy fragments; den, delta
    int irow[TT];
    bool ok[TT];
    bf16x8 qf[TT][NS], dyf[TT][NS];
    float inv_den[TT], delta_i[TT], Ei[TT], rowterm[TT];
    f32x4 acc[TT][NCT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int i = (wt0 + tt) * 16 + r;
        irow[tt] = i;
        ok[tt] = active && i < L;
        const int ic = min(i, L - 1);
        row_frags<D, KIND, true>(p.q + (base + ic) * D, ok[tt], qf[tt]);
        row_frags<D, KIND, false>(p.dy + (base + ic) * D, ok[tt], dyf[tt]);
        float dot = 0.f;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const bf16x8 yv = __builtin_bit_cast(bf16x8, ld16(p.y + (base + ic) * D + 8 * (4 * st + g)));
#pragma unroll
            for (int e = 0; e < 8; ++e) dot += (float)dyf[tt][st][e] * (float)yv[e];
        }
        dot += __shfl_xor(dot, 16, 64);
        dot += __shfl_xor(dot, 32, 64);
        const float den_i = ok[tt] ? p.den[base + ic] : 1.f;
        inv_den[tt] = 1.f / den_i;
        delta_i[tt] = ok[tt] ? dot * inv_den[tt] : 0.f;
        if (ok[tt] && g == 0) p.delta[base + i] = delta_i[tt];
        Ei[tt] = KIND != kMaskLit ? E[ic] : 0.f;
        rowterm[tt] = 0.f;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[tt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int wlast = min((wt0 + TT) * 16, L) - 1;   // the wave's last query row
    // Separable mask for 32-key sub-blocks wholly before or after the wave's rows (first row w0, last
    // wlast; the exponents decrease along the sequence): M_ij = exp2(E_i - E_w0) exp2(E_w0 - E_j) for
    // keys before, exp2(E_wl - E_i) exp2(E_j - E_wl) for keys after, every factor at most 1.  The row
    // factor is per tile; a key's column factor is the same for the 16 lanes of a row, so lane r < 8
    // computes that of key j0 + 16 (r / 4) + 4g + r % 4 and the others take it by DPP row broadcast.
    const int w0 = wt0 * 16;
    const float e_first = KIND != kMaskLit && active ? uniform(E[min(w0, L - 1)]) : 0.f;
    const float e_last = KIND != kMaskLit && active ? uniform(E[max(wlast, 0)]) : 0.f;
    float rowf_b[TT], rowf_a[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        rowf_b[tt] = KIND != kMaskLit ? fast_exp2(Ei[tt] - e_first) : 1.f;
        rowf_a[tt] = KIND != kMaskLit ? fast_exp2(e_last - Ei[tt]) : 1.f;
    }

    // causal: stages wholly after the workgroup's last query row are never needed
    const int nst_used = p.causal ? min(nst, (min((sb + 1) * nw * TT * 16, L) - 1) / SK + 1) : nst;
    for (int s = 0; s < nst_used; ++s) {
        const int buf = p.nbuf == 1 ? 0 : (s & 1);
        T *kbuf = Kb + (size_t)buf * SK * D;
        const T *vbuf = Vb + (size_t)buf * SK * D;
        wait_vm_all();
        __syncthreads();                                   // stage s is in LDS; buffer s+1 is free
        if (s + 1 < nst_used) {
            const int nb = (s + 1) & 1;
            stage_rows<D, T>(Kb + (size_t)nb * SK * D, kg, (s + 1) * SK, SK, L, wave, nw, lane);
            stage_rows<D, T>(Vb + (size_t)nb * SK * D, vg, (s + 1) * SK, SK, L, wave, nw, lane);
        }
        phi_stage<D, KIND>(kbuf, SK, min(SK, L - s * SK), tid, nt);
        __syncthreads();
        if (!active) continue;

        for (int h = 0; h < SK / kKB; ++h) {
            const int j0 = s * SK + h * kKB;
            if (j0 >= L) break;
            if (p.causal && j0 > wlast) break;
            // fragments shared by the wave's tiles: key and value rows (A operands of S^T and of
            // (dY V^T)^T), transposed keys (A operand of dphi(Q)^T), the keys' mask exponents.  With
            // two tiles they are read once up front; with one, where they are used (fewer registers)
            bf16x8 kr[2][NS], vr[2][NS], kt[NCT];
            if constexpr (TT > 1) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int st = 0; st < NS; ++st) {
                        kr[t][st] = rows_frag<D>(kbuf, h, t, st, r, g);
                        vr[t][st] = rows_frag<D>(vbuf, h, t, st, r, g);
                    }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) kt[ct] = tr_frag<D>(kbuf, h, ct, r, g);
            }
            auto krow = [&](int t, int st) { return TT > 1 ? kr[t][st] : rows_frag<D>(kbuf, h, t, st, r, g); };
            auto vrow = [&](int t, int st) { return TT > 1 ? vr[t][st] : rows_frag<D>(vbuf, h, t, st, r, g); };
            auto ktr = [&](int ct) { return TT > 1 ? kt[ct] : tr_frag<D>(kbuf, h, ct, r, g); };
            // region of this sub-block relative to the wave's rows (wave-uniform): 0 overlap, 1 every key
            // before every row, 2 every key after every row
            const int region = j0 + kKB - 1 < w0 ? 1 : j0 > wlast ? 2 : 0;
            f32x4 ej[2];
            float cl = 1.f;
#pragma unroll
            for (int t = 0; t < 2; ++t) ej[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (KIND != kMaskLit) {
                if (region == 0) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) ej[t] = *reinterpret_cast<const f32x4 *>(E + j0 + 16 * t + 4 * g);
                } else {
                    const float e = E[j0 + 16 * ((r >> 2) & 1) + 4 * g + (r & 3)];
                    cl = fast_exp2(region == 1 ? e_first - e : e - e_last);
                }
            }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                if (wt0 + tt >= ntiles) break;
                f32x4 sacc[2], dpacc[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    sacc[t] = dpacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < NS; ++st) {
                        sacc[t] = mfma_bf16(krow(t, st), qf[tt][st], sacc[t]);
                        dpacc[t] = mfma_bf16(vrow(t, st), dyf[tt][st], dpacc[t]);
                    }
                }
                // element (t, e): key j = j0 + 16 t + 4 g + e, query irow[tt]
                const int i = irow[tt];
                bf16x8 dsf;
                if (region == 0) {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int j = j0 + 16 * t + 4 * g + e;
                            float m = KIND != kMaskLit ? fast_exp2(-__builtin_fabsf(Ei[tt] - ej[t][e])) : 1.f;
                            if (p.causal && j > i) m = 0.f;
                            const float dp = dpacc[t][e] * inv_den[tt] - delta_i[tt];
                            const float w = dp * (sacc[t][e] * m);
                            rowterm[tt] += j < i ? w : (j > i ? -w : 0.f);
                            dsf[4 * t + e] = f2bf(dp * m);
                        }
                } else {
                    // every key on one side of the row (keys after the rows never reach here when causal)
                    const float rowf = region == 1 ? rowf_b[tt] : rowf_a[tt];
                    float wsum = 0.f;
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float m = KIND != kMaskLit ? bwd_bcast16(cl, 4 * t + e) * rowf : 1.f;
                            const float dp = dpacc[t][e] * inv_den[tt] - delta_i[tt];
                            wsum += dp * (sacc[t][e] * m);
                            dsf[4 * t + e] = f2bf(dp * m);
                        }
                    rowterm[tt] += region == 1 ? wsum : -wsum;
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) acc[tt][ct] = mfma_bf16(ktr(ct), dsf, acc[tt][ct]);
            }
        }
    }
    if (!active) return;

#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        // rows of dA (pairs where this row is the later / earlier index), then dq through phi
        float rt = rowterm[tt];
        rt += __shfl_xor(rt, 16, 64);
        rt += __shfl_xor(rt, 32, 64);
        const int i = irow[tt];
        const int ic = min(i, L - 1);
        if (KIND != kMaskLit && ok[tt] && g == 0) p.da_row[base + i] = rt;
        // acc[tt][ct][e] = dphi(q_i) at channel 16 ct + 4 g + e
        float x[NCT][4];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const bf16x4 q4 = *reinterpret_cast<const bf16x4 *>(p.q + (base + ic) * D + 16 * ct + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[ct][e] = (float)q4[e];
        }
        phi_backward<D, KIND>(x, acc[tt]);
        if (ok[tt]) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                store4(p.dq, p.g_bf16, (base + i) * D + 16 * ct + 4 * g, acc[tt][ct]);
        }
    }
}

// ================================ dk, dv ==============================================================
// TT key tiles per wave: the query and dY fragments a sub-block reads from LDS serve all of them.
template <int D, int KIND, int TT>
__global__ void __launch_bounds__(512) bwd_dkv_kernel(BwdParams p) {
    using T = __bf16;
    constexpr int NS = D / 32, NCT = D / 16;
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
    // causal: workgroups of earlier keys (more queries) first
    const int sb = tile % p.nsb;
    const int wt0 = (sb * nw + wave) * TT;         // this wave's first key tile
    const bool active = wt0 < ntiles;

    // LDS: [phi(Q) stages][dY stages][E][den][delta][scan scratch]
    T *Qb = reinterpret_cast<T *>(smem);
    T *Gb = Qb + (size_t)p.nbuf * SK * D;
    float *E = reinterpret_cast<float *>(Gb + (size_t)p.nbuf * SK * D);
    float *denT = E + (KIND == kMaskLit ? 0 : Lpad);
    float *dlT = denT + Lpad;
    double *scan_sh = reinterpret_cast<double *>(dlT + Lpad);

    const size_t base = (size_t)bh * L;
    const T *qg = p.q + base * D;
    const T *gg = p.dy + base * D;
    // causal: stages wholly before the workgroup's first key row are never needed
    const int s_begin = p.causal ? min(sb * nw * TT * 16, L - 1) / SK : 0;
    stage_rows<D, T>(Qb + (size_t)(p.nbuf == 1 ? 0 : (s_begin & 1)) * SK * D, qg, s_begin * SK, SK, L, wave, nw, lane);
    stage_rows<D, T>(Gb + (size_t)(p.nbuf == 1 ? 0 : (s_begin & 1)) * SK * D, gg, s_begin * SK, SK, L, wave, nw, lane);
    for (int t = tid; t < Lpad; t += nt) {
        denT[t] = t < L ? p.den[base + t] : 1.f;
        dlT[t] = t < L ? p.delta[base + t] : 0.f;
    }
    if constexpr (KIND != kMaskLit)
        build_exponents<KIND>(E, scan_sh, p.ll, bh, p.H, L, Lpad, min(sb * nw * TT * 16, L - 1), tid, nt);

    // this lane's key row j of each tile: phi(k), v fragments
    int jrow[TT];
    bool ok[TT];
    bf16x8 kf[TT][NS], vf[TT][NS];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int j = (wt0 + tt) * 16 + r;
        jrow[tt] = j;
        ok[tt] = active && j < L;
        const int jc = min(j, L - 1);
        row_frags<D, KIND, true>(p.k + (base + jc) * D, ok[tt], kf[tt]);
        row_frags<D, KIND, false>(p.v + (base + jc) * D, ok[tt], vf[tt]);
    }
    __syncthreads();   // tables written (build_exponents ends with a barrier only for D and S)
    float Ej[TT], colterm[TT];
    f32x4 acck[TT][NCT], accv[TT][NCT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        Ej[tt] = KIND != kMaskLit ? E[min(jrow[tt], L - 1)] : 0.f;
        colterm[tt] = 0.f;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acck[tt][ct] = accv[tt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int wfirst = wt0 * 16;                     // the wave's first key row
    const int wlast = min((wt0 + TT) * 16, L) - 1;   // and its last
    // Separable mask for 32-query sub-blocks wholly before or after the wave's keys (the exponents
    // decrease along the sequence): M_ij = exp2(E_j - E_wf) exp2(E_wf - E_i) for queries before,
    // exp2(E_wl - E_j) exp2(E_i - E_wl) for queries after, every factor at most 1.  The key factor is per
    // tile (formed per sub-block: registers); lane r < 8 computes the factor of query
    // i0 + 16 (r / 4) + 4g + r % 4 and the row's other lanes take it by DPP row broadcast.
    const float e_first = KIND != kMaskLit && active ? uniform(E[min(wfirst, L - 1)]) : 0.f;
    const float e_last = KIND != kMaskLit && active ? uniform(E[max(wlast, 0)]) : 0.f;

    for (int s = s_begin; s < nst; ++s) {
        const int buf = p.nbuf == 1 ? 0 : (s & 1);
        T *qbuf = Qb + (size_t)buf * SK * D;
        const T *gbuf = Gb + (size_t)buf * SK * D;
        wait_vm_all();
        __syncthreads();
        if (s + 1 < nst) {
            const int nb = (s + 1) & 1;
            stage_rows<D, T>(Qb + (size_t)nb * SK * D, qg, (s + 1) * SK, SK, L, wave, nw, lane);
            stage_rows<D, T>(Gb + (size_t)nb * SK * D, gg, (s + 1) * SK, SK, L, wave, nw, lane);
        }
        phi_stage<D, KIND>(qbuf, SK, min(SK, L - s * SK), tid, nt);
        __syncthreads();
        if (!active) continue;

        for (int h = 0; h < SK / kKB; ++h) {
            const int i0 = s * SK + h * kKB;
            if (i0 >= L) break;
            if (p.causal && i0 + kKB - 1 < wfirst) continue;   // every query before every key
            // fragments shared by the wave's tiles: phi(Q) and dY rows, their transposes (read once up
            // front with two tiles, where they are used with one), and the queries' divisors, deltas
            // and mask exponents
            bf16x8 qr[2][NS], gr[2][NS], qt[NCT], gt[NCT];
            if constexpr (TT > 1) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int st = 0; st < NS; ++st) {
                        qr[t][st] = rows_frag<D>(qbuf, h, t, st, r, g);
                        gr[t][st] = rows_frag<D>(gbuf, h, t, st, r, g);
                    }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    gt[ct] = tr_frag<D>(gbuf, h, ct, r, g);
                    qt[ct] = tr_frag<D>(qbuf, h, ct, r, g);
                }
            }
            auto qrow = [&](int t, int st) { return TT > 1 ? qr[t][st] : rows_frag<D>(qbuf, h, t, st, r, g); };
            auto grow = [&](int t, int st) { return TT > 1 ? gr[t][st] : rows_frag<D>(gbuf, h, t, st, r, g); };
            auto qtr = [&](int ct) { return TT > 1 ? qt[ct] : tr_frag<D>(qbuf, h, ct, r, g); };
            auto gtr = [&](int ct) { return TT > 1 ? gt[ct] : tr_frag<D>(gbuf, h, ct, r, g); };
            // region of this sub-block relative to the wave's keys (wave-uniform): 0 overlap, 1 every query
            // before every key (never reached when causal), 2 every query after every key
            const int region = i0 + kKB - 1 < wfirst ? 1 : i0 > wlast ? 2 : 0;
            float cl = 1.f;
            if constexpr (KIND != kMaskLit) {
                if (region != 0) {
                    const float e = E[i0 + 16 * ((r >> 2) & 1) + 4 * g + (r & 3)];
                    cl = fast_exp2(region == 1 ? e_first - e : e - e_last);
                }
            }
            // the queries' 1/den, delta and mask exponents (elements 4 g + e of half t; the exponents only
            // where the sub-block overlaps the wave's keys)
            auto query_vals = [&](int t, f32x4 &inv, f32x4 &dl, f32x4 &ei) {
                const int ib = i0 + 16 * t + 4 * g;
                const f32x4 dn = *reinterpret_cast<const f32x4 *>(denT + ib);
#pragma unroll
                for (int e = 0; e < 4; ++e) inv[e] = __builtin_amdgcn_rcpf(dn[e]);
                dl = *reinterpret_cast<const f32x4 *>(dlT + ib);
                ei = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (KIND != kMaskLit)
                    if (region == 0) ei = *reinterpret_cast<const f32x4 *>(E + ib);
            };
            f32x4 inv2[2], dl2[2], ei2[2];
            if constexpr (TT > 1) {
#pragma unroll
                for (int t = 0; t < 2; ++t) query_vals(t, inv2[t], dl2[t], ei2[t]);
            }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                if (wt0 + tt >= ntiles) break;
                f32x4 sacc[2], dpacc[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    sacc[t] = dpacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < NS; ++st) {
                        sacc[t] = mfma_bf16(qrow(t, st), kf[tt][st], sacc[t]);
                        dpacc[t] = mfma_bf16(grow(t, st), vf[tt][st], dpacc[t]);
                    }
                }
                // element (t, e): query i = i0 + 16 t + 4 g + e, key jrow[tt]
                const int j = jrow[tt];
                bf16x8 pf, dsf;
                float wsum = 0.f;
                const float keyf = KIND != kMaskLit && region != 0
                                       ? fast_exp2(region == 1 ? Ej[tt] - e_first : e_last - Ej[tt]) : 1.f;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    f32x4 inv, dl, ei;
                    if constexpr (TT > 1) {
                        inv = inv2[t];
                        dl = dl2[t];
                        ei = ei2[t];
                    } else {
                        query_vals(t, inv, dl, ei);
                    }
                    if (region == 0) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int i = i0 + 16 * t + 4 * g + e;
                            float m = KIND != kMaskLit ? fast_exp2(-__builtin_fabsf(ei[e] - Ej[tt])) : 1.f;
                            if (p.causal && j > i) m = 0.f;
                            const float pm = sacc[t][e] * m;
                            const float dp = dpacc[t][e] * inv[e] - dl[e];
                            const float w = dp * pm;
                            colterm[tt] += i < j ? w : (i > j ? -w : 0.f);
                            pf[4 * t + e] = f2bf(pm * inv[e]);
                            dsf[4 * t + e] = f2bf(dp * m);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float m = KIND != kMaskLit ? bwd_bcast16(cl, 4 * t + e) * keyf : 1.f;
                            const float pm = sacc[t][e] * m;
                            const float dp = dpacc[t][e] * inv[e] - dl[e];
                            wsum += dp * pm;
                            pf[4 * t + e] = f2bf(pm * inv[e]);
                            dsf[4 * t + e] = f2bf(dp * m);
                        }
                    }
                }
                if (region != 0) colterm[tt] += region == 1 ? wsum : -wsum;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    accv[tt][ct] = mfma_bf16(gtr(ct), pf, accv[tt][ct]);
                    acck[tt][ct] = mfma_bf16(qtr(ct), dsf, acck[tt][ct]);
                }
            }
        }
    }
    if (!active) return;

#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        float ctm = colterm[tt];
        ctm += __shfl_xor(ctm, 16, 64);
        ctm += __shfl_xor(ctm, 32, 64);
        const int j = jrow[tt];
        const int jc = min(j, L - 1);
        if (KIND != kMaskLit && ok[tt] && g == 0) p.da_col[base + j] = ctm;
        float x[NCT][4];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const bf16x4 k4 = *reinterpret_cast<const bf16x4 *>(p.k + (base + jc) * D + 16 * ct + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[ct][e] = (float)k4[e];
        }
        phi_backward<D, KIND>(x, acck[tt]);
        if (ok[tt]) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                store4(p.dk, p.g_bf16, (base + j) * D + 16 * ct + 4 * g, acck[tt][ct]);
                store4(p.dv, p.g_bf16, (base + j) * D + 16 * ct + 4 * g, accv[tt][ct]);
            }
        }
    }
}

// ================================ dlog(lambda) ========================================================
constexpr int kDllThreads = 256;

// LION-S: one workgroup per (batch, head): dll_u = sum_{t >= u} (da_row_t + da_col_t) for u >= 1 (fp64),
// dll_0 = 0.
__global__ void __launch_bounds__(kDllThreads) bwd_dll_s_kernel(BwdParams p) {
    __shared__ double sh[kDllThreads];
    __shared__ double total;
    const int tid = threadIdx.x, L = p.L;
    const size_t base = (size_t)blockIdx.x * L;
    const int seg = (L + kDllThreads - 1) / kDllThreads;
    const int t0 = tid * seg, t1 = min(t0 + seg, L);
    double s = 0.0;
    for (int t = t0; t < t1; ++t) s += (double)p.da_row[base + t] + (double)p.da_col[base + t];
    const double excl = block_excl_scan(s, sh, tid, kDllThreads);
    if (tid == kDllThreads - 1) total = excl + s;
    __syncthreads();
    double run = excl;   // sum of dA over u < t
    for (int t = t0; t < t1; ++t) {
        p.dll[base + t] = t == 0 ? 0.f : (float)(total - run);
        run += (double)p.da_row[base + t] + (double)p.da_col[base + t];
    }
}

// LION-D: dll_h = sum over batch entries and tokens of t (da_row_t + da_col_t), in two launches so the
// token sums spread over every (batch, head) rather than one workgroup per head.  The first forms the
// fp64 sum of one (batch, head) row and leaves it as two floats (hi, lo) in element 0 of its da_row and
// da_col rows (token 0 contributes nothing, and every read of the row precedes the barriers of the
// reduction); the second adds a head's B partials.
__global__ void __launch_bounds__(kDllThreads) bwd_dll_d_rows_kernel(BwdParams p) {
    __shared__ double sh[kDllThreads];
    const int tid = threadIdx.x, L = p.L;
    const size_t base = (size_t)blockIdx.x * L;
    double s = 0.0;
    for (int t = tid; t < L; t += kDllThreads) s += (double)t * ((double)p.da_row[base + t] + (double)p.da_col[base + t]);
    sh[tid] = s;
    __syncthreads();
    for (int o = kDllThreads / 2; o > 0; o >>= 1) {
        if (tid < o) sh[tid] += sh[tid + o];
        __syncthreads();
    }
    if (tid == 0) {
        const float hi = (float)sh[0];
        p.da_row[base] = hi;
        p.da_col[base] = (float)(sh[0] - (double)hi);
    }
}

__global__ void __launch_bounds__(kDllThreads) bwd_dll_d_kernel(BwdParams p, int B) {
    // one workgroup per head; its threads take the batch entries' partials in parallel
    __shared__ double sh[kDllThreads];
    const int tid = threadIdx.x, h = blockIdx.x;
    double s = 0.0;
    for (int b = tid; b < B; b += kDllThreads) {
        const size_t base = ((size_t)b * p.H + h) * p.L;
        s += (double)p.da_row[base] + (double)p.da_col[base];
    }
    sh[tid] = s;
    __syncthreads();
    for (int o = kDllThreads / 2; o > 0; o >>= 1) {
        if (tid < o) sh[tid] += sh[tid + o];
        __syncthreads();
    }
    if (tid == 0) p.dll[h] = (float)sh[0];
}

// LION-D from partials already summed over the tokens: four floats per (batch, head), two hi/lo pairs
// (one per half of dA); one workgroup per head adds its B entries.
__global__ void __launch_bounds__(kDllThreads) bwd_dll_d_parts_kernel(const float *part, float *dll, int B, int H) {
    __shared__ double sh[kDllThreads];
    const int tid = threadIdx.x, h = blockIdx.x;
    double s = 0.0;
    for (int b = tid; b < B; b += kDllThreads) {
        const float *q = part + ((size_t)b * H + h) * 4;
        s += ((double)q[0] + (double)q[1]) + ((double)q[2] + (double)q[3]);
    }
    sh[tid] = s;
    __syncthreads();
    for (int o = kDllThreads / 2; o > 0; o >>= 1) {
        if (tid < o) sh[tid] += sh[tid + o];
        __syncthreads();
    }
    if (tid == 0) dll[h] = (float)sh[0];
}

// ================================ host side ===========================================================
struct BwdShape {
    int tt, nw, nsb, sk, nbuf;
    size_t lds_dq, lds_dkv;
};

BwdShape bwd_shape(const BwdArgs &a) {
    const int ntiles = (a.L + 15) / 16;
    BwdShape sh;
    sh.nw = ntiles >= 6 ? 8 : 4;
    // two tiles per wave (the fragments a sub-block reads from LDS serve both) from 32 tiles on;
    // shorter sequences keep one (B64 H12 L197: 125 vs 136 us; B32 H16 L512: 349 vs 336 us; B8 H12
    // L4097: 3776 vs 2734 us); d = 128 keeps one (registers)
    sh.tt = a.d != 128 && ntiles >= 32 ? 2 : 1;
    sh.nsb = (ntiles + sh.tt * sh.nw - 1) / (sh.tt * sh.nw);
    const size_t per_row = 2 * (size_t)a.d * 2;      // two bf16 rows per streamed position
    const int lr = ((a.L + kKB - 1) / kKB) * kKB;
    if ((size_t)lr * per_row <= kStageBytes) {
        sh.sk = lr;
        sh.nbuf = 1;
    } else {
        sh.sk = (int)(kStageBytes / 2 / per_row);
        sh.nbuf = 2;
    }
    const int Lpad = ((a.L + sh.sk - 1) / sh.sk) * sh.sk;
    size_t lds = (size_t)sh.nbuf * sh.sk * per_row;
    if (a.kind != kMaskLit) lds += (size_t)Lpad * 4;
    const size_t scan = a.kind == kMaskS ? (size_t)sh.nw * 64 * 8 : 0;
    sh.lds_dq = lds + scan;
    sh.lds_dkv = lds + 2 * (size_t)Lpad * 4 + scan;
    return sh;
}

template <typename K>
void allow_lds(K *kernel, size_t lds) {
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
}

template <int D, int KIND, int TT>
void launch_grad_t(const BwdShape &sh, const BwdParams &p, hipStream_t stream) {
    allow_lds(&bwd_dq_kernel<D, KIND, TT>, sh.lds_dq);
    hipLaunchKernelGGL((bwd_dq_kernel<D, KIND, TT>), dim3(p.nblocks), dim3(sh.nw * 64), sh.lds_dq, stream, p);
    allow_lds(&bwd_dkv_kernel<D, KIND, TT>, sh.lds_dkv);
    hipLaunchKernelGGL((bwd_dkv_kernel<D, KIND, TT>), dim3(p.nblocks), dim3(sh.nw * 64), sh.lds_dkv, stream, p);
}

template <int D, int KIND>
void launch_grad(const BwdShape &sh, const BwdParams &p, hipStream_t stream) {
    if constexpr (D != 128) {
        if (sh.tt == 2) return launch_grad_t<D, KIND, 2>(sh, p, stream);
    }
    launch_grad_t<D, KIND, 1>(sh, p, stream);
}

template <int D, int KIND>
hipError_t launch_t(const BwdArgs &a, hipStream_t stream) {
    const BwdShape sh = bwd_shape(a);
    BwdParams p;
    p.q = reinterpret_cast<const __bf16 *>(a.q);
    p.k = reinterpret_cast<const __bf16 *>(a.k);
    p.v = reinterpret_cast<const __bf16 *>(a.v);
    p.ll = a.log_lambda;
    p.H = a.H;
    p.L = a.L;
    p.y = reinterpret_cast<const __bf16 *>(a.y);
    p.dy = reinterpret_cast<const __bf16 *>(a.dy);
    p.den = a.den;
    p.dq = a.dq;
    p.dk = a.dk;
    p.dv = a.dv;
    p.g_bf16 = a.g_bf16 ? 1 : 0;
    const size_t n = (size_t)a.B * a.H * a.L;
    p.delta = reinterpret_cast<float *>(a.workspace);
    p.da_row = p.delta + n;
    p.da_col = p.da_row + n;
    p.dll = a.dll;
    p.nsb = sh.nsb;
    p.nblocks = a.B * a.H * sh.nsb;
    p.sk = sh.sk;
    p.nbuf = sh.nbuf;
    p.causal = a.causal ? 1 : 0;
    launch_grad<D, KIND>(sh, p, stream);
    if constexpr (KIND != kMaskLit) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_dll(KIND, p.da_row, p.da_col, p.dll, a.B, a.H, a.L, stream);
    }
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_kind(const BwdArgs &a, hipStream_t stream) {
    switch (a.kind) {
    case kMaskLit: return launch_t<D, kMaskLit>(a, stream);
    case kMaskD: return launch_t<D, kMaskD>(a, stream);
    default: return launch_t<D, kMaskS>(a, stream);
    }
}

}  // namespace

Plan plan_full_bwd(const BwdArgs &a) {
    Plan p;
    const BwdShape sh = bwd_shape(a);
    p.ok = (a.d == 32 || a.d == 64 || a.d == 128) && sh.lds_dkv <= kLdsPerWorkgroup;
    p.workspace = 3 * (size_t)a.B * a.H * a.L * 4;
    return p;
}

hipError_t launch_dll(int kind, float *da_row, float *da_col, float *dll, int B, int H, int L, hipStream_t stream) {
    BwdParams p{};
    p.H = H;
    p.L = L;
    p.da_row = da_row;
    p.da_col = da_col;
    p.dll = dll;
    if (kind == kMaskS)
        hipLaunchKernelGGL(bwd_dll_s_kernel, dim3(B * H), dim3(kDllThreads), 0, stream, p);
    else {
        hipLaunchKernelGGL(bwd_dll_d_rows_kernel, dim3(B * H), dim3(kDllThreads), 0, stream, p);
        hipLaunchKernelGGL(bwd_dll_d_kernel, dim3(H), dim3(kDllThreads), 0, stream, p, B);
    }
    return hipGetLastError();
}

hipError_t launch_dll_parts(const float *part, float *dll, int B, int H, hipStream_t stream) {
    hipLaunchKernelGGL(bwd_dll_d_parts_kernel, dim3(H), dim3(kDllThreads), 0, stream, part, dll, B, H);
    return hipGetLastError();
}

hipError_t launch_full_bwd(const BwdArgs &a, hipStream_t stream) {
    if (single_chunk_bwd_ok(a)) return launch_single_chunk_bwd(a, stream);
    switch (a.d) {
    case 32: return dispatch_kind<32>(a, stream);
    case 64: return dispatch_kind<64>(a, stream);
    default: return dispatch_kind<128>(a, stream);
    }
}

}  // namespace lion
