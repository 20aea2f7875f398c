// lion_chunk_bwd.hip -- backward pass of the chunkwise form of LION.
//
// The gradients are those of the full form's backward (the chain rule of y = attention(q, k, v) with
// LION's mask; LION trains with the attention form, OpenReview abstract and reply "Concern 1",
// Theorem 3.3 Eq. 25), computed the way the chunkwise form computes y (reply "4: Practicality of
// Recurrent Inference"; blog "LION Part IV - Results", "LION Chunk"): inside a chunk of C tokens
// pair by pair, across chunks through d x (d+1) states, so the work per (batch, head) is
// O(L C d + L d^2) rather than O(L^2 d).
//
// With u_i = [dy_i / den_i, -delta_i] (delta_i = dy_i.y_i / den_i) and w_j = [v_j, 1], the gradient of
// the score of pair (i, j) is dp_ij = u_i.w_j, and
//   dphi(q_i) = sum_j M_ij dp_ij phi(k_j)        = (sum_j M_ij phi(k_j) w_j^T) u_i
//   dphi(k_j) = sum_i M_ij dp_ij phi(q_i)        = (sum_i M_ij phi(q_i) u_i^T) w_j
//   dv_j      = sum_i M_ij s_ij dy_i / den_i     = (sum_i M_ij phi(q_i) u_i^T)[:, :d]^T phi(k_j)
// so the keys' states are the forward pass's (phi(k) [v, 1]^T) and the queries' states are the same
// construction over phi(q) u^T.  For a token t of chunk c (first token s, last e), the tokens of
// earlier chunks enter through the state entering from the left, weighted by exp(A_t - A_{s-1}), and
// those of later chunks through the state entering from the right, weighted by exp(A_e - A_t); both
// exponents are sums of log(lambda) inside the chunk, so no prefix over the whole sequence is needed.
// The mask's gradient splits the same way: with w_ij = dp_ij M_ij s_ij,
//   dA_t = sum_{j<t} w_tj - sum_{j>t} w_tj  (row half) + sum_{i<t} w_it - sum_{i>t} w_it  (column half)
// and the row half over earlier chunks is phi(q_t) . (left state) u_t, times the weight, etc.
// dlog(lambda) then follows from dA as in the full form's backward (a reverse prefix sum for LION-S,
// sum_t t dA_t for LION-D).
//
// Two launches plus the dlog(lambda) one (states are stored with rows padded to 16 bytes):
//   walk:  one workgroup per (batch, head, direction, keys or queries) walks the chunks in order,
//          writing the state entering each chunk and then adding that chunk's tokens to its running
//          state (fp32 matrix cores, the state in accumulators);
//   main:  one workgroup per chunk forms the pair matrices M dp and M s in LDS (and the dA sums of
//          sign(i - j) M dp s), then dphi(q), dphi(k), dv and the rest of the dA halves from them and
//          from the four entering states, on the matrix cores in fp32; applies phi's Jacobian and
//          stores dq, dk, dv.
// Causal variant (M_ij = 0 for j > i): pairs above the diagonal drop out, and so do the keys' states
// entering from the right and the queries' states entering from the left (a key sees later queries).
#include "lion_device.h"
#include "lion_internal.h"

namespace lion {
namespace {

constexpr int kThreads = 256;   // a 16 x 16 grid of threads

struct CbParams {
    const __bf16 *q, *k, *v, *y, *dy;
    const float *den, *ll;
    int H, L, nch, causal;
    void *dq, *dk, *dv;
    int g_bf16;
    float *states;           // [B H][nch][4][D][D + 4] (D + 1 used): key-left, query-left, key-right, query-right
    float *da_row, *da_col;  // [B H L]
};

template <int D, int CT>
struct CbCfg {
    static constexpr int DP = D + 4;          // LDS row stride of token rows (floats)
    static constexpr int CP = CT + 4;         // LDS row stride of the pair matrices
    static constexpr int T = CT / 16;         // token rows per thread (rows grp, grp + 16, ...)
    static constexpr int TA = D / 16;         // contiguous channels per thread
    static constexpr int DS = D + 4;          // row stride of a state: D + 1 columns, padded to 16 bytes
    static constexpr int DD = D * DS;         // floats per state
    static constexpr int TOK = 4 * CT * DP + 2 * CT + 4;   // phi(q), phi(k), v, dy/den; -delta; cum, chunk total
    static constexpr int MAT = 2 * CT * CP;
    static constexpr int BUF = MAT > DD ? MAT : DD;
    static constexpr size_t LDS = (size_t)(TOK + BUF + 2 * CT) * 4;
    static constexpr size_t LDS_WALK = (size_t)TOK * 4;   // the walks stage tokens only
};

size_t cbwd_lds(int d, int C) {
    const int DP = d + 4, CP = C + 4, DD = d * (d + 4);
    const int tok = 4 * C * DP + 2 * C + 4, mat = 2 * C * CP;
    return (size_t)(tok + (mat > DD ? mat : DD) + 2 * C) * 4;
}

template <int N>
__device__ __forceinline__ void lds_load(float (&x)[N], const float *p) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int e = 0; e < N; e += 4) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(p + e);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[e + i] = t[i];
        }
    } else {
#pragma unroll
        for (int e = 0; e < N; ++e) x[e] = p[e];
    }
}

// Staging is split in two so a walk can issue the next chunk's loads before working on the current
// one: tok_load reads the chunk's rows into registers, tok_commit applies phi, forms u and -delta,
// writes the LDS rows and the prefix sums.
// WHICH: 0 everything, 1 the keys' rows only (phi(k), v), 2 the queries' only (phi(q), u, -delta).
template <int D, int CT>
struct TokRegs {
    static constexpr int SPR = D / 8;                 // 16-byte slots per row
    static constexpr int NSL = CT * SPR;              // a multiple of 64
    static constexpr int NIT = (NSL + kThreads - 1) / kThreads;
    bf16x8 q[NIT], k[NIT], v[NIT], y[NIT], d[NIT];
    float den[NIT];
    float ll;
};

template <int D, int KIND, int CT, int WHICH>
__device__ __forceinline__ void tok_load(const CbParams &p, int bh, int c, int n, TokRegs<D, CT> &R) {
    constexpr bool LQ = WHICH != 1, LK = WHICH != 2;
    using TR = TokRegs<D, CT>;
    const int tid = threadIdx.x;
    const size_t row0 = (size_t)bh * p.L + (size_t)c * CT;
#pragma unroll
    for (int it = 0; it < TR::NIT; ++it) {
        const int sl = it * kThreads + tid;
        const int row = sl / TR::SPR, cs = (sl % TR::SPR) * 8;
        if (sl < TR::NSL && row < n) {
            const size_t g = (row0 + row) * D + cs;
            if constexpr (LQ) {
                R.q[it] = __builtin_bit_cast(bf16x8, ld16(p.q + g));
                R.y[it] = __builtin_bit_cast(bf16x8, ld16(p.y + g));
                R.d[it] = __builtin_bit_cast(bf16x8, ld16(p.dy + g));
                R.den[it] = p.den[row0 + row];
            }
            if constexpr (LK) {
                R.k[it] = __builtin_bit_cast(bf16x8, ld16(p.k + g));
                R.v[it] = __builtin_bit_cast(bf16x8, ld16(p.v + g));
            }
        }
    }
    if constexpr (KIND == kMaskS)
        if (tid < 64) R.ll = tid < n ? p.ll[row0 + tid] : 0.f;
}

// Rows at or past n are zero; prefix sums (log2 units, relative to the chunk start, inclusive) past n
// repeat the last one; cum[CT] is the chunk's total.
template <int D, int KIND, int CT, int WHICH>
__device__ __forceinline__ void tok_commit(const CbParams &p, float *sm, int bh, int n, const TokRegs<D, CT> &R) {
    constexpr bool LQ = WHICH != 1, LK = WHICH != 2;
    using CF = CbCfg<D, CT>;
    using TR = TokRegs<D, CT>;
    constexpr int SPR = TR::SPR;
    float *Qs = sm, *Ks = Qs + CT * CF::DP, *Vs = Ks + CT * CF::DP, *Us = Vs + CT * CF::DP;
    float *nd = Us + CT * CF::DP, *cum = nd + CT;
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < TR::NIT; ++it) {
        if (it * kThreads + (tid & ~63) >= TR::NSL) break;   // whole waves
        const int sl = it * kThreads + tid;
        const int row = sl / SPR, cs = (sl % SPR) * 8;
        const bool ok = row < n;
        float fq[8] = {}, fk[8] = {}, fv[8] = {}, fu[8] = {};
        float ssq = 0.f, ssk = 0.f, part = 0.f, dinv = 0.f;
        if (ok) {
            if constexpr (LQ) {
                dinv = 1.f / R.den[it];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    fq[e] = phi_pre<KIND>((float)R.q[it][e]);
                    fu[e] = (float)R.d[it][e] * dinv;
                    ssq += fq[e] * fq[e];
                    part += (float)R.d[it][e] * (float)R.y[it][e];
                }
            }
            if constexpr (LK) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    fk[e] = phi_pre<KIND>((float)R.k[it][e]);
                    fv[e] = (float)R.v[it][e];
                    ssk += fk[e] * fk[e];
                }
            }
        }
        if constexpr (LQ) part = group_sum<SPR>(part);
        if constexpr (KIND == kMaskS) {
            const float sq = LQ ? inv_norm(group_sum<SPR>(ssq)) : 0.f;
            const float sk = LK ? inv_norm(group_sum<SPR>(ssk)) : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                fq[e] *= sq;
                fk[e] *= sk;
            }
        }
        float *dst[4] = {Qs, Ks, Vs, Us};
        const float *src[4] = {fq, fk, fv, fu};
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            if ((a == 0 || a == 3) ? !LQ : !LK) continue;
            f32x4 lo, hi;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lo[e] = src[a][e];
                hi[e] = src[a][4 + e];
            }
            *reinterpret_cast<f32x4 *>(dst[a] + row * CF::DP + cs) = lo;
            *reinterpret_cast<f32x4 *>(dst[a] + row * CF::DP + cs + 4) = hi;
        }
        if (LQ && sl % SPR == 0) nd[row] = ok ? -part * dinv : 0.f;
    }
    if (tid < 64) {
        const int t = tid;
        float c2 = 0.f, tot2 = 0.f;
        if constexpr (KIND == kMaskD) {
            const float lg = p.ll[bh % p.H] * kLog2e;
            c2 = (float)(min(t, n - 1) + 1) * lg;
            tot2 = (float)n * lg;
        } else if constexpr (KIND == kMaskS) {
            double x = (double)R.ll;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const double up = __shfl_up(x, o, 64);
                if (t >= o) x += up;
            }
            c2 = (float)(x * 1.4426950408889634);
            tot2 = (float)(__shfl(x, 63, 64) * 1.4426950408889634);
        }
        if (t < CT) cum[t] = c2;
        if (t == 0) cum[CT] = tot2;
    }
}

template <int D, int KIND, int CT, int WHICH = 0>
__device__ void stage_tokens(const CbParams &p, float *sm, int bh, int c, int n) {
    TokRegs<D, CT> R;
    tok_load<D, KIND, CT, WHICH>(p, bh, c, n, R);
    tok_commit<D, KIND, CT, WHICH>(p, sm, bh, n, R);
}

// ================================ entering states by sequential walks ================================
// One workgroup per (batch, head, direction, keys or queries) walks the chunks -- left to right for the
// states entering from the left, right to left for those entering from the right -- carrying its
// running state in registers, so each entering state is written once.  Causal runs only the keys'
// walk from the left and the queries' walk from the right.  The running state's first D columns live
// in matrix-core accumulators (16 x 16 tiles spread over the four waves), column D in thread a of the
// first D threads.  (Splitting a walk over two workgroups by rows measured slower where the pairs
// already fill the chip: the second workgroup stages the same tokens again.)
template <int D, int KIND, int CT, int WHICH>
__device__ void walk(const CbParams &p, float *sm, int bh, int dir) {
    using CF = CbCfg<D, CT>;
    constexpr int NA = D / 16, NTW = NA * NA / 4;   // 16 x 16 state tiles, per wave
    constexpr bool KEYS = WHICH == 1;
    const float *Qs = sm, *Ks = Qs + CT * CF::DP, *Vs = Ks + CT * CF::DP, *Us = Vs + CT * CF::DP;
    const float *nd = Us + CT * CF::DP, *cum = nd + CT;
    const float *X = KEYS ? Ks : Qs, *Y = KEYS ? Vs : Us;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int st = 2 * dir + (KEYS ? 0 : 1);
    f32x4 acc[NTW];   // state rows 16 ta + 4 g + e, column 16 tb + r of tile w + 4 u = NA ta + tb
#pragma unroll
    for (int u = 0; u < NTW; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    float z = 0.f;    // column D of row tid (tid < D)
    TokRegs<D, CT> R;
    {
        const int c = dir == 0 ? 0 : p.nch - 1;
        const int n = min(CT, p.L - c * CT);
        tok_load<D, KIND, CT, WHICH>(p, bh, c, n, R);
        tok_commit<D, KIND, CT, WHICH>(p, sm, bh, n, R);
        __syncthreads();
    }
#pragma unroll 1
    for (int step = 0; step < p.nch; ++step) {
        const int c = dir == 0 ? step : p.nch - 1 - step;
        const int n = min(CT, p.L - c * CT);
        const int cn = dir == 0 ? c + 1 : c - 1;             // the next chunk of the walk
        const int nn = min(CT, p.L - cn * CT);
        const bool more = step + 1 < p.nch;
        if (more) tok_load<D, KIND, CT, WHICH>(p, bh, cn, nn, R);   // in flight while this chunk is summed
        // the state entering chunk c is the running sum so far
        float *out = p.states + (((size_t)bh * p.nch + c) * 4 + st) * CF::DD;
#pragma unroll
        for (int u = 0; u < NTW; ++u) {
            const int tile = w + 4 * u, ta = tile / NA, tb = tile % NA;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[(16 * ta + 4 * g + e) * CF::DS + 16 * tb + r] = acc[u][e];
        }
        if (tid < D) {
            out[tid * CF::DS + D] = z;
#pragma unroll
            for (int pad = 1; pad < 4; ++pad) out[tid * CF::DS + D + pad] = 0.f;
        }
        // then decay it across the chunk and add the chunk's own tokens, weighted towards the chunk's
        // far end (its right end walking from the left, its left end walking from the right), on the
        // matrix cores: state[a][b] += sum_j (w_j x_j[a]) y_j[b]
        const float tot2 = cum[CT];
        const float dec = KIND == kMaskLit ? 1.f : fast_exp2(tot2);
#pragma unroll
        for (int u = 0; u < NTW; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[u][e] *= dec;
        z *= dec;
#pragma unroll 2
        for (int k0 = 0; k0 < CT; k0 += 4) {
            const int j = k0 + g;   // rows past n are zero
            const float wj = KIND == kMaskLit ? 1.f : fast_exp2(dir == 0 ? tot2 - cum[j] : cum[j]);
#pragma unroll
            for (int u = 0; u < NTW; ++u) {
                const int tile = w + 4 * u, ta = tile / NA, tb = tile % NA;
                acc[u] = mfma_f32(wj * X[j * CF::DP + 16 * ta + r], Y[j * CF::DP + 16 * tb + r], acc[u]);
            }
        }
        if (tid < D) {
            for (int j = 0; j < n; ++j) {
                const float wj = KIND == kMaskLit ? 1.f : fast_exp2(dir == 0 ? tot2 - cum[j] : cum[j]);
                z += wj * X[j * CF::DP + tid] * (KEYS ? 1.f : nd[j]);
            }
        }
        __syncthreads();   // before the next chunk's tokens overwrite these
        if (more) {
            tok_commit<D, KIND, CT, WHICH>(p, sm, bh, nn, R);
            __syncthreads();
        }
    }
}

template <int D, int KIND, int CT>
__global__ void __launch_bounds__(kThreads) cbwd_walk_kernel(CbParams p) {
    extern __shared__ __attribute__((aligned(16))) float sm[];
    const int ns = p.causal ? 2 : 4;
    const int bh = blockIdx.x / ns, s = blockIdx.x % ns;
    // causal: s = 0 keys from the left, s = 1 queries from the right; else s = 2 dir + (queries)
    const int dir = p.causal ? s : s >> 1;
    const bool keys = p.causal ? s == 0 : (s & 1) == 0;
    if (keys) walk<D, KIND, CT, 1>(p, sm, bh, dir);
    else walk<D, KIND, CT, 2>(p, sm, bh, dir);
}

// ================================ main ===============================================================
// The transposed Jacobian of phi at the raw inputs x (TA channels of one row; the 16 threads of a row
// hold its D channels) applied to g in place.
template <int TA, int KIND>
__device__ __forceinline__ void phi_backward_row(const float (&x)[TA], float (&g)[TA]) {
    if constexpr (KIND == kMaskLit) {
#pragma unroll
        for (int e = 0; e < TA; ++e)
            if (!(x[e] > 0.f)) g[e] *= fast_exp2(x[e] * kLog2e);
    } else if constexpr (KIND == kMaskS) {
        float sig[TA], sv[TA], ss = 0.f;
#pragma unroll
        for (int e = 0; e < TA; ++e) {
            sig[e] = __builtin_amdgcn_rcpf(1.f + fast_exp2(-x[e] * kLog2e));
            sv[e] = x[e] * sig[e];
            ss += sv[e] * sv[e];
        }
        const float inv = inv_norm(group_sum<16>(ss));
        float pg = 0.f;
#pragma unroll
        for (int e = 0; e < TA; ++e) pg += sv[e] * inv * g[e];
        pg = group_sum<16>(pg);
#pragma unroll
        for (int e = 0; e < TA; ++e) {
            const float ds = sig[e] * (1.f + x[e] * (1.f - sig[e]));
            g[e] = ds * (g[e] - sv[e] * inv * pg) * inv;
        }
    }
}

template <int TA>
__device__ __forceinline__ void load_raw(const __bf16 *src, float (&x)[TA]) {
    __bf16 b[TA];
    __builtin_memcpy(b, src, sizeof(b));
#pragma unroll
    for (int e = 0; e < TA; ++e) x[e] = (float)b[e];
}

template <int TA>
__device__ __forceinline__ void store_row(void *base, bool bf16, size_t off, const float (&g)[TA]) {
    if (bf16) {
        __bf16 b[TA];
#pragma unroll
        for (int e = 0; e < TA; ++e) b[e] = f2bf(g[e]);
        __builtin_memcpy(reinterpret_cast<__bf16 *>(base) + off, b, sizeof(b));
    } else {
        __builtin_memcpy(reinterpret_cast<float *>(base) + off, g, sizeof(g));
    }
}

// The pair and state products run on the matrix cores in fp32 (v_mfma_f32_16x16x4f32: lane 16 g + r
// supplies A[r][k0 + g] and B[k0 + g][r] and receives D[4 g + e][r]); every operand is read from the
// fp32 LDS tiles, so the inputs keep their fp32 values.  Wave w takes 16 x 16 tiles w, w + 4, ...
template <int D, int KIND, int CT>
__global__ void __launch_bounds__(kThreads) cbwd_main_kernel(CbParams p) {
    using CF = CbCfg<D, CT>;
    constexpr int T = CF::T, TA = CF::TA, DP = CF::DP, CP = CF::CP, DS = CF::DS;
    constexpr int NT = CT / 16, NA = D / 16;
    constexpr int NOUT = (NT * NA + 3) / 4;   // output tiles per wave
    extern __shared__ __attribute__((aligned(16))) float sm[];
    const int bh = blockIdx.x / p.nch, c = blockIdx.x % p.nch;
    const int n = min(CT, p.L - c * CT);
    float *Qs = sm, *Ks = Qs + CT * DP, *Vs = Ks + CT * DP, *Us = Vs + CT * DP;
    const float *nd = Us + CT * DP, *cum = nd + CT;
    float *buf = sm + CF::TOK;
    float *D1 = buf, *D2 = D1 + CT * CP;
    float *dar = sm + CF::TOK + CF::BUF, *dac = dar + CT;   // dA halves of the chunk's tokens
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    for (int t = tid; t < 2 * CT; t += kThreads) dar[t] = 0.f;
    stage_tokens<D, KIND, CT>(p, sm, bh, c, n);
    __syncthreads();
    const float tot2 = cum[CT];
    const bool causal = p.causal != 0;

    // ---- pair matrices D1 = M dp and D2 = M s; the dA sums of sign(i - j) M dp s straight from them
    for (int tile = w; tile < NT * NT; tile += 4) {
        const int ti = tile / NT, tj = tile % NT;
        f32x4 x = {0.f, 0.f, 0.f, 0.f}, s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int k0 = 0; k0 < D; k0 += 4) {
            x = mfma_f32(Us[(16 * ti + r) * DP + k0 + g], Vs[(16 * tj + r) * DP + k0 + g], x);
            s = mfma_f32(Qs[(16 * ti + r) * DP + k0 + g], Ks[(16 * tj + r) * DP + k0 + g], s);
        }
        const int j = 16 * tj + r;
        float csum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * ti + 4 * g + e;
            const bool ok = i < n && j < n && !(causal && j > i);
            float m = 0.f;
            if (ok) m = KIND == kMaskLit ? 1.f : fast_exp2(-fabsf(cum[i] - cum[j]));
            const float dp = x[e] + nd[i];
            D1[i * CP + j] = m * dp;
            D2[i * CP + j] = m * s[e];
            if constexpr (KIND != kMaskLit) {
                const float sw = (j < i ? 1.f : (j > i ? -1.f : 0.f)) * m * dp * s[e];
                const float rs = group_sum<16>(sw);           // over this tile's 16 columns
                if (r == 0) atomicAdd(&dar[i], rs);
                csum -= sw;
            }
        }
        if constexpr (KIND != kMaskLit) {
            csum += __shfl_xor(csum, 16, 64);
            csum += __shfl_xor(csum, 32, 64);                // over this tile's 16 rows
            if (g == 0) atomicAdd(&dac[j], csum);
        }
    }
    __syncthreads();

    // ---- the entering states this chunk needs (zero: nothing left of the first chunk or right of
    // the last; causal, the keys' state from the right and the queries' state from the left), each
    // loaded into registers while the previous work runs
    int sts[4], nst = 0;
    {
        const int c_last = p.nch - 1;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const bool right = st >= 2, keys = (st & 1) == 0;
            if (!((right ? c == c_last : c == 0) || (causal && keys == right))) sts[nst++] = st;
        }
    }
    constexpr int NV = (CF::DD / 4 + kThreads - 1) / kThreads;   // 16-byte pieces of a state per thread
    f32x4 sreg[NV];
    auto load_state = [&](int st) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(p.states + (((size_t)bh * p.nch + c) * 4 + st) * CF::DD);
#pragma unroll
        for (int v = 0; v < NV; ++v)
            if (v * kThreads + tid < CF::DD / 4) sreg[v] = src[v * kThreads + tid];
    };
    if (nst > 0) load_state(sts[0]);

    // ---- intra-chunk parts of the output tiles (rows t = 16 tt + 4 g + e, channels 16 ta + r)
    f32x4 aq[NOUT], ak[NOUT], av[NOUT];
#pragma unroll
    for (int u = 0; u < NOUT; ++u) {
        aq[u] = ak[u] = av[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int tile = w + 4 * u;
        if (tile >= NT * NA) break;
        const int tt = tile / NA, ta = tile % NA;
#pragma unroll 4
        for (int j0 = 0; j0 < CT; j0 += 4) {
            const int jr = j0 + g;
            aq[u] = mfma_f32(D1[(16 * tt + r) * CP + jr], Ks[jr * DP + 16 * ta + r], aq[u]);
            ak[u] = mfma_f32(D1[jr * CP + 16 * tt + r], Qs[jr * DP + 16 * ta + r], ak[u]);
            av[u] = mfma_f32(D2[jr * CP + 16 * tt + r], Us[jr * DP + 16 * ta + r], av[u]);
        }
    }
    __syncthreads();   // the pair matrices' space takes the states next

    // ---- apply the entering states
#pragma unroll 1
    for (int k = 0; k < nst; ++k) {
        const int st = sts[k];
        const bool right = st >= 2, keys = (st & 1) == 0;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            if (v * kThreads + tid < CF::DD / 4) reinterpret_cast<f32x4 *>(buf)[v * kThreads + tid] = sreg[v];
        __syncthreads();
        if (k + 1 < nst) load_state(sts[k + 1]);
        const float sgn = right ? -1.f : 1.f;
        const float *Xs = keys ? Us : Vs;   // what the state multiplies: u (keys' states), w (queries')
        const float *Ps = keys ? Qs : Ks;   // the dA half dots the result with phi of the same token
#pragma unroll
        for (int u = 0; u < NOUT; ++u) {
            const int tile = w + 4 * u;
            if (tile >= NT * NA) break;
            const int tt = tile / NA, ta = tile % NA, a = 16 * ta + r;
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int b0 = 0; b0 < D; b0 += 4)
                o = mfma_f32(Xs[(16 * tt + r) * DP + b0 + g], buf[a * DS + b0 + g], o);
            const float last = buf[a * DS + D];
            float part[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * tt + 4 * g + e;
                const float f = KIND == kMaskLit ? 1.f : fast_exp2(right ? tot2 - cum[t] : cum[t]);
                const float oe = o[e] + last * (keys ? nd[t] : 1.f);
                if (keys) aq[u][e] += f * oe;
                else ak[u][e] += f * oe;
                part[e] = sgn * f * Ps[t * DP + a] * oe;
            }
            if constexpr (KIND != kMaskLit) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ps = group_sum<16>(part[e]);   // over this tile's 16 channels
                    if (r == 0) atomicAdd(keys ? &dar[16 * tt + 4 * g + e] : &dac[16 * tt + 4 * g + e], ps);
                }
            }
            if (!keys) {   // dv: the state's first D columns, transposed, times phi(k_t)
                f32x4 ov = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
                for (int a0 = 0; a0 < D; a0 += 4)
                    ov = mfma_f32(Ks[(16 * tt + r) * DP + a0 + g], buf[(a0 + g) * DS + 16 * ta + r], ov);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * tt + 4 * g + e;
                    const float f = KIND == kMaskLit ? 1.f : fast_exp2(right ? tot2 - cum[t] : cum[t]);
                    av[u][e] += f * ov[e];
                }
            }
        }
        __syncthreads();
    }

    // ---- the outputs into the token tiles (no longer read), then phi's Jacobian and the stores with
    // thread (ti, ta) owning rows ti + 16 r and channels ta TA .. + TA - 1
#pragma unroll
    for (int u = 0; u < NOUT; ++u) {
        const int tile = w + 4 * u;
        if (tile >= NT * NA) break;
        const int tt = tile / NA, ta = tile % NA;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int at = (16 * tt + 4 * g + e) * DP + 16 * ta + r;
            Qs[at] = aq[u][e];
            Ks[at] = ak[u][e];
            Vs[at] = av[u][e];
        }
    }
    __syncthreads();
    const int ti = tid >> 4, ta = tid & 15, a0 = ta * TA;
    const size_t row0 = (size_t)bh * p.L + (size_t)c * CT;
    const bool gb = p.g_bf16 != 0;
#pragma unroll
    for (int rr = 0; rr < T; ++rr) {
        const int t = ti + 16 * rr;
        if (t >= n) break;   // the row's 16 threads agree; later rr only grow
        const size_t off = (row0 + t) * D + a0;
        float gq[TA], gk[TA], gv[TA];
        lds_load(gq, Qs + t * DP + a0);
        lds_load(gk, Ks + t * DP + a0);
        lds_load(gv, Vs + t * DP + a0);
        if constexpr (KIND != kMaskD) {
            float xq[TA], xk[TA];
            load_raw(p.q + off, xq);
            load_raw(p.k + off, xk);
            phi_backward_row<TA, KIND>(xq, gq);
            phi_backward_row<TA, KIND>(xk, gk);
        }
        store_row(p.dq, gb, off, gq);
        store_row(p.dk, gb, off, gk);
        store_row(p.dv, gb, off, gv);
        if constexpr (KIND != kMaskLit) {
            if (ta == 0) {
                p.da_row[row0 + t] = dar[t];
                p.da_col[row0 + t] = dac[t];
            }
        }
    }
}

// ================================ host side ===========================================================
template <typename K>
void allow_lds(K *kernel, size_t lds) {
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
}

struct CbLayout {
    size_t states, da;   // float offsets into the workspace
    size_t floats;
};

CbLayout cbwd_layout(int B, int H, int L, int d, int C) {
    const size_t bh = (size_t)B * H, nch = (size_t)((L + C - 1) / C);
    const size_t dd = (size_t)d * (d + 4);
    CbLayout w;
    w.states = 0;
    w.da = 4 * bh * nch * dd;
    w.floats = w.da + 2 * (((bh * L) + 3) / 4) * 4;
    return w;
}

template <int D, int KIND, int CT>
hipError_t launch_cbwd_t(const BwdArgs &a, hipStream_t stream) {
    using CF = CbCfg<D, CT>;
    const CbLayout w = cbwd_layout(a.B, a.H, a.L, a.d, CT);
    float *ws = reinterpret_cast<float *>(a.workspace);
    CbParams p;
    p.q = reinterpret_cast<const __bf16 *>(a.q);
    p.k = reinterpret_cast<const __bf16 *>(a.k);
    p.v = reinterpret_cast<const __bf16 *>(a.v);
    p.y = reinterpret_cast<const __bf16 *>(a.y);
    p.dy = reinterpret_cast<const __bf16 *>(a.dy);
    p.den = a.den;
    p.ll = a.log_lambda;
    p.H = a.H;
    p.L = a.L;
    p.nch = (a.L + CT - 1) / CT;
    p.causal = a.causal ? 1 : 0;
    p.dq = a.dq;
    p.dk = a.dk;
    p.dv = a.dv;
    p.g_bf16 = a.g_bf16 ? 1 : 0;
    p.states = ws + w.states;
    const size_t n = (size_t)a.B * a.H * a.L;
    p.da_row = ws + w.da;
    p.da_col = p.da_row + ((n + 3) / 4) * 4;
    const int nblk = a.B * a.H * p.nch;
    if (p.nch > 1) {
        allow_lds(&cbwd_walk_kernel<D, KIND, CT>, CF::LDS_WALK);
        hipLaunchKernelGGL((cbwd_walk_kernel<D, KIND, CT>), dim3(a.B * a.H * (a.causal ? 2 : 4)), dim3(kThreads),
                           CF::LDS_WALK, stream, p);
    }
    allow_lds(&cbwd_main_kernel<D, KIND, CT>, CF::LDS);
    hipLaunchKernelGGL((cbwd_main_kernel<D, KIND, CT>), dim3(nblk), dim3(kThreads), CF::LDS, stream, p);
    if (KIND != kMaskLit) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_dll(KIND, p.da_row, p.da_col, a.dll, a.B, a.H, a.L, stream);
    }
    return hipGetLastError();
}

template <int D, int KIND>
hipError_t launch_cbwd_c(const BwdArgs &a, hipStream_t stream) {
    return a.C == 16 ? launch_cbwd_t<D, KIND, 16>(a, stream) : launch_cbwd_t<D, KIND, 32>(a, stream);
}

template <int D>
hipError_t launch_cbwd_kind(const BwdArgs &a, hipStream_t stream) {
    switch (a.kind) {
    case kMaskLit: return launch_cbwd_c<D, kMaskLit>(a, stream);
    case kMaskD: return launch_cbwd_c<D, kMaskD>(a, stream);
    default: return launch_cbwd_c<D, kMaskS>(a, stream);
    }
}

}  // namespace

// Chunks of 64 and 128 run on the bf16 matrix-core kernels (lion_chunk_bwd_mfma.hip); 16 and 32 here.
Plan plan_chunk_bwd(const BwdArgs &a) {
    if (a.C >= 64) return plan_chunk_bwd_mfma(a);
    Plan p;
    const bool dims = a.d == 32 || a.d == 64 || a.d == 128;
    const bool cs = a.C == 16 || a.C == 32;
    p.ok = dims && cs && cbwd_lds(a.d, a.C) <= kLdsPerWorkgroup;
    p.workspace = p.ok ? cbwd_layout(a.B, a.H, a.L, a.d, a.C).floats * 4 : 0;
    return p;
}

hipError_t launch_chunk_bwd(const BwdArgs &a, hipStream_t stream) {
    if (a.C >= 64) return launch_chunk_bwd_mfma(a, stream);
    switch (a.d) {
    case 32: return launch_cbwd_kind<32>(a, stream);
    case 64: return launch_cbwd_kind<64>(a, stream);
    default: return launch_cbwd_kind<128>(a, stream);
    }
}

}  // namespace lion
