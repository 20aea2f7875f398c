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
// One workgroup per (batch, head).  Its first half of waves runs the forward recurrence over
// tokens 0, 1, ..., its second half the backward one over L-1, L-2, ...; both advance one token
// per step.  During the first ceil(L/2) steps each direction parks its partial (y, c) of the
// token it visits; after a barrier each direction meets tokens the other one has parked and
// finishes them.  The parking buffer is LDS when it fits, else a global workspace.
//
// State layout: direction wave w owns value columns 16w .. 16w+15; lane (r = lane % 16,
// g = lane / 16) holds S[rows g*D/4 .. g*D/4 + D/4 - 1][column 16w + r] in registers.  q^T S is a
// per-lane partial dot plus a 4-lane reduction; the row-sum state z is spread one row per lane and
// q.z is a full-wave reduction.
#include <type_traits>

#include "lion_device.h"
#include "lion_internal.h"

namespace lion {
namespace {

constexpr int kT = 16;                  // tokens staged per step block
constexpr int kLdsBufMax = 64 * 1024;   // parking buffer kept in LDS up to this many bytes

struct RnnParams {
    const void *q, *k, *v;
    const float *ll;
    float eps;
    int H, L;
    void *y;
    int out_bf16;
    float *den_out;
    float *ws;   // global parking buffer [B*H][L+1][D+1], or null when it lives in LDS
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

__device__ __forceinline__ float load_coherent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int KIND, bool BF16, bool LDSBUF>
__global__ void __launch_bounds__(1024) birnn_kernel(RnnParams p) {
    using T = std::conditional_t<BF16, __bf16, float>;
    constexpr int NWD = D / 16;            // waves per direction
    constexpr int NTD = NWD * 64;          // threads per direction
    constexpr int RPL = D / 4;             // state rows per lane
    constexpr int ZPL = (D + 63) / 64;     // z rows per lane
    constexpr int TPT = D / 4;             // staging threads per token (4 channels each)
    constexpr int DROW = D + 1;            // parking row: y[0..D-1], c
    static_assert(NTD / TPT == kT, "one staging pass per block");

    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int dir = tid / NTD;             // 0 forward, 1 backward
    const int dt = tid % NTD;              // thread index within the direction
    const int lane = tid & 63, dwave = dt >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int col = 16 * dwave + r;
    const int L = p.L;
    const int bh = blockIdx.x;
    const size_t base = (size_t)bh * L;

    // LDS: per direction [Qs T x D][Ks T x D][Vs T x D][dec T][diag T], then (optionally) parking buffer
    constexpr int STAGE = kT * (3 * D + 2);
    float *stage = reinterpret_cast<float *>(smem) + dir * STAGE;
    float *Qs = stage, *Ks = Qs + kT * D, *Vs = Ks + kT * D, *dec = Vs + kT * D, *sdiag = dec + kT;
    float *buf = LDSBUF ? reinterpret_cast<float *>(smem) + 2 * STAGE : p.ws + (size_t)bh * (L + 1) * DROW;

    const T *qg = reinterpret_cast<const T *>(p.q) + base * D;
    const T *kg = reinterpret_cast<const T *>(p.k) + base * D;
    const T *vg = reinterpret_cast<const T *>(p.v) + base * D;
    const float lg_head = (KIND == kMaskD) ? p.ll[bh % p.H] * kLog2e : 0.f;

    float S[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) S[i] = 0.f;
    float z[ZPL];
#pragma unroll
    for (int u = 0; u < ZPL; ++u) z[u] = 0.f;

    const int h = (L + 1) / 2;             // steps of the first phase
    const bool odd = (L & 1) != 0;

    // token visited at step s by this direction
    auto token_at = [&](int s) { return dir == 0 ? s : L - 1 - s; };

    for (int s0 = 0; s0 < L; s0 += kT) {
        // ---- stage kT steps of this direction: phi(q), phi(k), v, decay, diagonal -----------------
        {
            const int tl = dt / TPT, c4 = (dt % TPT) * 4;
            const int s = s0 + tl;
            const bool valid = s < L;
            const int t = valid ? token_at(s) : 0;
            float xq[4], xk[4], xv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xq[e] = valid ? (float)qg[(size_t)t * D + c4 + e] : 0.f;
                xk[e] = valid ? (float)kg[(size_t)t * D + c4 + e] : 0.f;
                xv[e] = valid ? (float)vg[(size_t)t * D + c4 + e] : 0.f;
            }
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xq[e] = phi_pre<KIND>(xq[e]);
                xk[e] = phi_pre<KIND>(xk[e]);
                sq += xq[e] * xq[e];
                sk += xk[e] * xk[e];
            }
            if constexpr (KIND == kMaskS) {
                const float fq = inv_norm(group_sum<TPT>(sq)), fk = inv_norm(group_sum<TPT>(sk));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xq[e] *= fq;
                    xk[e] *= fk;
                }
            }
            float dg = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) dg += xq[e] * xk[e];
            dg = group_sum<TPT>(dg);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Qs[tl * D + c4 + e] = valid ? xq[e] : 0.f;
                Ks[tl * D + c4 + e] = valid ? xk[e] : 0.f;
                Vs[tl * D + c4 + e] = xv[e];
            }
            if (dt % TPT == 0) {
                sdiag[tl] = valid ? dg : 0.f;
                // decay applied before adding token t: lambda_t forward, lambda_{t+1} backward
                float dcy = 1.f;
                if constexpr (KIND == kMaskD) dcy = fast_exp2(lg_head);
                if constexpr (KIND == kMaskS) {
                    const int td = dir == 0 ? t : t + 1;
                    dcy = (valid && td < L) ? fast_exp2(p.ll[base + td] * kLog2e) : 1.f;
                }
                dec[tl] = dcy;
            }
        }
        __syncthreads();

        // ---- advance the recurrence kT steps -------------------------------------------------------
        const int nsteps = min(kT, L - s0);
        for (int tl = 0; tl < nsteps; ++tl) {
            const int s = s0 + tl;
            if (s == h) {
                // phase change: everything parked in the first phase is visible from here on
                if constexpr (!LDSBUF) __threadfence();
                __syncthreads();
            }
            const int t = token_at(s);
            const float dcy = dec[tl];
            const float vc = Vs[tl * D + col];
            const float *qr = Qs + tl * D + g * RPL;
            const float *kr = Ks + tl * D + g * RPL;
            float ypart = 0.f;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                S[i] = __builtin_fmaf(dcy, S[i], kr[i] * vc);
                ypart = __builtin_fmaf(qr[i], S[i], ypart);
            }
            ypart += __shfl_xor(ypart, 16, 64);
            ypart += __shfl_xor(ypart, 32, 64);
            float cpart = 0.f;
#pragma unroll
            for (int u = 0; u < ZPL; ++u) {
                const int zr = lane + 64 * u;
                if (zr < D) {
                    z[u] = __builtin_fmaf(dcy, z[u], Ks[tl * D + zr]);
                    cpart = __builtin_fmaf(Qs[tl * D + zr], z[u], cpart);
                }
            }
            const float cden = wave_sum(cpart);

            if (s < h) {
                // park this direction's partial; the parking side removes the diagonal, except the
                // backward visit of the middle token of an odd L, which goes to the extra row L
                const bool middle_b = odd && dir == 1 && s == h - 1;
                const float dg = middle_b ? 0.f : sdiag[tl];
                float *row = buf + (size_t)(middle_b ? L : t) * DROW;
                if (g == 0) row[col] = ypart - dg * vc;
                if (dwave == 0 && lane == 0) row[D] = cden - dg;
            } else {
                const float *row = buf + (size_t)t * DROW;
                float yo, co;
                if constexpr (LDSBUF) {
                    yo = row[col];
                    co = row[D];
                } else {
                    yo = load_coherent(row + col);
                    co = load_coherent(row + D);
                }
                const float div = cden + co + p.eps;
                const float out = (ypart + yo) / div;
                if (g == 0) {
                    if (p.out_bf16)
                        reinterpret_cast<__bf16 *>(p.y)[(base + t) * D + col] = f2bf(out);
                    else
                        reinterpret_cast<float *>(p.y)[(base + t) * D + col] = out;
                }
                if (p.den_out && dwave == 0 && lane == 0) p.den_out[base + t] = div;
            }
        }
        __syncthreads();
    }

    // ---- middle token of an odd L: both partials were parked in the first phase --------------------
    if (odd) {
        if (h >= L) {  // L == 1: the phase change above never ran
            if constexpr (!LDSBUF) __threadfence();
            __syncthreads();
        }
        if (dir == 0) {
            const int m = h - 1;
            const float *rf = buf + (size_t)m * DROW;
            const float *rb = buf + (size_t)L * DROW;
            float yf, yb, cf, cb;
            if constexpr (LDSBUF) {
                yf = rf[col]; yb = rb[col]; cf = rf[D]; cb = rb[D];
            } else {
                yf = load_coherent(rf + col); yb = load_coherent(rb + col);
                cf = load_coherent(rf + D); cb = load_coherent(rb + D);
            }
            const float div = cf + cb + p.eps;
            const float out = (yf + yb) / div;
            if (g == 0) {
                if (p.out_bf16)
                    reinterpret_cast<__bf16 *>(p.y)[(base + m) * D + col] = f2bf(out);
                else
                    reinterpret_cast<float *>(p.y)[(base + m) * D + col] = out;
            }
            if (p.den_out && dwave == 0 && lane == 0) p.den_out[base + m] = div;
        }
    }
}

template <int D>
size_t park_bytes(int L) {
    return (size_t)(L + 1) * (D + 1) * 4;
}

size_t park_bytes_rt(int L, int d) { return (size_t)(L + 1) * (d + 1) * 4; }

bool park_in_lds(int L, int d) { return park_bytes_rt(L, d) <= (size_t)kLdsBufMax; }

template <int D, int KIND, bool BF16>
hipError_t launch_t(const AttnArgs &a, hipStream_t stream) {
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
    p.ws = reinterpret_cast<float *>(a.workspace);
    const int nt = 2 * (D / 16) * 64;
    size_t lds = (size_t)2 * kT * (3 * D + 2) * 4;
    const int grid = a.B * a.H;
    if (park_in_lds(a.L, D)) {
        lds += park_bytes<D>(a.L);
        if (lds > 64 * 1024)
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&birnn_kernel<D, KIND, BF16, true>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        hipLaunchKernelGGL((birnn_kernel<D, KIND, BF16, true>), dim3(grid), dim3(nt), lds, stream, p);
    } else {
        hipLaunchKernelGGL((birnn_kernel<D, KIND, BF16, false>), dim3(grid), dim3(nt), lds, stream, p);
    }
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

}  // namespace

Plan plan_birnn(const AttnArgs &a) {
    Plan p;
    p.ok = true;   // staging is at most 2 * 16 * (3 * 128 + 2) * 4 bytes; parking beyond 64 KiB goes to HBM
    p.workspace = park_in_lds(a.L, a.d) ? 0 : (size_t)a.B * a.H * park_bytes_rt(a.L, a.d);
    return p;
}

hipError_t launch_birnn(const AttnArgs &a, hipStream_t stream) {
    return a.in_bf16 ? dispatch_d<true>(a, stream) : dispatch_d<false>(a, stream);
}

}  // namespace lion
