// lion_mask.h -- the log-space mask generator shared by the full and chunkwise kernels.
//
// The mask of LION is M_ij = exp(-|A_i - A_j|) with A_t the prefix sums of log(lambda) -- the cumsum
// construction of the pages ("LION: A bidirectional framework ...", reply "P3: LION-S uses cumsum
// (parallel scan)").  Kernels keep a per-position exponent table E_t = (A_t - A_ref) log2(e) in LDS
// and only ever exponentiate non-positive differences of it.  For LION-S the prefix sums are taken
// in fp64 (a workgroup-wide scan), so rounding does not accumulate along long sequences; LION-D's
// table is the single product (t - t_ref) log2(lambda_h).
#pragma once

#include "lion_device.h"

namespace lion {

// Exclusive scan of one double per thread over the workgroup (nt a multiple of 64, <= 1024).
__device__ __forceinline__ double block_excl_scan(double x, double *sh, int tid, int nt) {
    sh[tid] = x;
    __syncthreads();
    if (tid < 64) {
        const int per = nt / 64;
        double local = 0.0;
        for (int u = 0; u < per; ++u) local += sh[tid * per + u];
        double incl = local;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            double t = __shfl_up(incl, o, 64);
            if (tid >= o) incl += t;
        }
        double run = incl - local;
        for (int u = 0; u < per; ++u) {
            double t = sh[tid * per + u];
            sh[tid * per + u] = run;
            run += t;
        }
    }
    __syncthreads();
    double r = sh[tid];
    __syncthreads();
    return r;
}

// Mask exponent table E[0 .. Lpad) for one (batch, head), relative to position t_ref; entries past
// L - 1 repeat E[L - 1].
template <int KIND>
__device__ __forceinline__ void build_exponents(float *E, double *scan_sh, const float *ll, int bh, int H, int L, int Lpad,
                                int t_ref, int tid, int nt) {
    if constexpr (KIND == kMaskD) {
        const float lg = ll[bh % H] * kLog2e;
        for (int t = tid; t < Lpad; t += nt) E[t] = (float)(min(t, L - 1) - t_ref) * lg;
        __syncthreads();
    } else if constexpr (KIND == kMaskS) {
        const float *row = ll + (size_t)bh * L;
        const int seg = (L + nt - 1) / nt;
        const int t0 = tid * seg, t1 = min(t0 + seg, L);
        double s = 0.0;
        for (int t = t0; t < t1; ++t) s += (double)row[t];
        const double excl = block_excl_scan(s, scan_sh, tid, nt);
        // A at t_ref, computed by the thread whose segment holds it
        __shared__ double a_ref;
        if (t_ref >= t0 && t_ref < t1) {
            double a = excl;
            for (int t = t0; t <= t_ref; ++t) a += (double)row[t];
            a_ref = a;
        }
        __syncthreads();
        const double ar = a_ref;
        double a = excl;
        for (int t = t0; t < t1; ++t) {
            a += (double)row[t];
            E[t] = (float)((a - ar) * 1.4426950408889634);
        }
        __syncthreads();
        // positions past the end repeat the last exponent, so every difference a kernel forms with
        // them stays <= 0 where real positions' would
        const float elast = E[L - 1];
        for (int t = L + tid; t < Lpad; t += nt) E[t] = elast;
        __syncthreads();
    }
}

}  // namespace lion
