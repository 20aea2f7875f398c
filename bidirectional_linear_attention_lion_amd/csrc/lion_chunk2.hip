// lion_chunk2.hip -- chunkwise form with the masks of two token orders averaged.
//
// The patch-reordered vision models average the masks of two patch orders, M = (M_b + M_c) / 2 (reply
// "P2: Comparison against vision SSMs", item 1, Figure 7 b and c).  The attention is linear in M, so
//   y = (num_b + num_c) / (S_b + S_c + 2 eps) = (y_b den_b + y_c den_c) / (den_b + den_c)
// with y_x, den_x = S_x + eps the chunkwise form's fp32 output and row sums under one order each.  The
// second order is the chunkwise form applied to the tokens rearranged into that order (each token
// keeps its own decay), so this file only adds two kernels around two chunkwise launches:
//   gather:  q, k, v (and LION-S's log(lambda)) rearranged into the second order, in the workspace;
//   combine: y and den_out of the averaged mask from the two launches' fp32 results, the second
//            order's results read back at each token's position in it.
#include "lion_device.h"
#include "lion_internal.h"

namespace lion {
namespace {

constexpr int kThreads = 256;

struct C2Layout {
    size_t q, k, v, ll, yb, yc, db, dc, inner;   // byte offsets into the workspace
    size_t bytes;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

C2Layout c2_layout(const AttnArgs &a, size_t inner_bytes) {
    const size_t rows = (size_t)a.B * a.H * a.L, elems = rows * a.d;
    const size_t esz = a.in_bf16 ? 2 : 4;
    C2Layout w;
    size_t off = 0;
    w.q = off, off = align256(off + elems * esz);
    w.k = off, off = align256(off + elems * esz);
    w.v = off, off = align256(off + elems * esz);
    w.ll = off, off = align256(off + (a.kind == kMaskS ? rows * 4 : 0));
    w.yb = off, off = align256(off + elems * 4);
    w.yc = off, off = align256(off + elems * 4);
    w.db = off, off = align256(off + rows * 4);
    w.dc = off, off = align256(off + rows * 4);
    w.inner = off, off = align256(off + inner_bytes);
    w.bytes = off;
    return w;
}

// Row p of (batch, head) bh in the second order is token order[p]: 16-byte pieces of q, k, v.
__global__ void __launch_bounds__(kThreads) c2_gather_kernel(const u32x4 *q, const u32x4 *k, const u32x4 *v,
                                                            const float *ll, const int *order, u32x4 *q2, u32x4 *k2,
                                                            u32x4 *v2, float *ll2, int L, int pieces, size_t total) {
    const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= total) return;
    const size_t row = i / pieces;
    const int piece = (int)(i % pieces);
    const size_t bh = row / L;
    const int p = (int)(row % L);
    const int t = min(max(order[p], 0), L - 1);   // a non-permutation gives wrong values, never a bad access
    const size_t src = (bh * L + t) * pieces + piece;
    q2[i] = q[src];
    k2[i] = k[src];
    v2[i] = v[src];
    if (ll2 && piece == 0) ll2[row] = ll[bh * L + t];
}

// One thread per (row of the second order, channel group of 4): token t = order[p].
__global__ void __launch_bounds__(kThreads) c2_combine_kernel(const float *yb, const float *yc, const float *db,
                                                             const float *dc, const int *order, void *y, int y_bf16,
                                                             float *den_out, int L, int d, size_t total) {
    const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= total) return;
    const int groups = d / 4;
    const size_t row = i / groups;   // row of the second order
    const int grp = (int)(i % groups);
    const size_t bh = row / L;
    const int p = (int)(row % L);
    const int t = min(max(order[p], 0), L - 1);
    const size_t trow = bh * L + t;
    const float dbv = db[trow], dcv = dc[row];
    const float inv = 1.f / (dbv + dcv);
    const f32x4 a = *reinterpret_cast<const f32x4 *>(yb + trow * d + 4 * grp);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(yc + row * d + 4 * grp);
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (a[e] * dbv + b[e] * dcv) * inv;
    if (y_bf16) {
        bf16x4 ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[e] = f2bf(o[e]);
        *reinterpret_cast<bf16x4 *>(reinterpret_cast<__bf16 *>(y) + trow * d + 4 * grp) = ob;
    } else {
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(y) + trow * d + 4 * grp) = o;
    }
    if (den_out && grp == 0) den_out[trow] = 0.5f * (dbv + dcv);
}

AttnArgs inner_args(const AttnArgs &a) {
    AttnArgs b = a;
    b.order = nullptr;
    b.out_bf16 = false;
    return b;
}

}  // namespace

Plan plan_chunk2(const AttnArgs &a) {
    const Plan inner = plan_chunk(inner_args(a));
    Plan p;
    p.ok = inner.ok && !a.causal && a.d % 4 == 0;
    p.workspace = p.ok ? c2_layout(a, inner.workspace).bytes : 0;
    return p;
}

hipError_t launch_chunk2(const AttnArgs &a, hipStream_t stream) {
    const Plan inner_plan = plan_chunk(inner_args(a));
    const C2Layout w = c2_layout(a, inner_plan.workspace);
    char *ws = reinterpret_cast<char *>(a.workspace);
    if (a.kind == kMaskLit) {   // the mask is all ones in any order: the one-order form is the answer
        AttnArgs b = a;
        b.order = nullptr;
        b.workspace = inner_plan.workspace ? ws + w.inner : nullptr;
        b.workspace_bytes = inner_plan.workspace;
        return launch_chunk(b, stream);
    }
    const size_t rows = (size_t)a.B * a.H * a.L;
    const int esz = a.in_bf16 ? 2 : 4;
    const int pieces = a.d * esz / 16;
    const size_t ng = rows * pieces;
    float *ll2 = a.kind == kMaskS ? reinterpret_cast<float *>(ws + w.ll) : nullptr;
    hipLaunchKernelGGL(c2_gather_kernel, dim3((unsigned)((ng + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                       reinterpret_cast<const u32x4 *>(a.q), reinterpret_cast<const u32x4 *>(a.k),
                       reinterpret_cast<const u32x4 *>(a.v), a.log_lambda, a.order,
                       reinterpret_cast<u32x4 *>(ws + w.q), reinterpret_cast<u32x4 *>(ws + w.k),
                       reinterpret_cast<u32x4 *>(ws + w.v), ll2, a.L, pieces, ng);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the tokens' own order
    AttnArgs b = inner_args(a);
    b.y = ws + w.yb;
    b.den_out = reinterpret_cast<float *>(ws + w.db);
    b.workspace = inner_plan.workspace ? ws + w.inner : nullptr;
    b.workspace_bytes = inner_plan.workspace;
    if ((e = launch_chunk(b, stream)) != hipSuccess) return e;
    // the second order
    AttnArgs c = b;
    c.q = ws + w.q;
    c.k = ws + w.k;
    c.v = ws + w.v;
    if (ll2) c.log_lambda = ll2;
    c.y = ws + w.yc;
    c.den_out = reinterpret_cast<float *>(ws + w.dc);
    if ((e = launch_chunk(c, stream)) != hipSuccess) return e;
    const size_t nc = rows * (a.d / 4);
    hipLaunchKernelGGL(c2_combine_kernel, dim3((unsigned)((nc + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                       reinterpret_cast<const float *>(ws + w.yb), reinterpret_cast<const float *>(ws + w.yc),
                       reinterpret_cast<const float *>(ws + w.db), reinterpret_cast<const float *>(ws + w.dc),
                       a.order, a.y, a.out_bf16 ? 1 : 0, a.den_out, a.L, a.d, nc);
    return hipGetLastError();
}

}  // namespace lion
