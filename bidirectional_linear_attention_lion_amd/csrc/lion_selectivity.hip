// lion_selectivity.hip -- LION-S selectivity prologue: the decays (and the key-path input scale) from the
// layer input.
//
// LION-S's lambda_i is input-dependent, the scalar version of Mamba-2's state matrix ("LION: A
// bidirectional framework that trains like a Transformer and infers like an RNN", reply "1. Some
// equations/notations are not clear enough", Eq. 5a); its two coefficients come from zero-order-hold
// discretisation: exp(a_i) on the state and exp(a_i) - 1 on the input (reply "Concern 8").  Per head h:
//   z_i = x_i . w_h + b_h,   a_i = log(lambda_i) = log sigmoid(z_i),   key scale exp(a_i) - 1 = -sigmoid(-z_i),
// and optionally the scaled raw keys k'_i = (exp(a_i) - 1) k_i, which the attention entry points then take
// as k.  log(lambda) feeds the mask generator of every form directly.
//
// z is a GEMM with a narrow N (the heads): a workgroup computes a 16-token x 16-head tile on the matrix
// cores, A = x rows (16 tokens, 32 channels per step), B = w rows (16 heads), its four waves taking every
// fourth channel step (so four waves per tile wait on memory at once) and adding their partial tiles in
// LDS; the D layout gives lane (r, g) the four consecutive tokens 4g .. 4g+3 of head r, stored as one
// 16-byte vector.  The key scaling reads the tile's 256 scales back from LDS so the 256 key rows are read
// and written coalesced by the whole workgroup.
#include "lion_device.h"
#include "lion_internal.h"

namespace lion {
namespace {

constexpr int kSelWaves = 4;   // waves per 16-token x 16-head tile, splitting the channel sum

struct SelParams {
    const __bf16 *x, *w;
    const float *bias;
    int B, L, H, Dm, d;
    float *ll, *ks;
    const __bf16 *k;
    __bf16 *k_out;
    int tok_tiles, head_tiles;
};

__device__ __forceinline__ float log_sigmoid(float z) {
    // -log(1 + exp(-z)) without overflow: the exponential only of a non-positive argument
    return z >= 0.f ? -log1pf(__expf(-z)) : z - log1pf(__expf(z));
}

__global__ void __launch_bounds__(kSelWaves * 64) selectivity_kernel(SelParams p) {
    __shared__ f32x4 part_sh[kSelWaves][64];        // each wave's partial sums, per lane
    __shared__ float scale_sh[16][17];              // [token][head], padded
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    int bid = blockIdx.x;
    const int ht = bid % p.head_tiles;
    bid /= p.head_tiles;
    const int tt0 = bid % p.tok_tiles;
    const int b = bid / p.tok_tiles;
    const int i0 = tt0 * 16, h0 = ht * 16;          // the workgroup's tile
    const int L = p.L, H = p.H, Dm = p.Dm;

    // A: token i0 + r (clamped; its results are not stored), B: head h0 + r (clamped likewise); wave w
    // takes the 32-channel steps w, w + 4, ...
    const __bf16 *xr = p.x + ((size_t)b * L + min(i0 + r, L - 1)) * Dm + 8 * g;
    const __bf16 *wr = p.w + (size_t)min(h0 + r, H - 1) * Dm + 8 * g;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c0 = 32 * wave; c0 < Dm; c0 += 32 * kSelWaves) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(xr + c0));
        const bf16x8 bw = __builtin_bit_cast(bf16x8, ld16(wr + c0));
        acc = mfma_bf16(a, bw, acc);
    }
    part_sh[wave][lane] = acc;
    __syncthreads();
    acc = part_sh[0][lane];
#pragma unroll
    for (int w2 = 1; w2 < kSelWaves; ++w2) acc += part_sh[w2][lane];
    // acc[e] = z minus bias, token i0 + 4g + e, head h0 + r
    const int h = h0 + r;
    const bool hv = h < H;
    const float bh = hv ? p.bias[h] : 0.f;
    f32x4 llv, ksv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float z = acc[e] + bh;
        llv[e] = log_sigmoid(z);
        ksv[e] = -__builtin_amdgcn_rcpf(1.f + __expf(z));
    }
    const int t0 = i0 + 4 * g;
    if (wave == 0 && hv) {
        const size_t row = ((size_t)b * H + h) * L + t0;
        if (t0 + 3 < L && (L & 3) == 0) {
            *reinterpret_cast<f32x4 *>(p.ll + row) = llv;
            if (p.ks) *reinterpret_cast<f32x4 *>(p.ks + row) = ksv;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (t0 + e < L) {
                    p.ll[row + e] = llv[e];
                    if (p.ks) p.ks[row + e] = ksv[e];
                }
        }
    }
    if (!p.k) return;   // uniform over the workgroup: no barrier follows

    // scaled keys of the tile: rows (head h0 + hh, token i0 + tt), 16-byte chunks spread over the
    // workgroup; every load of a batch is issued before its first store (a chunk is read and written by
    // one lane only, so this holds with k_out == k as well)
    if (wave == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) scale_sh[4 * g + e][r] = ksv[e];
    }
    __syncthreads();
    constexpr int kBatch = 4;
    constexpr int NT = kSelWaves * 64;
    const int tid = threadIdx.x;
    const int cpr = p.d / 8;               // 16-byte chunks per key row
    const int nch = 256 * cpr;
    for (int c0 = 0; c0 < nch; c0 += NT * kBatch) {
        u32x4 kv[kBatch];
        size_t off[kBatch];
        float sc[kBatch];
        bool ok[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int c = c0 + NT * u + tid;
            const int rowi = c / cpr, ch = c % cpr;
            const int hh = rowi / 16, tt = rowi % 16;
            const int hx = h0 + hh, tx = i0 + tt;
            ok[u] = c < nch && hx < H && tx < L;
            off[u] = (((size_t)b * H + min(hx, H - 1)) * L + min(tx, L - 1)) * p.d + 8 * ch;
            sc[u] = scale_sh[tt & 15][hh & 15];
            if (ok[u]) kv[u] = ld16(p.k + off[u]);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (!ok[u]) continue;
            const bf16x8 x8 = __builtin_bit_cast(bf16x8, kv[u]);
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = f2bf(sc[u] * (float)x8[e]);
            st16(p.k_out + off[u], __builtin_bit_cast(u32x4, o));
        }
    }
}

}  // namespace

Plan plan_selectivity(const SelArgs &a) {
    Plan p;
    p.ok = a.Dm % 32 == 0 && (!a.k || a.d % 8 == 0);
    p.workspace = 0;
    return p;
}

hipError_t launch_selectivity(const SelArgs &a, hipStream_t stream) {
    SelParams p;
    p.x = reinterpret_cast<const __bf16 *>(a.x);
    p.w = reinterpret_cast<const __bf16 *>(a.w);
    p.bias = a.bias;
    p.B = a.B;
    p.L = a.L;
    p.H = a.H;
    p.Dm = a.Dm;
    p.d = a.d;
    p.ll = a.log_lambda;
    p.ks = a.key_scale;
    p.k = reinterpret_cast<const __bf16 *>(a.k);
    p.k_out = reinterpret_cast<__bf16 *>(a.k_out);
    p.tok_tiles = (a.L + 15) / 16;
    p.head_tiles = (a.H + 15) / 16;
    const long grid = (long)a.B * p.tok_tiles * p.head_tiles;
    hipLaunchKernelGGL(selectivity_kernel, dim3((unsigned)grid), dim3(kSelWaves * 64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace lion
