// lion_chunk.hip -- chunkwise form of LION bidirectional masked linear attention.
//
// Chunking is how the pages parallelise LION inference when memory is short ("LION: A
// bidirectional framework that trains like a Transformer and infers like an RNN", reply
// "4: Practicality of Recurrent Inference"; blog "LION Part IV - Results", "LION Chunk").  The
// pages print no chunk equations; the ones used here follow from the mask M_ij = exp(-|A_i - A_j|)
// (A = prefix sums of log(lambda)).  For chunk c = tokens s_c .. e_c, a_c = exp(A_{e_c} - A_{e_{c-1}})
// its total decay, and [v, 1] the value row with the row-sum column appended:
//   local states   Fl_c = sum_{j in c} exp(A_{e_c} - A_j)     phi(k_j) [v_j, 1]^T
//                  Gl_c = sum_{j in c} exp(A_j - A_{e_{c-1}}) phi(k_j) [v_j, 1]^T
//   carried states F_c = a_c F_{c-1} + Fl_c   (F_{-1} = 0),   G_c = a_c G_{c+1} + Gl_c   (G_n = 0)
//   out_i = sum_{j in c} M_ij (phi(q_i).phi(k_j)) [v_j, 1]
//           + exp(A_i - A_{e_{c-1}}) phi(q_i)^T F_{c-1} + exp(A_{e_c} - A_i) phi(q_i)^T G_{c+1}
//   y_i = out_i[:d] / (out_i[d] + eps)
// Every exponent is <= 0, and all of them are differences of prefix sums taken inside one chunk, so
// no long-range prefix sum (and its rounding) is ever formed.
//
// Causal variant (keys after the query masked out): only the forward states exist -- out_i keeps the
// intra-chunk keys j <= i and the F_{c-1} term -- so no backward state is folded, scanned or applied.
//
// Three launches, each parallel over (batch, head, chunk):
//   state: one workgroup per chunk stages the chunk's keys and values in LDS and folds them into Fl_c
//          and Gl_c on the matrix cores;
//   scan:  the carried states, elementwise over the d x (d+1) entries, sequential over the chunks of
//          one (batch, head), in place over the local states;
//   out:   one workgroup per chunk: intra-chunk masked attention (matrix-core tiles, mask in
//          registers) plus F_{c-1} and G_{c+1} applied to the decayed queries.
// A state is stored as its d x d value part in the input type plus its row-sum column in fp32.  A fold
// multiplies phi(K)^T by the weighted values w_j v_j; the row-sum column rides along as two extra
// columns of that operand holding w_j as a bf16 high part plus the bf16 rounding of the remainder,
// so the row-sum state -- whose error a nearly cancelling denominator amplifies -- keeps about 2^-17
// relative accuracy.  The value part is stored in the fold's own register layout: lane (r, g) of
// tile (ct, nt) holds state[16 ct + r][16 nt + 4 g + e], which is exactly an A operand of the output
// product when the contraction slots of group g are the key channels 16 nt + 4 g + e; the queries use
// the same channel assignment, so neither side needs a transpose.
#include <type_traits>

#include "lion_device.h"
#include "lion_internal.h"
#include "lion_stage.h"

namespace lion {
namespace {

constexpr int kKB = 32;   // keys per sub-block

__host__ __device__ constexpr int cpad(int C) { return (C + kKB - 1) / kKB * kKB; }
__host__ __device__ constexpr int state_waves(int d) { return d == 128 ? 8 : 4; }

struct ChunkParams {
    const void *q, *k, *v;
    const float *ll;
    float eps;
    int H, L, C, n;        // n: chunks per (batch, head)
    void *y;
    int out_bf16;
    float *den_out;
    unsigned char *fs;     // forward states, [B*H*n] slots
    unsigned char *gs;     // backward states, [B*H*n] slots
    float *tot;            // log2 of each chunk's total decay, [B*H*n]
    int ng;                // resident path: row groups per (batch, head)
    int causal;            // keys after the query masked out: forward states only
};

template <int D, bool BF16>
struct ChunkCfg {
    using T = std::conditional_t<BF16, __bf16, float>;
    using RT = RowTile<D, T>;
    static constexpr int NDT = D / 16;                    // key-channel tiles
    static constexpr int NCT = NDT + 1;                   // value tiles plus the weight tile
    static constexpr int HW = NDT >= 2 ? 2 : 1;           // key-channel tiles per bf16 fragment
    static constexpr int NP = NDT / HW;                   // bf16 fragments over the d channels
    static constexpr int NQ = BF16 ? NP : D / 4;          // query fragments per tile
    using QFrag = std::conditional_t<BF16, bf16x8, float>;
    static constexpr size_t VBYTES = (size_t)D * D * sizeof(T);
    // bf16 slots are whole KiB so a workgroup can copy one into LDS with 1 KiB direct loads
    static constexpr size_t SLOT = BF16 ? (VBYTES + (size_t)D * 4 + 1023) & ~(size_t)1023
                                        : (VBYTES + (size_t)D * 4 + 15) & ~(size_t)15;
};

// Element offset of lane `lane`'s four values of tile (ct, nt) in a state slot's value part.
template <int D, bool BF16>
__device__ __forceinline__ int slot_off(int ct, int nt, int lane) {
    using Cf = ChunkCfg<D, BF16>;
    return (((ct * Cf::NP + nt / Cf::HW) * 64 + lane) * Cf::HW + nt % Cf::HW) * 4;
}

// Contraction channel of fp32 step s for lane group g: channels 16 nt + 4 g + e, s = 4 nt + e.
__device__ __forceinline__ int f32_ch(int s, int g) { return 16 * (s / 4) + 4 * g + (s & 3); }

// LION-S chunk-local exponents E[t] = sum_{u <= t} log2(lambda_{cs + u}) (fp64 scan), for t < rows;
// entries past the chunk's last token repeat its total.  Needs rows <= threads; ends with a barrier.
__device__ void chunk_exponents_s(float *E, double *wsum, const float *ll, int cn, int rows, int tid) {
    double x = tid < cn ? (double)ll[tid] * 1.4426950408889634 : 0.0;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    for (int w = 0; w < wave; ++w) x += wsum[w];
    if (tid < rows) E[tid] = (float)x;
    __syncthreads();
}

// phi over `rows` staged key rows in place (LIT: elu + 1; S: silu, L2-normalised per row).
template <int D, int KIND, typename T>
__device__ __forceinline__ void phi_rows(T *kb, int rows, int tid, int nt) {
    using RT = RowTile<D, T>;
    const int nslot = rows * RT::CPK;
    const int lane = tid & 63;
    for (int sl0 = 0; sl0 < nslot; sl0 += nt) {
        const int sl = sl0 + tid;
        if (sl - lane >= nslot) break;   // whole wave past the end (nslot is a multiple of 64)
        T x[RT::VEC];
        __builtin_memcpy(x, kb + (size_t)sl * RT::VEC, 16);
        float f[RT::VEC], ss = 0.f;
#pragma unroll
        for (int e = 0; e < RT::VEC; ++e) {
            f[e] = phi_pre<KIND>((float)x[e]);
            ss += f[e] * f[e];
        }
        float scl = 1.f;
        if constexpr (KIND == kMaskS) scl = inv_norm(group_sum<RT::CPK>(ss));
#pragma unroll
        for (int e = 0; e < RT::VEC; ++e) x[e] = (T)(f[e] * scl);
        __builtin_memcpy(kb + (size_t)sl * RT::VEC, x, 16);
    }
}

// V^T (or K^T) fragment of sub-block h, channel tile ct, from a row-major staged bf16 tile:
// lane (r, g) gets rows h*32 + {4g + e, 16 + 4g + e} of column 16 ct + r.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16 *tile, int h, int ct, int r, int g) {
    using RT = RowTile<D, __bf16>;
    const int row = h * kKB + 4 * g + (r >> 2), col = 16 * ct + 4 * (r & 3);
    const bf16x4 lo4 = read_tr_b16(tile + RT::off(row, col));
    const bf16x4 hi4 = read_tr_b16(tile + RT::off(row + 16, col));
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = lo4[e];
        f[4 + e] = hi4[e];
    }
    return f;
}

// LDS of the state and output kernels: keys, values, exponent table, scan scratch, and for the bf16
// output kernel the two carried states.
template <int D, bool BF16>
__host__ __device__ size_t chunk_lds(int C, int nw, bool with_states) {
    const int cp = cpad(C);
    // keys, values, exponents, scan scratch, and the state kernel's fold-weight table (2 per key)
    size_t b = 2 * (size_t)cp * D * sizeof(typename ChunkCfg<D, BF16>::T) + (size_t)cp * 4 + (size_t)nw * 8 +
               (size_t)cp * 8;
    b = (b + 15) & ~(size_t)15;
    if (BF16 && with_states) b += 2 * ChunkCfg<D, BF16>::SLOT;
    return b;
}

// Rows of keys or values into a chunk kernel's tile: direct loads, or (bf16 inputs of fp32 arithmetic,
// INB with T = float) converted exactly through registers.
template <int D, typename T, bool INB>
__device__ __forceinline__ void stage_input(T *tile, const void *src, int row0, int nrows, int L, int tid, int nt) {
    if constexpr (INB && !std::is_same_v<T, __bf16>)
        stage_rows_cvt<D>(tile, reinterpret_cast<const __bf16 *>(src), row0, nrows, L, tid, nt);
    else
        stage_rows<D, T>(tile, reinterpret_cast<const T *>(src), row0, nrows, L, uniform(tid >> 6), nt >> 6, tid & 63);
}

// ================================ state kernel ========================================================
template <int D, int KIND, bool BF16, bool INB = BF16>
__global__ void __launch_bounds__(state_waves(D) * 64) chunk_state_kernel(ChunkParams p) {
    using Cf = ChunkCfg<D, BF16>;
    using T = typename Cf::T;
    using RT = typename Cf::RT;
    constexpr int NW = state_waves(D), NT = NW * 64;
    constexpr int NDT = Cf::NDT, NCT = Cf::NCT;
    constexpr bool kColOwn = NW == NDT;   // wave w owns key-channel tile nt = w; ct = u is static
    constexpr int MAXT = (NCT * NDT + NW - 1) / NW;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int L = p.L, n = p.n;
    const int bid = blockIdx.x, bh = bid / n, c = bid % n;
    const int cs = c * p.C, cn = min(p.C, L - cs);
    const int rows = cpad(cn);
    const int cp = cpad(p.C);

    T *Ks = reinterpret_cast<T *>(smem);
    T *Vs = Ks + cp * D;
    float *E = reinterpret_cast<float *>(Vs + cp * D);
    double *wsum = reinterpret_cast<double *>(E + cp);
    const size_t base = (size_t)bh * L;
    using TI = std::conditional_t<INB, __bf16, T>;
    stage_input<D, T, INB>(Ks, reinterpret_cast<const TI *>(p.k) + base * D, cs, rows, L, tid, NT);
    stage_input<D, T, INB>(Vs, reinterpret_cast<const TI *>(p.v) + base * D, cs, rows, L, tid, NT);

    float lgD = 0.f;
    if constexpr (KIND == kMaskD) lgD = p.ll[bh % p.H] * kLog2e;
    if constexpr (KIND == kMaskS) chunk_exponents_s(E, wsum, p.ll + base + cs, cn, rows, tid);
    // exponent of local token t relative to A_{e_{c-1}}
    auto Ex = [&](int t) -> float {
        if constexpr (KIND == kMaskLit) return 0.f;
        else if constexpr (KIND == kMaskD) return (float)(t + 1) * lgD;
        else return E[t];
    };
    wait_vm_all();
    __syncthreads();
    if constexpr (KIND != kMaskD) {
        phi_rows<D, KIND, T>(Ks, rows, tid, NT);
        __syncthreads();
    }
    const float etot = Ex(cn - 1);
    // bf16: the fold weights of every key of the chunk, once per workgroup (0 past the chunk's end); the
    // sub-block loop reads them back four at a time instead of recomputing them in every lane
    float *Wf = reinterpret_cast<float *>(wsum + NW), *Wg = Wf + cp;
    if constexpr (BF16) {
        for (int j = tid; j < cp; j += NT) {
            float a = j < cn ? 1.f : 0.f, b = a;
            if constexpr (KIND != kMaskLit) {
                if (j < cn) {
                    const float ej = Ex(j);
                    a = fast_exp2(fminf(etot - ej, 0.f));
                    b = fast_exp2(fminf(ej, 0.f));
                }
            }
            Wf[j] = a;
            Wg[j] = b;
        }
        __syncthreads();
    }

    auto tile_of = [&](int u, int &ct, int &nt) -> bool {
        if constexpr (kColOwn) {
            ct = u;
            nt = wave;
            return u < NCT;
        } else {
            const int tt = wave + NW * u;
            ct = tt / NDT;
            nt = tt % NDT;
            return tt < NCT * NDT;
        }
    };

    f32x4 sf[MAXT], sg[MAXT];
    float zf[MAXT], zg[MAXT];   // bf16: this lane's part of the row sums of the weight tile
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
        sf[u] = sg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        zf[u] = zg[u] = 0.f;
    }

    for (int h = 0; h < rows / kKB; ++h) {
        // fold weights of the sub-block's tokens 4g + e and 16 + 4g + e; 0 past the chunk's end
        float wf[2][4], wg[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if constexpr (BF16) {
                const f32x4 a4 = *reinterpret_cast<const f32x4 *>(Wf + h * kKB + 16 * t + 4 * g);
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(Wg + h * kKB + 16 * t + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wf[t][e] = a4[e];
                    wg[t][e] = b4[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = h * kKB + 16 * t + 4 * g + e;
                    const float valid = j < cn ? 1.f : 0.f;
                    float a = valid, b = valid;
                    if constexpr (KIND != kMaskLit) {
                        const float ej = Ex(j);
                        a *= fast_exp2(fminf(etot - ej, 0.f));
                        b *= fast_exp2(fminf(ej, 0.f));
                    }
                    wf[t][e] = a;
                    wg[t][e] = b;
                }
            }
        }
        // bf16: the fold weights multiply the key fragment (A operand), once per sub-block, rather than
        // every value tile's B operand: A = bf16(w k) for the value tiles.  The row sums (the weight
        // tile) are accumulated in fp32 on the vector ALU from the same fragment, w times the exact key:
        // a nearly cancelling denominator amplifies their error, so they get no bf16 rounding at all
        bf16x8 af{}, ag{};
        auto weighted = [&](const bf16x8 &kf, const float (&w)[2][4], bf16x8 &hi) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) hi[4 * t + e] = f2bf(w[t][e] * (float)kf[4 * t + e]);
        };
        auto rowsum = [&](const bf16x8 &kf, const float (&w)[2][4], float &z) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) z = fmaf(w[t][e], (float)kf[4 * t + e], z);
        };
        bf16x8 kfr{};
        if constexpr (BF16 && kColOwn) {
            kfr = tr_frag<D>(Ks, h, wave, r, g);
            weighted(kfr, wf, af);
            if (!p.causal) weighted(kfr, wg, ag);
        }
#pragma unroll
        for (int u = 0; u < MAXT; ++u) {
            int ct, nt;
            if (!tile_of(u, ct, nt)) break;
            if constexpr (BF16) {
                if constexpr (!kColOwn) {
                    kfr = tr_frag<D>(Ks, h, nt, r, g);
                    if (ct < NDT) {
                        weighted(kfr, wf, af);
                        if (!p.causal) weighted(kfr, wg, ag);
                    }
                }
                if (ct < NDT) {
                    const bf16x8 vv = tr_frag<D>(Vs, h, ct, r, g);
                    sf[u] = mfma_bf16(af, vv, sf[u]);
                    if (!p.causal) sg[u] = mfma_bf16(ag, vv, sg[u]);
                } else {
                    rowsum(kfr, wf, zf[u]);
                    if (!p.causal) rowsum(kfr, wg, zg[u]);
                }
            } else {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = h * kKB + 16 * t + 4 * g + e;
                        const float a = Ks[RT::off(row, 16 * nt + r)];
                        const float vv = ct < NDT ? Vs[RT::off(row, 16 * ct + r)] : (r == 0 ? 1.f : 0.f);
                        sf[u] = mfma_f32(a, wf[t][e] * vv, sf[u]);
                        if (!p.causal) sg[u] = mfma_f32(a, wg[t][e] * vv, sg[u]);
                    }
            }
        }
    }

    // store: value tiles in register layout, the row sums as fp32
    const bool want_f = c < n - 1, want_g = c > 0 && !p.causal;
    unsigned char *fslot = p.fs + (size_t)bid * Cf::SLOT;
    unsigned char *gslot = p.gs + (size_t)bid * Cf::SLOT;
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
        int ct, nt;
        if (!tile_of(u, ct, nt)) break;
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            if (which == 0 ? !want_f : !want_g) continue;
            const f32x4 s = which == 0 ? sf[u] : sg[u];
            unsigned char *slot = which == 0 ? fslot : gslot;
            if (ct < NDT) {
                T *dst = reinterpret_cast<T *>(slot) + slot_off<D, BF16>(ct, nt, lane);
                if constexpr (BF16) {
                    bf16x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = f2bf(s[e]);
                    *reinterpret_cast<bf16x4 *>(dst) = o;
                } else {
                    *reinterpret_cast<f32x4 *>(dst) = s;
                }
            } else if constexpr (BF16) {
                // lane (r, g) summed key channel 16 nt + r over its keys 4g + e, 16 + 4g + e of every
                // sub-block: the four lane groups' parts added
                float z = which == 0 ? zf[u] : zg[u];
                z += __shfl_xor(z, 16, 64);
                z += __shfl_xor(z, 32, 64);
                if (g == 0) *reinterpret_cast<float *>(slot + Cf::VBYTES + (size_t)(16 * nt + r) * 4) = z;
            } else {
                f32x4 z;
#pragma unroll
                for (int e = 0; e < 4; ++e) z[e] = s[e] + __shfl_xor(s[e], 1, 64);
                if (r == 0) *reinterpret_cast<f32x4 *>(slot + Cf::VBYTES + (size_t)(16 * nt + 4 * g) * 4) = z;
            }
        }
    }
    if (tid == 0) p.tot[bid] = etot;
}

// ================================ scan kernel =========================================================
// One thread per 16-byte vector of a slot, sequential over the chunks of its (batch, head): forward
// states F_c = a_c F_{c-1} + Fl_c for c = 0 .. n-2, backward G_c = a_c G_{c+1} + Gl_c for c = n-1 .. 1,
// each written over the local state of the same chunk.  Loads run kU chunks ahead.
constexpr int kScanThreads = 256;
constexpr int kU = 8;

template <int D, bool BF16>
__host__ __device__ constexpr int scan_vectors() {
    return (int)(ChunkCfg<D, BF16>::VBYTES / 16) + D / 4;
}

template <int D, bool BF16>
__global__ void __launch_bounds__(kScanThreads) chunk_scan_kernel(ChunkParams p) {
    using Cf = ChunkCfg<D, BF16>;
    using T = typename Cf::T;
    constexpr int NVV = (int)(Cf::VBYTES / 16);
    constexpr int NV = scan_vectors<D, BF16>();
    constexpr int NBLK = (NV + kScanThreads - 1) / kScanThreads;
    constexpr int VEC = 16 / (int)sizeof(T);
    const int n = p.n;
    const int bid = blockIdx.x;
    const int blk = bid % NBLK, dir = (bid / NBLK) & 1, bh = bid / (2 * NBLK);
    const int vi = blk * kScanThreads + (int)threadIdx.x;
    if (vi >= NV || (p.causal && dir == 1)) return;   // this kernel has no barriers
    const bool zpart = vi >= NVV;
    const size_t off = zpart ? Cf::VBYTES + (size_t)(vi - NVV) * 16 : (size_t)vi * 16;
    unsigned char *base = (dir == 0 ? p.fs : p.gs) + (size_t)bh * n * Cf::SLOT + off;
    const float *tot = p.tot + (size_t)bh * n;
    const int steps = n - 1;
    auto chunk_of = [&](int k) { return dir == 0 ? k : n - 1 - k; };

    // each chunk's total is loaded with its state vector, kU chunks ahead: vector-memory waits count in
    // issue order, so a total loaded just before its use would also wait for every prefetched vector
    // (loads past the last step reread the last step's chunk, so that every load is unconditional and
    // lands straight in its buffer)
    auto chunk_at = [&](int k) { return chunk_of(min(k, steps - 1)); };
    u32x4 buf[kU];
    float tb[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        buf[u] = ld16(base + (size_t)chunk_at(u) * Cf::SLOT);
        tb[u] = tot[chunk_at(u)];
    }
    float run[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < steps; k0 += kU) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int k = k0 + u;
            if (k >= steps) break;
            const int c = chunk_of(k);
            const u32x4 x = buf[u];
            const float a = fast_exp2(tb[u]);
            buf[u] = ld16(base + (size_t)chunk_at(k + kU) * Cf::SLOT);
            tb[u] = tot[chunk_at(k + kU)];
            u32x4 o;
            if (zpart || !BF16) {
                // whole-vector reinterpretation (a bit_cast of one element of a u32x4 is not used:
                // it has been seen to read element 0 for every index)
                const f32x4 xf = __builtin_bit_cast(f32x4, x);
                f32x4 of;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    run[i] = a * run[i] + xf[i];
                    of[i] = run[i];
                }
                o = __builtin_bit_cast(u32x4, of);
            } else {
                const bf16x8 xb = __builtin_bit_cast(bf16x8, x);
                bf16x8 ob;
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    run[i] = a * run[i] + (float)xb[i];
                    ob[i] = f2bf(run[i]);
                }
                o = __builtin_bit_cast(u32x4, ob);
            }
            st16(base + (size_t)c * Cf::SLOT, o);
        }
    }
}

// ================================ output kernel =======================================================
template <int D, int KIND, int NW, int QT, bool BF16, bool INB = BF16>
__global__ void __launch_bounds__(NW * 64) chunk_out_kernel(ChunkParams p) {
    using Cf = ChunkCfg<D, BF16>;
    using T = typename Cf::T;
    using RT = typename Cf::RT;
    using QFrag = typename Cf::QFrag;
    constexpr int NT = NW * 64;
    constexpr int NDT = Cf::NDT, NQ = Cf::NQ, HW = Cf::HW;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int L = p.L, n = p.n;
    const int bid = blockIdx.x, bh = bid / n, c = bid % n;
    const int cs = c * p.C, cn = min(p.C, L - cs);
    const int rows = cpad(cn);
    const int cp = cpad(p.C);
    const int tiles = (cn + 15) / 16;

    T *Ks = reinterpret_cast<T *>(smem);
    T *Vs = Ks + cp * D;
    float *E = reinterpret_cast<float *>(Vs + cp * D);
    double *wsum = reinterpret_cast<double *>(E + cp);
    // bf16: the carried states F_{c-1} and G_{c+1} are copied into LDS beside the keys and values
    unsigned char *Fsm = reinterpret_cast<unsigned char *>(smem) + chunk_lds<D, BF16>(p.C, NW, false);
    unsigned char *Gsm = Fsm + Cf::SLOT;
    const size_t base = (size_t)bh * L;
    using TI = std::conditional_t<INB, __bf16, T>;
    stage_input<D, T, INB>(Ks, reinterpret_cast<const TI *>(p.k) + base * D, cs, rows, L, tid, NT);
    stage_input<D, T, INB>(Vs, reinterpret_cast<const TI *>(p.v) + base * D, cs, rows, L, tid, NT);
    if constexpr (BF16) {
        if (c > 0) stage_flat(Fsm, p.fs + (size_t)(bid - 1) * Cf::SLOT, (int)(Cf::SLOT / 1024), wave, NW, lane);
        if (c < n - 1 && !p.causal)
            stage_flat(Gsm, p.gs + (size_t)(bid + 1) * Cf::SLOT, (int)(Cf::SLOT / 1024), wave, NW, lane);
    }

    float lgD = 0.f;
    if constexpr (KIND == kMaskD) lgD = p.ll[bh % p.H] * kLog2e;
    if constexpr (KIND == kMaskS) chunk_exponents_s(E, wsum, p.ll + base + cs, cn, rows, tid);
    auto Ex = [&](int t) -> float {
        if constexpr (KIND == kMaskLit) return 0.f;
        else if constexpr (KIND == kMaskD) return (float)(t + 1) * lgD;
        else return E[t];
    };
    const float etot = Ex(cn - 1);

    // ---- queries of this wave's tiles (channels in fragment order), phi, decay exponents ---------
    QFrag qf[QT][NQ];
    float Ei[QT], den[QT];
    f32x4 acc[QT][NDT];
    const TI *qg = reinterpret_cast<const TI *>(p.q) + base * D;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int tl = wave + NW * qt;
        const int il = 16 * tl + r;
        const bool ok = tl < tiles && il < cn;
        const TI *src = qg + (size_t)(cs + min(il, cn - 1)) * D + 4 * g;
        float x[NQ][8];
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
            if constexpr (BF16) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    if (hh < HW) {
                        const bf16x4 v4 = *reinterpret_cast<const bf16x4 *>(src + 16 * (HW * s + hh));
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[s][4 * hh + e] = phi_pre<KIND>((float)v4[e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[s][4 * hh + e] = 0.f;
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += x[s][e] * x[s][e];
            } else {
                x[s][0] = phi_pre<KIND>((float)src[16 * (s / 4) + (s & 3)]);
                ss += x[s][0] * x[s][0];
            }
        }
        float sc = ok ? 1.f : 0.f;
        if constexpr (KIND == kMaskS) {
            ss += __shfl_xor(ss, 16, 64);
            ss += __shfl_xor(ss, 32, 64);
            sc *= inv_norm(ss);
        }
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
            if constexpr (BF16) {
                bf16x8 f;
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = f2bf(x[s][e] * sc);
                qf[qt][s] = f;
            } else {
                qf[qt][s] = x[s][0] * sc;
            }
        }
        Ei[qt] = Ex(ok ? il : 0);
        den[qt] = 0.f;
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) acc[qt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    wait_vm_all();
    __syncthreads();

    // ---- inter-chunk terms: F_{c-1} on exp(A_i - A_{e_{c-1}}) q_i, G_{c+1} on exp(A_{e_c} - A_i) q_i ----
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        if (which == 0 ? c == 0 : (c == n - 1 || p.causal)) continue;
        const unsigned char *slot;
        if constexpr (BF16) slot = which == 0 ? Fsm : Gsm;
        else slot = which == 0 ? p.fs + (size_t)(bid - 1) * Cf::SLOT : p.gs + (size_t)(bid + 1) * Cf::SLOT;
        const T *sv = reinterpret_cast<const T *>(slot);
        const float *sz = reinterpret_cast<const float *>(slot + Cf::VBYTES);
        f32x4 z4[NDT];
#pragma unroll
        for (int nt = 0; nt < NDT; ++nt) z4[nt] = *reinterpret_cast<const f32x4 *>(sz + 16 * nt + 4 * g);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            if (wave + NW * qt >= tiles) break;
            float dq = 1.f;
            if constexpr (KIND != kMaskLit) dq = which == 0 ? fast_exp2(Ei[qt]) : fast_exp2(etot - Ei[qt]);
            float zdot = 0.f;
            QFrag qd[NQ];
#pragma unroll
            for (int s = 0; s < NQ; ++s) {
                if constexpr (BF16) {
                    bf16x8 f;
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const float xv = (float)qf[qt][s][k];
                        if (k / 4 < HW) zdot += xv * z4[HW * s + k / 4][k & 3];
                        f[k] = f2bf(dq * xv);
                    }
                    qd[s] = f;
                } else {
                    zdot += qf[qt][s] * z4[s / 4][s & 3];
                    qd[s] = dq * qf[qt][s];
                }
            }
            den[qt] += dq * zdot;
#pragma unroll
            for (int ct = 0; ct < NDT; ++ct) {
                if constexpr (BF16) {
#pragma unroll
                    for (int s = 0; s < NQ; ++s) {
                        const T *src = sv + slot_off<D, BF16>(ct, HW * s, lane);
                        bf16x8 a;
                        if constexpr (HW == 2) {
                            a = *reinterpret_cast<const bf16x8 *>(src);
                        } else {
                            const bf16x4 h4 = *reinterpret_cast<const bf16x4 *>(src);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                a[e] = h4[e];
                                a[4 + e] = f2bf(0.f);
                            }
                        }
                        acc[qt][ct] = mfma_bf16(a, qd[s], acc[qt][ct]);
                    }
                } else {
#pragma unroll
                    for (int nt = 0; nt < NDT; ++nt) {
                        const f32x4 a4 = *reinterpret_cast<const f32x4 *>(sv + slot_off<D, BF16>(ct, nt, lane));
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[qt][ct] = mfma_f32(a4[e], qd[4 * nt + e], acc[qt][ct]);
                    }
                }
            }
        }
    }

    // ---- intra-chunk masked attention -----------------------------------------------------------
    if constexpr (KIND != kMaskD) {
        phi_rows<D, KIND, T>(Ks, rows, tid, NT);
        __syncthreads();
    }
    // causal: the last query row of this wave's tiles bounds the keys it needs
    const int wlast = 16 * (wave + NW * ((tiles - 1 - wave) / NW)) + 15;
    for (int h = 0; h < rows / kKB; ++h) {
        const int j0 = h * kKB;
        const bool partial = j0 + kKB > cn;
        if (wave >= tiles) break;
        if (p.causal && j0 > wlast) break;
        bf16x8 vfr[BF16 ? NDT : 1];
        if constexpr (BF16) {
#pragma unroll
            for (int ct = 0; ct < NDT; ++ct) vfr[ct] = tr_frag<D>(Vs, h, ct, r, g);
        }
        QFrag kf[2][BF16 ? NQ : 1];
        if constexpr (BF16) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int s = 0; s < NQ; ++s) {
                    const int row = j0 + 16 * t + r;
                    bf16x8 f;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        if (hh < HW) {
                            const bf16x4 v4 =
                                *reinterpret_cast<const bf16x4 *>(Ks + RT::off(row, 16 * (HW * s + hh) + 4 * g));
#pragma unroll
                            for (int e = 0; e < 4; ++e) f[4 * hh + e] = v4[e];
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) f[4 * hh + e] = f2bf(0.f);
                        }
                    }
                    kf[t][s] = f;
                }
        }
        float Ej[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) Ej[t][e] = Ex(j0 + 16 * t + 4 * g + e);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            if (wave + NW * qt >= tiles) break;
            f32x4 sa[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                sa[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NQ; ++s) {
                    if constexpr (BF16)
                        sa[t] = mfma_bf16(kf[t][s], qf[qt][s], sa[t]);
                    else
                        sa[t] = mfma_f32(Ks[RT::off(j0 + 16 * t + r, f32_ch(s, g))], qf[qt][s], sa[t]);
                }
            }
            float pv[2][4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float pe = sa[t][e];
                    if constexpr (KIND != kMaskLit) pe *= fast_exp2(-__builtin_fabsf(Ei[qt] - Ej[t][e]));
                    pv[t][e] = pe;
                }
            // keys past the chunk's end, and (causal) keys after the query: both rare, so the masking is
            // behind wave-uniform branches
            if (partial) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) pv[t][e] = j0 + 16 * t + 4 * g + e < cn ? pv[t][e] : 0.f;
            }
            if (p.causal && j0 + kKB - 1 > 16 * (wave + NW * qt)) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (j0 + 16 * t + 4 * g + e > 16 * (wave + NW * qt) + r) pv[t][e] = 0.f;
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
                for (int ct = 0; ct < NDT; ++ct) acc[qt][ct] = mfma_bf16(vfr[ct], pf, acc[qt][ct]);
            } else {
#pragma unroll
                for (int ct = 0; ct < NDT; ++ct)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[qt][ct] =
                                mfma_f32(Vs[RT::off(j0 + 16 * t + 4 * g + e, 16 * ct + r)], pv[t][e], acc[qt][ct]);
            }
        }
    }

    // ---- epilogue ------------------------------------------------------------------------------
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int tl = wave + NW * qt;
        if (tl >= tiles) break;
        float dsum = den[qt];
        dsum += __shfl_xor(dsum, 16, 64);
        dsum += __shfl_xor(dsum, 32, 64);
        const float div = dsum + p.eps;
        const int il = 16 * tl + r;
        if (il < cn) {
            const float inv = 1.f / div;
            const size_t row = base + cs + il;
            if (p.out_bf16) {
                __bf16 *yo = reinterpret_cast<__bf16 *>(p.y) + row * D;
#pragma unroll
                for (int ct = 0; ct < NDT; ++ct) {
                    bf16x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = f2bf(acc[qt][ct][e] * inv);
                    *reinterpret_cast<bf16x4 *>(yo + 16 * ct + 4 * g) = o;
                }
            } else {
                float *yo = reinterpret_cast<float *>(p.y) + row * D;
#pragma unroll
                for (int ct = 0; ct < NDT; ++ct) {
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

// ================================ resident kernel =====================================================
// Short sequences -- every key and value row of a (batch, head) fits in LDS (at most 256 rows, so at
// most 4 chunks): one workgroup of 16 waves per (batch, head), one launch, no workspace.  Waves
// 4c .. 4c+3 fold chunk c into its local states Fl_c and Gl_c, which stay in LDS; then wave w computes
// query tile w: its chunk's intra-chunk attention plus every other chunk's local state applied to the
// query with the decay in between,
//   F_{c-1} q = sum_{c' < c} exp(A_{e_{c-1}} - A_{e_{c'}}) Fl_{c'} q,
//   G_{c+1} q = sum_{c' > c} exp(A_{e_{c'-1}} - A_{e_c}) Gl_{c'} q,
// a direct sum over at most three states in place of the carried scan.  Keys pass through registers
// on their way into LDS: phi is applied there and rows past L are zeroed, so padded keys add nothing to
// any state, score or row sum and no later step masks them.
//
// Longer sequences with C = 64 are cut into row groups of whole chunks (128 rows) and take
// three launches: a group-state kernel folds each group's keys straight into the group's own states
// (forward relative to the group's last token, backward relative to the token before its first); a
// scan over the groups turns these into carried states in place; and this kernel processes each group
// as above (a 128-row group is one workgroup of 8 waves, two per CU), with the carried states of all
// earlier and of all later groups as two more states applied to every query of the group.
constexpr int kFuseRows = 256;    // one launch up to this many rows
constexpr int kGroupRows = 128;   // row group of longer sequences (C = 64)

__host__ __device__ constexpr bool fused_ok(int L, int C, int d, bool bf16) {
    return bf16 && d <= 64 && C % 64 == 0 && L >= 1 && (L <= kFuseRows || C == 64);
}
__host__ __device__ constexpr int fused_rows(int L, int C) { return L <= kFuseRows ? kFuseRows : kGroupRows; }
__host__ __device__ constexpr int fused_groups(int L, int C) { return (L + fused_rows(L, C) - 1) / fused_rows(L, C); }

// Contraction fragments over the key channels: fragment s of lane (r, g) holds the eight consecutive
// channels 32 s + 8 g .. 32 s + 8 g + 7 (d = 16: lanes g >= 2 hold zeros), so a query or key fragment
// is one 16-byte read.  A state slot holds, per 16-wide value tile ct and fragment s, the A operand
// state[16 ct + r][channels of (s, g)], followed by the row sums as a two-row A-operand tile (row 0
// their bf16 high part, row 1 the bf16 rounding of the remainder).
template <int D>
struct Fuse {
    static constexpr int NDT = D / 16;
    static constexpr int NF = (D + 31) / 32;
    static constexpr int VB = NDT * NF * 1024;
    static constexpr int SLOT = VB + NF * 128;
    static constexpr int SLOTK = (SLOT + 1023) & ~1023;   // a group state in the workspace: whole KiB
    // element offsets: fragment s of value tile ct as read by `lane`
    __device__ static __forceinline__ int rd(int ct, int s, int lane) { return ((ct * NF + s) * 64 + lane) * 8; }
    // where lane (r, g) of a fold tile (ct, nt), holding channels 16 nt + 4 g + e, writes its four values
    __device__ static __forceinline__ int wr(int ct, int nt, int r, int g) {
        return ((ct * NF + nt / 2) * 64 + (2 * (nt % 2) + g / 2) * 16 + r) * 8 + 4 * (g % 2);
    }
    // row-sum tile: row rr (0 or 1) of fragment s as read by group g, and where fold lane (rr, g) of tile nt writes
    __device__ static __forceinline__ int zrd(int s, int rr, int g) { return ((s * 2 + rr) * 4 + g) * 8; }
    __device__ static __forceinline__ int zwr(int nt, int rr, int g) {
        return (((nt / 2) * 2 + rr) * 4 + 2 * (nt % 2) + g / 2) * 8 + 4 * (g % 2);
    }
    // whether group g's channels of a fragment exist (only d = 16 has empty groups)
    __device__ static __forceinline__ bool has_ch(int g) { return 8 * g < D || D >= 32; }
};

// Chunk-local states a ROWS-row workgroup keeps in LDS: forward states of chunks 0 .. NCH-2 and
// backward states of chunks 1 .. NCH-1 (the only ones ever read), NCH = ROWS / 64 the most chunks a
// group holds; LIT: one state per chunk.
template <int KIND, int ROWS>
__host__ __device__ constexpr int fuse_slots() { return KIND == kMaskLit ? ROWS / 64 : 2 * (ROWS / 64) - 2; }

// LDS of the resident kernel: [K rows][V rows][chunk states][incoming F, G][E][totals][scratch]
template <int D, int KIND, int ROWS>
__host__ __device__ constexpr size_t fused_lds(bool incoming) {
    return 2 * (size_t)ROWS * D * 2 + (size_t)fuse_slots<KIND, ROWS>() * Fuse<D>::SLOT +
           (incoming ? 2 * (size_t)Fuse<D>::SLOTK : 0) + (size_t)ROWS * 4 + 16 * 4 + 16 * 8 +
           2 * (size_t)ROWS * 4;   // + the fold-weight table
}

// LION-S exponents relative to each chunk's start, E[t] = sum_{u = cs(t)}^{t} log2(lambda_u): one fp64 scan
// over the sequence (threads 0 .. 255), differenced in fp64 at the chunk starts; positions past L - 1
// get the last chunk's total.  `llt` is thread tid's log(lambda) (0 past L), loaded by the caller ahead
// of its other loads.  Needs rows <= 256; all threads call it.
__device__ __forceinline__ float load_ll(const float *ll, int L, int tid) { return tid < L ? ll[tid] : 0.f; }
__device__ void fused_exponents_s(float *E, double *sh, float llt, int L, int C, int rows, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
    double x = (double)llt * 1.4426950408889634;
    if (wave < 4) {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (lane == 63) sh[wave] = x;
    }
    __syncthreads();
    if (wave < 4)
        for (int w = 0; w < wave; ++w) x += sh[w];
    if (tid == 0) sh[4] = 0.0;
    if (tid < rows && (tid + 1) % C == 0 && (tid + 1) / C < 4) sh[4 + (tid + 1) / C] = x;
    __syncthreads();
    if (tid < rows) E[tid] = (float)(x - sh[4 + tid / C]);
    __syncthreads();
}

template <int D, int KIND, int ROWS>
__global__ void __launch_bounds__(ROWS / 16 * 64) chunk_fused_kernel(ChunkParams p) {
    using F = Fuse<D>;
    using T = __bf16;
    using RT = RowTile<D, T>;
    constexpr int NW = ROWS / 16, NT = NW * 64, NCH = ROWS / 64;
    constexpr int NDT = F::NDT, NCT = NDT + 1, NF = F::NF;
    constexpr bool kColOwn = NDT == 4;   // the 4 waves of a chunk own one key-channel tile each
    constexpr int MAXT = (NCT * NDT + 3) / 4;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int C = p.C, ng = p.ng;
    const int bh = blockIdx.x / ng, gi = blockIdx.x % ng;   // (batch, head) and row group
    const int L = min(ROWS, p.L - gi * ROWS);                 // rows of this group
    const int n = (L + C - 1) / C;                           // chunks of this group
    const int rows = cpad(L);
    const size_t base = (size_t)bh * p.L + (size_t)gi * ROWS;
    const bool has_fin = gi > 0, has_gin = gi + 1 < ng && !p.causal;

    T *Ks = reinterpret_cast<T *>(smem);
    T *Vs = Ks + ROWS * D;
    unsigned char *sl = reinterpret_cast<unsigned char *>(Vs + ROWS * D);
    unsigned char *fin = sl + fuse_slots<KIND, ROWS>() * F::SLOT;
    unsigned char *gin = fin + F::SLOTK;
    float *E = reinterpret_cast<float *>(fin + (ng > 1 ? 2 * F::SLOTK : 0));
    float *tot = E + ROWS;
    double *sh = reinterpret_cast<double *>(tot + 16);
    // forward state of chunk c (c <= NCH - 2; LIT: any c), backward state of chunk c (c >= 1)
    auto fslot = [&](int c) { return sl + (size_t)c * F::SLOT; };
    auto gslot = [&](int c) { return sl + (size_t)(NCH - 2 + c) * F::SLOT; };

    // log(lambda) first (its wait does not wait for the bulk loads behind it); values straight to LDS,
    // keys into registers; the carried states of the other groups straight to LDS
    const float llt = KIND == kMaskS ? load_ll(p.ll + base, L, tid) : 0.f;
    stage_rows<D, T>(Vs, reinterpret_cast<const T *>(p.v) + base * D, 0, rows, L, wave, NW, lane);
    if (has_fin) stage_flat(fin, p.fs + (size_t)(blockIdx.x - 1) * F::SLOTK, F::SLOTK / 1024, wave, NW, lane);
    if (has_gin) stage_flat(gin, p.gs + (size_t)(blockIdx.x + 1) * F::SLOTK, F::SLOTK / 1024, wave, NW, lane);
    constexpr int KPER = (ROWS * RT::CPK + NT - 1) / NT;   // 16-byte key chunks per thread
    u32x4 kx[KPER];
    {
        const T *kg = reinterpret_cast<const T *>(p.k) + base * D;
#pragma unroll
        for (int u = 0; u < KPER; ++u) {
            const int c16 = min(tid + u * NT, rows * RT::CPK - 1);
            kx[u] = ld16(kg + (size_t)min(c16 / RT::CPK, L - 1) * D + (c16 % RT::CPK) * RT::VEC);
        }
    }
    // this wave's query tile: row 16 wave + r, fragment s = channels 32 s + 8 g .. + 7
    const int ntiles = (L + 15) / 16;
    const int i = 16 * wave + r;
    u32x4 qraw[NF];
    {
        const T *src = reinterpret_cast<const T *>(p.q) + (base + min(i, L - 1)) * D;
#pragma unroll
        for (int s = 0; s < NF; ++s) qraw[s] = ld16(src + min(32 * s + 8 * g, D - 8));
    }

    float lgD = 0.f;
    if constexpr (KIND == kMaskD) lgD = p.ll[bh % p.H] * kLog2e;
    if constexpr (KIND == kMaskS) fused_exponents_s(E, sh, llt, L, C, rows, tid);
    // exponent of token t of the chunk starting at cs, relative to the end of the chunk before it
    auto Ex = [&](int t, int cs) -> float {
        if constexpr (KIND == kMaskLit) return 0.f;
        else if constexpr (KIND == kMaskD) return (float)(t - cs + 1) * lgD;
        else return E[t];
    };
    wait_vm_all();
    // phi on the keys (rows past L written as zeros); a row's chunks sit in consecutive lanes
#pragma unroll
    for (int u = 0; u < KPER; ++u) {
        const int c16 = tid + u * NT, row = c16 / RT::CPK;
        u32x4 o;
        if constexpr (KIND == kMaskD) {
            o = row < L ? kx[u] : u32x4{0u, 0u, 0u, 0u};
        } else {
            const bf16x8 x = __builtin_bit_cast(bf16x8, kx[u]);
            float f[8], ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                f[e] = phi_pre<KIND>((float)x[e]);
                ss += f[e] * f[e];
            }
            float scl = row < L ? 1.f : 0.f;
            if constexpr (KIND == kMaskS) scl *= inv_norm(group_sum<RT::CPK>(ss));
            bf16x8 y;
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = f2bf(f[e] * scl);
            o = __builtin_bit_cast(u32x4, y);
        }
        if (c16 < rows * RT::CPK) st16(Ks + RT::off(row, (c16 % RT::CPK) * RT::VEC), o);
    }
    // fold weights of every row of the group, forward and backward relative to its own chunk, once per
    // workgroup; the fold reads them four at a time
    float *W = reinterpret_cast<float *>(sh + 16);   // [2][ROWS]
    if constexpr (KIND != kMaskLit) {
        for (int t = tid; t < rows; t += NT) {
            const int ccs = (t / C) * C, ccn = min(C, L - ccs);
            const float ej = Ex(t, ccs);
            W[t] = fast_exp2(fminf(Ex(ccs + ccn - 1, ccs) - ej, 0.f));
            W[ROWS + t] = fast_exp2(fminf(ej, 0.f));
        }
    }
    __syncthreads();

    // ---- fold: waves 4c .. 4c+3 -> Fl_c, Gl_c ---------------------------------------------------
    // A wave always uses one key-channel tile nt (A operand), so the per-key fold weights are applied
    // once per sub-block to that fragment; the value fragments enter the products unweighted.  The
    // row sums are accumulated in fp32 on the vector ALU, w times the exact key, and stored as a bf16
    // high part plus the bf16 rounding of the remainder (~2^-17).
    if (wave < 4 * n) {
        const int c = wave >> 2, k = wave & 3;
        const int cs = c * C, cn = min(C, L - cs);
        const float etot = Ex(cs + cn - 1, cs);
        const int nt = k % NDT;
        auto ct_of = [&](int u) { return kColOwn ? u : (k + 4 * u) / NDT; };
        auto has = [&](int u) { return kColOwn ? u < NCT : k + 4 * u < NCT * NDT; };
        f32x4 sf[MAXT], sg[MAXT];
#pragma unroll
        for (int u = 0; u < MAXT; ++u) sf[u] = sg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        float zf = 0.f, zg = 0.f;   // row sums of key channel 16 nt + r over this lane's keys
        for (int h = cs / kKB; h < (cs + cpad(cn)) / kKB; ++h) {
            float wf[2][4], wg[2][4];
            if constexpr (KIND != kMaskLit) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4 *>(W + h * kKB + 16 * t + 4 * g);
                    const f32x4 b4 = *reinterpret_cast<const f32x4 *>(W + ROWS + h * kKB + 16 * t + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        wf[t][e] = a4[e];
                        wg[t][e] = b4[e];
                    }
                }
            }
            const bf16x8 kfr = tr_frag<D>(Ks, h, nt, r, g);
            bf16x8 af = kfr, ag = kfr;
            if constexpr (KIND != kMaskLit) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float kv = (float)kfr[4 * t + e];
                        af[4 * t + e] = f2bf(wf[t][e] * kv);
                        ag[4 * t + e] = f2bf(wg[t][e] * kv);
                    }
            }
#pragma unroll
            for (int u = 0; u < MAXT; ++u) {
                if (!has(u)) break;
                const int ct = ct_of(u);
                if (ct < NDT) {
                    const bf16x8 vv = tr_frag<D>(Vs, h, ct, r, g);
                    sf[u] = mfma_bf16(af, vv, sf[u]);
                    if (KIND != kMaskLit && !p.causal) sg[u] = mfma_bf16(ag, vv, sg[u]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float kv = (float)kfr[e];
                        if constexpr (KIND == kMaskLit) {
                            zf += kv;
                        } else {
                            zf = fmaf(wf[e / 4][e % 4], kv, zf);
                            zg = fmaf(wg[e / 4][e % 4], kv, zg);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < MAXT; ++u) {
            if (!has(u)) break;
            const int ct = ct_of(u);
#pragma unroll
            for (int which = 0; which < (KIND == kMaskLit ? 1 : 2); ++which) {
                // LIT: the two local states coincide; one copy in the forward slot serves both.  The last
                // chunk's forward and the first chunk's backward state are never read.
                if (KIND != kMaskLit && (which == 0 ? c == n - 1 : (c == 0 || p.causal))) continue;
                const f32x4 sv = which == 0 ? sf[u] : sg[u];
                T *slot = reinterpret_cast<T *>(which == 0 ? fslot(c) : gslot(c));
                bf16x4 o;
                if (ct < NDT) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = f2bf(sv[e]);
                    *reinterpret_cast<bf16x4 *>(slot + F::wr(ct, nt, r, g)) = o;
                } else {
                    // row sums z[16 nt + 4 g + e]: this lane's part summed over the four lane groups, then
                    // gathered from the lane holding channel 16 nt + 4 g + e
                    float zs = which == 0 ? zf : zg;
                    zs += __shfl_xor(zs, 16, 64);
                    zs += __shfl_xor(zs, 32, 64);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float z = __shfl(zs, 4 * g + e, 64);
                        const __bf16 zh = f2bf(z);
                        o[e] = r == 0 ? zh : f2bf(z - (float)zh);
                    }
                    if (r < 2) *reinterpret_cast<bf16x4 *>(slot + F::VB / 2 + F::zwr(nt, r, g)) = o;
                }
            }
        }
        if (k == 0 && lane == 0) tot[c] = etot;
    }
    __syncthreads();
    if (wave >= ntiles) return;   // no barriers below

    // ---- query tile `wave` of chunk c -----------------------------------------------------------
    const int c = (16 * wave) / C;
    const int cs = c * C, cn = min(C, L - cs);
    const bool ok = i < cs + cn;
    const float etot = tot[c];
    bf16x8 qf[NF];
    float Ei, den = 0.f;
    f32x4 acc[NDT];
    {
        float x[NF][8];
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < NF; ++s) {
            const bf16x8 qv = __builtin_bit_cast(bf16x8, qraw[s]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xv = F::has_ch(g) ? phi_pre<KIND>((float)qv[e]) : 0.f;
                x[s][e] = xv;
                ss += xv * xv;
            }
        }
        float sc = ok ? 1.f : 0.f;
        if constexpr (KIND == kMaskS) {
            ss += __shfl_xor(ss, 16, 64);
            ss += __shfl_xor(ss, 32, 64);
            sc *= inv_norm(ss);
        }
#pragma unroll
        for (int s = 0; s < NF; ++s) {
            bf16x8 f;
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = f2bf(x[s][e] * sc);
            qf[s] = f;
        }
        Ei = Ex(ok ? i : cs, cs);
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // other chunks' local states applied to the query; the decay between them scales the product
    f32x4 accz = f32x4{0.f, 0.f, 0.f, 0.f};   // row sums: rows 0 (high part) and 1 (low part) of a tile
    // chunks -1 and n stand for the carried states of all earlier and all later groups
    // (causal: earlier chunks and groups only)
    const int c2_end = p.causal ? c : (has_gin ? n + 1 : n);
    for (int c2 = has_fin ? -1 : 0; c2 < c2_end; ++c2) {
        if (c2 == c) continue;
        float ex = c2 < c ? Ei : etot - Ei;
        for (int c3 = min(c, c2) + 1; c3 < max(c, c2); ++c3) ex += tot[c3];
        const unsigned char *sb = c2 < 0 ? fin : c2 == n ? gin : (c2 < c || KIND == kMaskLit) ? fslot(c2) : gslot(c2);
        const T *sv = reinterpret_cast<const T *>(sb);
        // every LDS read of the slot is issued before the first product, so their latencies overlap
        bf16x8 sa[NDT][NF], za[NF];
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct)
#pragma unroll
            for (int s = 0; s < NF; ++s) {
                sa[ct][s] = bf16x8{};
                if (F::has_ch(g)) sa[ct][s] = *reinterpret_cast<const bf16x8 *>(sv + F::rd(ct, s, lane));
            }
#pragma unroll
        for (int s = 0; s < NF; ++s) {
            za[s] = bf16x8{};
            if (r < 2 && F::has_ch(g)) za[s] = *reinterpret_cast<const bf16x8 *>(sv + F::VB / 2 + F::zrd(s, r, g));
        }
        if constexpr (KIND == kMaskLit) {
#pragma unroll
            for (int s = 0; s < NF; ++s) {
#pragma unroll
                for (int ct = 0; ct < NDT; ++ct) acc[ct] = mfma_bf16(sa[ct][s], qf[s], acc[ct]);
                accz = mfma_bf16(za[s], qf[s], accz);
            }
        } else {
            const float dq = fast_exp2(ex);
            f32x4 tv[NDT], tz = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ct = 0; ct < NDT; ++ct) tv[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NF; ++s) {
#pragma unroll
                for (int ct = 0; ct < NDT; ++ct) tv[ct] = mfma_bf16(sa[ct][s], qf[s], tv[ct]);
                tz = mfma_bf16(za[s], qf[s], tz);
            }
#pragma unroll
            for (int ct = 0; ct < NDT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[ct][e] += dq * tv[ct][e];
            accz[0] += dq * tz[0];
            accz[1] += dq * tz[1];
        }
    }
    // rows 0 and 1 of the row-sum tile sit in lanes g = 0 (elements 0, 1); other lanes hold zeros
    den += accz[0] + accz[1];

    // intra-chunk attention over the chunk's keys (padded keys are zero rows: no mask needed; causal:
    // keys after the query zeroed, sub-blocks wholly after the tile skipped)
    for (int h = cs / kKB; h < (cs + cpad(cn)) / kKB; ++h) {
        const int j0 = h * kKB;
        if (p.causal && j0 > 16 * wave + 15) break;
        bf16x8 vfr[NDT], kf[2][NF];
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) vfr[ct] = tr_frag<D>(Vs, h, ct, r, g);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int s = 0; s < NF; ++s) {
                kf[t][s] = bf16x8{};
                if (F::has_ch(g)) kf[t][s] = *reinterpret_cast<const bf16x8 *>(Ks + RT::off(j0 + 16 * t + r, 32 * s + 8 * g));
            }
        f32x4 sa[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            sa[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NF; ++s) sa[t] = mfma_bf16(kf[t][s], qf[s], sa[t]);
        }
        bf16x8 pf;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float pe = sa[t][e];
                if constexpr (KIND != kMaskLit) pe *= fast_exp2(-__builtin_fabsf(Ei - Ex(j0 + 16 * t + 4 * g + e, cs)));
                if (p.causal && j0 + 16 * t + 4 * g + e > i) pe = 0.f;
                den += pe;
                pf[4 * t + e] = f2bf(pe);
            }
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) acc[ct] = mfma_bf16(vfr[ct], pf, acc[ct]);
    }

    // epilogue
    den += __shfl_xor(den, 16, 64);
    den += __shfl_xor(den, 32, 64);
    const float div = den + p.eps;
    if (ok) {
        const float inv = 1.f / div;
        const size_t row = base + i;
        if (p.out_bf16) {
            __bf16 *yo = reinterpret_cast<__bf16 *>(p.y) + row * D;
#pragma unroll
            for (int ct = 0; ct < NDT; ++ct) {
                bf16x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = f2bf(acc[ct][e] * inv);
                *reinterpret_cast<bf16x4 *>(yo + 16 * ct + 4 * g) = o;
            }
        } else {
            float *yo = reinterpret_cast<float *>(p.y) + row * D;
#pragma unroll
            for (int ct = 0; ct < NDT; ++ct) {
                f32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = acc[ct][e] * inv;
                *reinterpret_cast<f32x4 *>(yo + 16 * ct + 4 * g) = o;
            }
        }
        if (p.den_out && g == 0) p.den_out[row] = div;
    }
}

// ================================ group states ========================================================
// The own states of one row group (ROWS rows, whole chunks) of a long sequence, folded straight from the
// group's keys and values: Fg = sum_j 2^(E_last - E_j) phi(k_j) [v_j, 1]^T (relative to the group's
// last token) and Gg = sum_j 2^(E_j) phi(k_j) [v_j, 1]^T (relative to the token before its first),
// E_j = log2 of the decay product from the group's first token through token j; both equal the decayed
// sums of the group's chunk-local states.  Eight waves: wave (dir, nt) folds key-channel tile nt of one
// direction over all the group's keys (LIT: one state, written as both).  The states go to the
// workspace in the resident kernel's slot layout, with the group's log2 decay total.
template <int D, int KIND, int ROWS>
__global__ void __launch_bounds__(512) group_state_kernel(ChunkParams p) {
    using F = Fuse<D>;
    using T = __bf16;
    using RT = RowTile<D, T>;
    constexpr int NT = 512, NDT = F::NDT;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int ng = p.ng, bh = blockIdx.x / ng, gi = blockIdx.x % ng;
    const int L = min(ROWS, p.L - gi * ROWS);
    const int rows = cpad(L);
    const size_t base = (size_t)bh * p.L + (size_t)gi * ROWS;

    T *Ks = reinterpret_cast<T *>(smem);
    T *Vs = Ks + ROWS * D;
    float *E = reinterpret_cast<float *>(Vs + ROWS * D);
    double *sh = reinterpret_cast<double *>(E + ROWS);

    const float llt = KIND == kMaskS ? load_ll(p.ll + base, L, tid) : 0.f;
    stage_rows<D, T>(Vs, reinterpret_cast<const T *>(p.v) + base * D, 0, rows, L, wave, 8, lane);
    constexpr int KPER = (ROWS * RT::CPK + NT - 1) / NT;
    u32x4 kx[KPER];
    {
        const T *kg = reinterpret_cast<const T *>(p.k) + base * D;
#pragma unroll
        for (int u = 0; u < KPER; ++u) {
            const int c16 = min(tid + u * NT, rows * RT::CPK - 1);
            kx[u] = ld16(kg + (size_t)min(c16 / RT::CPK, L - 1) * D + (c16 % RT::CPK) * RT::VEC);
        }
    }
    float lgD = 0.f;
    if constexpr (KIND == kMaskD) lgD = p.ll[bh % p.H] * kLog2e;
    if constexpr (KIND == kMaskS) fused_exponents_s(E, sh, llt, L, ROWS, rows, tid);   // one "chunk": the group
    auto Ex = [&](int t) -> float {
        if constexpr (KIND == kMaskLit) return 0.f;
        else if constexpr (KIND == kMaskD) return (float)(t + 1) * lgD;
        else return E[t];
    };
    wait_vm_all();
#pragma unroll
    for (int u = 0; u < KPER; ++u) {
        const int c16 = tid + u * NT, row = c16 / RT::CPK;
        u32x4 o;
        if constexpr (KIND == kMaskD) {
            o = row < L ? kx[u] : u32x4{0u, 0u, 0u, 0u};
        } else {
            const bf16x8 x = __builtin_bit_cast(bf16x8, kx[u]);
            float f[8], ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                f[e] = phi_pre<KIND>((float)x[e]);
                ss += f[e] * f[e];
            }
            float scl = row < L ? 1.f : 0.f;
            if constexpr (KIND == kMaskS) scl *= inv_norm(group_sum<RT::CPK>(ss));
            bf16x8 y;
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = f2bf(f[e] * scl);
            o = __builtin_bit_cast(u32x4, y);
        }
        if (c16 < rows * RT::CPK) st16(Ks + RT::off(row, (c16 % RT::CPK) * RT::VEC), o);
    }

    // fold weights of every row, both directions, once per workgroup (forward relative to the group's
    // last token, backward to the token before its first); the sub-block loop reads them four at a time
    float *W = reinterpret_cast<float *>(sh + 16);   // [2][ROWS]
    if constexpr (KIND != kMaskLit) {
        const float etot = Ex(L - 1);
        for (int j = tid; j < rows; j += NT) {
            const float ej = Ex(j);
            W[j] = fast_exp2(fminf(etot - ej, 0.f));
            W[ROWS + j] = fast_exp2(fminf(ej, 0.f));
        }
    }
    __syncthreads();   // keys (phi applied) and the weight table in LDS

    const int nt = wave & 3, dir = wave >> 2;
    if (nt < NDT && (KIND != kMaskLit || dir == 0) && !(p.causal && dir == 1)) {
        f32x4 acc[NDT];
#pragma unroll
        for (int ct = 0; ct < NDT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        float zs = 0.f;   // row sums of key channel 16 nt + r over this lane's keys, fp32
        for (int h = 0; h < rows / kKB; ++h) {
            const bf16x8 kfr = tr_frag<D>(Ks, h, nt, r, g);
            bf16x8 af = kfr;
            if constexpr (KIND != kMaskLit) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const f32x4 w4 = *reinterpret_cast<const f32x4 *>(W + dir * ROWS + h * kKB + 16 * t + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float k = (float)kfr[4 * t + e];
                        af[4 * t + e] = f2bf(w4[e] * k);
                        zs = fmaf(w4[e], k, zs);
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) zs += (float)kfr[e];
            }
#pragma unroll
            for (int ct = 0; ct < NDT; ++ct) acc[ct] = mfma_bf16(af, tr_frag<D>(Vs, h, ct, r, g), acc[ct]);
        }
        zs += __shfl_xor(zs, 16, 64);
        zs += __shfl_xor(zs, 32, 64);
#pragma unroll
        for (int dd = 0; dd < 2; ++dd) {
            if ((KIND != kMaskLit && dd != dir) || (p.causal && dd == 1)) continue;
            T *dst = reinterpret_cast<T *>((dd == 0 ? p.fs : p.gs) + (size_t)blockIdx.x * F::SLOTK);
#pragma unroll
            for (int ct = 0; ct < NDT; ++ct) {
                bf16x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = f2bf(acc[ct][e]);
                *reinterpret_cast<bf16x4 *>(dst + F::wr(ct, nt, r, g)) = o;
            }
            // the row-sum tile: row 0 the bf16 high parts, row 1 the bf16 rounding of the remainders, of key
            // channels 16 nt + 4 g' + e held by fold lane (rr, g'): gather lane (r = 4 g' + e)'s sum
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float z = __shfl(zs, 4 * g + e, 64);
                const __bf16 zh = f2bf(z);
                o[e] = r == 0 ? zh : f2bf(z - (float)zh);
            }
            if (r < 2) *reinterpret_cast<bf16x4 *>(dst + F::VB / 2 + F::zwr(nt, r, g)) = o;
        }
    }
    if (tid == 0) p.tot[blockIdx.x] = Ex(L - 1);
}

template <int D, int ROWS>
__host__ __device__ constexpr size_t group_state_lds() {
    return 2 * (size_t)ROWS * D * 2 + (size_t)ROWS * 4 + 16 * 8 + 2 * (size_t)ROWS * 4;   // + fold-weight table
}

// ================================ group scan ==========================================================
// Carried group states of the resident path, in place: F_g <- 2^t_g F_{g-1} + F_g for g = 1 .. ng-2 and
// G_g <- 2^t_g G_{g+1} + G_g for g = ng-2 .. 1 (the last forward and first backward states are never
// read), accumulated in fp32 -- the row sums from their high plus low parts, re-split when stored.
// One wave per (batch, head, direction, 1 KiB piece of the value part), plus one for the 256 bytes of
// row sums.  The wave copies its piece of kScanSeg groups straight into LDS, waits once, then walks
// them in order: the sequential chain touches only LDS and never waits on a global load.
constexpr int kScanSeg = 32;
constexpr int kScanWave = 64;

template <int D>
__host__ __device__ constexpr int group_scan_waves() {
    return Fuse<D>::VB / 1024 + 1;
}

template <int D>
__global__ void __launch_bounds__(kScanWave) group_scan_kernel(ChunkParams p) {
    using F = Fuse<D>;
    constexpr int NWV = group_scan_waves<D>();
    extern __shared__ __align__(16) unsigned char buf[];   // kScanSeg KiB
    const int lane = threadIdx.x;
    const int ng = p.ng;
    const int pc = blockIdx.x % NWV, dir = (blockIdx.x / NWV) & 1, bh = blockIdx.x / (2 * NWV);
    if (p.causal && dir == 1) return;   // no barriers in this kernel
    const bool zu = pc == NWV - 1;
    // bytes this wave copies per group, and where they start in a state
    const int pbytes = zu ? F::NF * 128 : 1024;
    const int poff = zu ? F::VB : pc * 1024;
    unsigned char *base = (dir == 0 ? p.fs : p.gs) + (size_t)bh * ng * F::SLOTK + poff;
    const float *tg = p.tot + (size_t)bh * ng;
    const int steps = ng - 1;
    auto group_of = [&](int k) { return dir == 0 ? k : ng - 1 - k; };
    // this lane's unit: a value piece (lane), or row sums (lanes < 2 NF * 4 / 2): high piece hi, low piece hi + 4
    const bool active = zu ? lane < F::NF * 4 : true;
    const int o_hi = zu ? ((lane / 4) * 8 + lane % 4) * 16 : lane * 16;
    const int o_lo = zu ? o_hi + 64 : o_hi;

    float run[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < steps; s0 += kScanSeg) {
        const int ns = min(kScanSeg, steps - s0);
        for (int k = 0; k < ns; ++k)
            if (lane * 16 < pbytes) load_lds16(buf + k * 1024, base + (size_t)group_of(s0 + k) * F::SLOTK + lane * 16);
        // the segment's totals, lane k holding step k's (read back with readlane: no wait inside the chain)
        const float tgl = lane < ns ? tg[group_of(s0 + lane)] : 0.f;
        wait_vm_all();   // also drains the previous segment's stores
        for (int k = 0; k < ns; ++k) {
            const int gg = uniform(group_of(s0 + k));
            const float a = fast_exp2(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tgl), k)));
            const bf16x8 xh = *reinterpret_cast<const bf16x8 *>(buf + k * 1024 + o_hi);
            const bf16x8 xl = *reinterpret_cast<const bf16x8 *>(buf + k * 1024 + o_lo);
            bf16x8 oh, ol;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                run[e] = a * run[e] + (float)xh[e] + (zu ? (float)xl[e] : 0.f);
                oh[e] = f2bf(run[e]);
                ol[e] = f2bf(run[e] - (float)oh[e]);
            }
            unsigned char *dst = base + (size_t)gg * F::SLOTK;
            if (active) *reinterpret_cast<bf16x8 *>(dst + o_hi) = oh;
            if (zu && active) *reinterpret_cast<bf16x8 *>(dst + o_lo) = ol;
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

template <int D>
void launch_group_scan(const ChunkParams &p, unsigned bhs, hipStream_t stream) {
    hipLaunchKernelGGL((group_scan_kernel<D>), dim3(bhs * 2 * group_scan_waves<D>()), dim3(kScanWave),
                       kScanSeg * 1024, stream, p);
}

template <int D, bool BF16>
size_t workspace_t(const AttnArgs &a) {
    if constexpr (BF16 && D <= 64) {
        if (fused_ok(a.L, a.C, D, BF16)) {
            // resident path: one launch (states in LDS), or group states and totals
            const size_t ng = (size_t)fused_groups(a.L, a.C);
            if (ng < 2) return 0;
            const size_t nb = (size_t)a.B * a.H * ng;
            return 2 * nb * Fuse<D>::SLOTK + ((nb * 4 + 15) & ~(size_t)15);
        }
    }
    const size_t n = (size_t)((a.L + a.C - 1) / a.C);
    if (n < 2) return 0;   // one chunk
    const size_t nb = (size_t)a.B * a.H * n;
    return 2 * nb * ChunkCfg<D, BF16>::SLOT + ((nb * 4 + 15) & ~(size_t)15);
}

template <int D, int KIND, bool BF16, bool INB = BF16>
hipError_t launch_t(const AttnArgs &a, hipStream_t stream) {
    using Cf = ChunkCfg<D, BF16>;
    ChunkParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.ll = a.log_lambda;
    p.eps = a.eps;
    p.H = a.H;
    p.L = a.L;
    p.C = a.C;
    p.n = (a.L + a.C - 1) / a.C;
    p.y = a.y;
    p.out_bf16 = a.out_bf16 ? 1 : 0;
    p.den_out = a.den_out;
    const size_t nb = (size_t)a.B * a.H * p.n;
    p.fs = p.gs = nullptr;
    p.tot = nullptr;
    p.ng = 1;
    p.causal = a.causal ? 1 : 0;
    if constexpr (BF16 && D <= 64) {
        if (fused_ok(a.L, a.C, D, BF16)) {
            const int rows = fused_rows(a.L, a.C);
            p.ng = fused_groups(a.L, a.C);
            const unsigned grid = (unsigned)(a.B * a.H * p.ng);
            if (p.ng > 1) {
                const size_t ngt = (size_t)a.B * a.H * p.ng;
                p.fs = reinterpret_cast<unsigned char *>(a.workspace);
                p.gs = p.fs + ngt * Fuse<D>::SLOTK;
                p.tot = reinterpret_cast<float *>(p.gs + ngt * Fuse<D>::SLOTK);
            }
            auto run = [&](auto rows_c) {
                constexpr int ROWS = decltype(rows_c)::value;
                if constexpr (ROWS == kGroupRows) {   // groups: states, scan, then outputs
                    constexpr size_t lds1 = group_state_lds<D, ROWS>();
                    allow_lds(&group_state_kernel<D, KIND, ROWS>, lds1);
                    hipLaunchKernelGGL((group_state_kernel<D, KIND, ROWS>), dim3(grid), dim3(512), lds1, stream, p);
                    if (p.ng > 2) launch_group_scan<D>(p, (unsigned)(a.B * a.H), stream);
                }
                const size_t lds = fused_lds<D, KIND, ROWS>(p.ng > 1);
                allow_lds(&chunk_fused_kernel<D, KIND, ROWS>, lds);
                hipLaunchKernelGGL((chunk_fused_kernel<D, KIND, ROWS>), dim3(grid), dim3(ROWS / 16 * 64), lds, stream, p);
            };
            if (rows == kGroupRows) run(std::integral_constant<int, kGroupRows>{});
            else run(std::integral_constant<int, kFuseRows>{});
            return hipGetLastError();
        }
    }
    if (p.n > 1) {
        p.fs = reinterpret_cast<unsigned char *>(a.workspace);
        p.gs = p.fs + nb * Cf::SLOT;
        p.tot = reinterpret_cast<float *>(p.gs + nb * Cf::SLOT);
        constexpr int NW1 = state_waves(D);
        const size_t lds1 = chunk_lds<D, BF16>(a.C, NW1, false);
        allow_lds(&chunk_state_kernel<D, KIND, BF16, INB>, lds1);
        hipLaunchKernelGGL((chunk_state_kernel<D, KIND, BF16, INB>), dim3((unsigned)nb), dim3(NW1 * 64), lds1, stream,
                           p);
        constexpr int NBLK = (scan_vectors<D, BF16>() + kScanThreads - 1) / kScanThreads;
        hipLaunchKernelGGL((chunk_scan_kernel<D, BF16>), dim3((unsigned)(a.B * a.H * 2 * NBLK)), dim3(kScanThreads), 0,
                           stream, p);
    }
    // output workgroups: the chunk's C/16 query tiles over 4 waves (C <= 64: one tile each; C = 128: two
    // tiles each, which share every key and value fragment read -- 53 against 55 us on B8 H12 L4097 for
    // 8 waves of one tile) or 8 waves (C >= 256, or d = 128)
    auto out = [&](auto kernel, int nw) {
        const size_t lds = chunk_lds<D, BF16>(a.C, nw, true);
        allow_lds(kernel, lds);
        hipLaunchKernelGGL(kernel, dim3((unsigned)nb), dim3(nw * 64), lds, stream, p);
    };
    if (a.C <= 64) out(&chunk_out_kernel<D, KIND, 4, 1, BF16, INB>, 4);
    else if (D == 128) out(&chunk_out_kernel<D, KIND, 8, 1, BF16, INB>, 8);
    else if (a.C <= 128) out(&chunk_out_kernel<D, KIND, 4, 2, BF16, INB>, 4);
    else out(&chunk_out_kernel<D, KIND, 8, (D == 128 ? 1 : 2), BF16, INB>, 8);
    return hipGetLastError();
}

template <int D, bool BF16, bool INB>
hipError_t dispatch_kind(const AttnArgs &a, hipStream_t stream) {
    switch (a.kind) {
    case kMaskLit: return launch_t<D, kMaskLit, BF16, INB>(a, stream);
    case kMaskD: return launch_t<D, kMaskD, BF16, INB>(a, stream);
    default: return launch_t<D, kMaskS, BF16, INB>(a, stream);
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

template <int D, bool BF16>
Plan plan_t(const AttnArgs &a) {
    Plan p;
    p.ok = chunk_lds<D, BF16>(a.C, 8, true) <= kLdsPerWorkgroup;
    p.workspace = workspace_t<D, BF16>(a);
    return p;
}

}  // namespace

Plan plan_chunk(const AttnArgs &a) {
    const bool bf16c = !a.fp32c;   // the arithmetic sets the tiles and states
    switch (a.d) {
    case 16: return bf16c ? plan_t<16, true>(a) : plan_t<16, false>(a);
    case 32: return bf16c ? plan_t<32, true>(a) : plan_t<32, false>(a);
    case 64: return bf16c ? plan_t<64, true>(a) : plan_t<64, false>(a);
    default: return bf16c ? plan_t<128, true>(a) : plan_t<128, false>(a);
    }
}

hipError_t launch_chunk(const AttnArgs &a, hipStream_t stream) {
    if (!a.fp32c) return dispatch_d<true, true>(a, stream);
    return a.in_bf16 ? dispatch_d<false, true>(a, stream) : dispatch_d<false, false>(a, stream);
}

}  // namespace lion
