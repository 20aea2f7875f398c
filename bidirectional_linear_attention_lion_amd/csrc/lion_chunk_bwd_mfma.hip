// lion_chunk_bwd_mfma.hip -- backward pass of the chunkwise form for chunks of 64 and 128 tokens, every
// product on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16); and the full form's backward for a
// sequence of at most 256 tokens (d <= 64), which is one chunk of up to 256 (no walk, no states).
//
// The gradients and their chunkwise split are those of lion_chunk_bwd.hip (the chain rule of the
// attention form, OpenReview abstract and reply "Concern 1", Theorem 3.3 Eq. 25, organised like the
// chunkwise form, reply "4: Practicality of Recurrent Inference"; blog "LION Part IV - Results", "LION
// Chunk"): pairs inside a chunk formed directly, the rest of the sequence through the four states
// entering each chunk,
//   keys'    F = sum_j w_j phi(k_j) [v_j, 1]^T,   queries'  G = sum_i w_i phi(q_i) [dy_i / den_i, -delta_i]^T,
// from the left and from the right.  Operands are rounded to bf16 as in the full form's backward
// (phi(q), phi(k), the masked dS and P / den), and so are the states' d x d blocks; sums are fp32.
//
//   walk: a workgroup per (batch, head, direction, keys or queries) walks the chunks in order.  Its
//         running state is fp32 in matrix-core accumulators; each chunk's tokens are staged as bf16
//         with their weight folded in (X' = w_j phi(k_j), or w_i phi(q_i) / den_i), so the update is
//         S^T <- e^{tot} S^T + Y^T X' with Y = v or dy (the last column, 1 or -dy.y, enters as a 17th
//         row tile holding it as a bf16 hi/lo pair).  The state entering each chunk is written as bf16
//         d x d rows plus its last column in fp32.
//   main: a workgroup of 2 C / 16 waves per chunk: C / 16 query-side waves (one 16-row query tile each)
//         and C / 16 key-side waves.  The pair part is the full form's backward restricted to the chunk:
//         S^T and dP^T against the chunk's keys, then dphi(Q)^T += phi(K)^T dS^T on the query side; S and
//         dP against its queries, then dV^T += dY^T (P / den) and dphi(K)^T += phi(Q)^T dS on the key
//         side.  The entering states, staged into the space of the value and dy tiles, then add (f the
//         weight from the chunk's near end to the token)
//           dphi(q_i) += f_i (F dy_i / den_i - F_d delta_i),   dphi(k_j) += f_j (G v_j + G_d),
//           dv_j += f_j G^T phi(k_j)
//         and the dA halves phi(q_i).(that) and phi(k_j).(that), plus from the left, minus from the right.
// Causal variant: pairs above the diagonal drop out, and so do the keys' state from the right and the
// queries' state from the left.
#include "lion_device.h"
#include "lion_internal.h"
#include "lion_stage.h"
#include "lion_bwd_tiles.h"

namespace lion {
namespace {

constexpr int kWalkThreads = 256;

struct MbParams {
    const __bf16 *q, *k, *v, *y, *dy;
    const float *den, *ll;
    int H, L, nch, causal, nbh;   // nbh: B H
    void *dq, *dk, *dv;
    int g_bf16;
    __bf16 *st;                // [B H][nch][4][D][D]: key-left, query-left, key-right, query-right
    float *stz;                // [B H][nch][4][D]: the states' last column
    float *da_row, *da_col;    // [B H L]
    float *dll_part;           // LION-D lone chunk: [B H][2 halves][hi, lo] of sum_t t dA_t, or null
};

// Inclusive prefix sums of the chunk's log decays in log2 units relative to the chunk start (cum[t],
// repeating the last one past n) and the chunk's total (cum[CT]); run by one whole wave.  LION-S reads
// the decays from ll_row (n of them), LION-D forms them from the head's log(lambda).
template <int KIND, int CT>
__device__ __forceinline__ void chunk_cum(float *cum, const float *ll, const float *ll_row, int h, int n, int lane) {
    if constexpr (KIND == kMaskD) {
        const float lg = ll[h] * kLog2e;
        for (int t = lane; t < CT; t += 64) cum[t] = (float)(min(t, n - 1) + 1) * lg;
        if (lane == 0) cum[CT] = (float)n * lg;
    } else if constexpr (KIND == kMaskS) {
        constexpr int R = CT / 64;   // consecutive tokens per lane
        double x[R], s = 0.0;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int t = lane * R + k;
            s += t < n ? (double)ll_row[t] : 0.0;
            x[k] = s;
        }
        double incl = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double up = __shfl_up(incl, o, 64);
            if (lane >= o) incl += up;
        }
        const double excl = incl - s;
#pragma unroll
        for (int k = 0; k < R; ++k) cum[lane * R + k] = (float)((excl + x[k]) * 1.4426950408889634);
        const double tot = __shfl(incl, 63, 64);
        if (lane == 0) cum[CT] = (float)(tot * 1.4426950408889634);
    } else {
        for (int t = lane; t <= CT; t += 64) cum[t] = 0.f;
    }
}

// x's bits where ok, else zero (a select on whole 32-bit words: a select on bf16 elements compiles to
// branches)
__device__ __forceinline__ u32x4 keep_if(bf16x8 x, bool ok) {
    const u32x4 b = __builtin_bit_cast(u32x4, x);
    const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
    return b & m;
}

// ================================ walk ===============================================================
template <int D, int CT, bool KEYS>
struct WalkRegs {
    static constexpr int SPR = D / 8;                     // 16-byte slots per row
    static constexpr int NIT = CT * SPR / kWalkThreads;   // slots per thread
    bf16x8 x[NIT], y[NIT], z[KEYS ? 1 : NIT];             // keys: k, v; queries: q, dy, y
    float den[KEYS ? 1 : NIT];
    float ll[CT / 64];                                    // LION-S: tokens R lane + k of the chunk
};

// Rows past n load row n - 1 (walk_commit zeroes them): no branch around the loads, so the compiler can
// count the loads in flight and wait for one chunk's without waiting for the next one's.
template <int D, int KIND, int CT, bool KEYS>
__device__ __forceinline__ void walk_load(const MbParams &p, int bh, int c, int n, WalkRegs<D, CT, KEYS> &R) {
    using WR = WalkRegs<D, CT, KEYS>;
    const int tid = threadIdx.x;
    const size_t row0 = (size_t)bh * p.L + (size_t)c * CT;
#pragma unroll
    for (int it = 0; it < WR::NIT; ++it) {
        const int sl = it * kWalkThreads + tid;
        const int row = min(sl / WR::SPR, n - 1), cs = (sl % WR::SPR) * 8;
        const size_t g = (row0 + row) * D + cs;
        if constexpr (KEYS) {
            R.x[it] = __builtin_bit_cast(bf16x8, ld16(p.k + g));
            R.y[it] = __builtin_bit_cast(bf16x8, ld16(p.v + g));
        } else {
            R.x[it] = __builtin_bit_cast(bf16x8, ld16(p.q + g));
            R.y[it] = __builtin_bit_cast(bf16x8, ld16(p.dy + g));
            R.z[it] = __builtin_bit_cast(bf16x8, ld16(p.y + g));
            R.den[it] = p.den[row0 + row];
        }
    }
    if constexpr (KIND == kMaskS) {
        constexpr int RL = CT / 64;
#pragma unroll
        for (int k = 0; k < RL; ++k) R.ll[k] = p.ll[row0 + min((tid & 63) * RL + k, n - 1)];
    }
}

// LION-S: the chunk's inclusive prefix sums of log(lambda) in log2 units (cum[t], repeating the last one
// past n) and its total (cum[CT]) from the decays walk_load left in registers; run by one whole wave.
template <int D, int CT, bool KEYS>
__device__ __forceinline__ void walk_scan(float *cum, const WalkRegs<D, CT, KEYS> &R, int n, int lane) {
    constexpr int RL = CT / 64;
    double x[RL], s = 0.0;
#pragma unroll
    for (int k = 0; k < RL; ++k) {
        s += lane * RL + k < n ? (double)R.ll[k] : 0.0;
        x[k] = s;
    }
    double incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double up = __shfl_up(incl, o, 64);
        if (lane >= o) incl += up;
    }
    const double excl = incl - s;
#pragma unroll
    for (int k = 0; k < RL; ++k) cum[lane * RL + k] = (float)((excl + x[k]) * 1.4426950408889634);
    const double tot = __shfl(incl, 63, 64);
    if (lane == 0) cum[CT] = (float)(tot * 1.4426950408889634);
}

// Prefix sum at row t of a chunk of n rows (log2 units): LION-D in closed form from lg = log2(lambda_h),
// LION-S from the scanned table.
template <int KIND, int CT>
__device__ __forceinline__ float walk_cum(const float *cum, float lg, int t, int n) {
    if constexpr (KIND == kMaskD) return (float)(min(t, n - 1) + 1) * lg;
    else if constexpr (KIND == kMaskS) return cum[min(t, CT)];
    else return 0.f;
}

// The chunk's rows into one buffer of LDS tiles: Xt = w phi(x) (/ den for queries), Yt = v or dy (rows
// at or past n zero), cz = the last column's entries (queries: -dy.y; keys: unused).  No barrier inside.
template <int D, int KIND, int CT, bool KEYS>
__device__ __forceinline__ void walk_commit(__bf16 *Xt, __bf16 *Yt, const float *cum, float *cz, int n, int dir,
                                            float lg, const WalkRegs<D, CT, KEYS> &R) {
    using WR = WalkRegs<D, CT, KEYS>;
    using RT = RowTile<D, __bf16>;
    constexpr int SPR = WR::SPR;
    const int tid = threadIdx.x;
    const float tot = KIND == kMaskD ? (float)n * lg : walk_cum<KIND, CT>(cum, lg, CT, n + 1);
#pragma unroll
    for (int it = 0; it < WR::NIT; ++it) {
        const int sl = it * kWalkThreads + tid;
        const int row = sl / SPR, cs = (sl % SPR) * 8;
        const bool ok = row < n;
        // rows past n hold row n - 1's values (finite): computed alike, zeroed through the scale
        float fx[8], ss = 0.f, part = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            fx[e] = phi_pre<KIND>((float)R.x[it][e]);
            ss += fx[e] * fx[e];
            if constexpr (!KEYS) part += (float)R.y[it][e] * (float)R.z[it][e];
        }
        float scl = ok ? 1.f : 0.f;
        if constexpr (KIND == kMaskS) scl *= inv_norm(group_sum<SPR>(ss));
        if constexpr (KIND != kMaskLit) {
            const float cr = walk_cum<KIND, CT>(cum, lg, row, n);
            scl *= fast_exp2(dir == 0 ? tot - cr : cr);
        }
        if constexpr (!KEYS) {
            part = group_sum<SPR>(part);
            scl *= __builtin_amdgcn_rcpf(R.den[it]);
            if (sl % SPR == 0) cz[row] = ok ? -part : 0.f;
        }
        bf16x8 xo;
#pragma unroll
        for (int e = 0; e < 8; ++e) xo[e] = f2bf(fx[e] * scl);
        *reinterpret_cast<bf16x8 *>(Xt + RT::off(row, cs)) = xo;
        *reinterpret_cast<u32x4 *>(Yt + RT::off(row, cs)) = keep_if(R.y[it], ok);
    }
}

// State tiles: 16 x 16 tiles (tb, ta) of S^T, tb < NA + 1 (the last one holds the last column in its
// first two rows), ta < NA; wave w takes tiles w, w + 4, ... with ta = tile % NA, tb = tile / NA, which for
// NA a multiple of 4 is ta = w + 4 (u % (NA / 4)), tb = u / (NA / 4): tb then is known at compile time.
template <int NA>
__device__ __forceinline__ void walk_tile(int w, int u, int &ta, int &tb) {
    if constexpr (NA % 4 == 0) {
        ta = w + 4 * (u % (NA / 4));
        tb = u / (NA / 4);
    } else {
        ta = (w + 4 * u) % NA;
        tb = (w + 4 * u) / NA;
    }
}

template <int D, int CT>
struct WalkLds {
    static constexpr int TILE = CT * D;                              // bf16 elements per tile
    static constexpr int CUM = CT + 4, CZ = CT;                      // floats per buffer
    static constexpr size_t BYTES = (size_t)4 * TILE * 2 + (size_t)2 * (CUM + CZ) * 4;
};

// The staged tiles, prefix sums and last-column entries are double-buffered: chunk s is summed from
// buffer s & 1 while chunk s + 1 is staged into the other, so a step needs one barrier (two for LION-S,
// whose prefix sums are scanned by one wave first).
template <int D, int KIND, int CT, bool KEYS>
__device__ void walk(const MbParams &p, unsigned char *smem, int bh, int dir) {
    using WL = WalkLds<D, CT>;
    constexpr int NA = D / 16, NT = NA * (NA + 1), NU = (NT + 3) / 4;
    __bf16 *Xt0 = reinterpret_cast<__bf16 *>(smem);
    float *cum0 = reinterpret_cast<float *>(Xt0 + 4 * WL::TILE);
    auto Xt = [&](int b) { return Xt0 + 2 * b * WL::TILE; };
    auto Yt = [&](int b) { return Xt0 + (2 * b + 1) * WL::TILE; };
    auto cum = [&](int b) { return cum0 + b * (WL::CUM + WL::CZ); };
    auto cz = [&](int b) { return cum0 + b * (WL::CUM + WL::CZ) + WL::CUM; };
    const int tid = threadIdx.x, w = uniform(tid >> 6), lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int st = 2 * dir + (KEYS ? 0 : 1);
    const float lg = KIND == kMaskD ? p.ll[bh % p.H] * kLog2e : 0.f;
    f32x4 acc[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Two chunks of loads in flight: the rows of the chunk after next are issued while this chunk is
    // summed, into the register set the next chunk's rows have just left (the loop takes two steps per
    // iteration so each set, and each buffer, stays fixed).
    WalkRegs<D, CT, KEYS> RA, RB;
    auto chunk_of = [&](int step) { return dir == 0 ? step : p.nch - 1 - step; };
    auto rows_of = [&](int step) { return min(CT, p.L - chunk_of(step) * CT); };
    walk_load<D, KIND, CT, KEYS>(p, bh, chunk_of(0), rows_of(0), RA);
    if constexpr (KIND == kMaskS) {
        if (w == 0) walk_scan<D, CT, KEYS>(cum(0), RA, rows_of(0), lane);
        __syncthreads();
    }
    walk_commit<D, KIND, CT, KEYS>(Xt(0), Yt(0), cum(0), cz(0), rows_of(0), dir, lg, RA);
    __syncthreads();
    walk_load<D, KIND, CT, KEYS>(p, bh, chunk_of(min(1, p.nch - 1)), rows_of(min(1, p.nch - 1)), RA);
    // one chunk, summed from buffer b: R1 holds (or is receiving) the next chunk's rows, R2 takes the
    // chunk after next
    auto one_step = [&](int step, int b, WalkRegs<D, CT, KEYS> &R1, WalkRegs<D, CT, KEYS> &R2) {
        const int c = chunk_of(step), n = rows_of(step);
        {   // unconditionally (past the end: the last chunk again, unused), for the same reason as above
            const int s2 = min(step + 2, p.nch - 1);
            walk_load<D, KIND, CT, KEYS>(p, bh, chunk_of(s2), rows_of(s2), R2);
        }
        // the state entering chunk c is the running sum so far
        const size_t so = ((size_t)bh * p.nch + c) * 4 + st;
        __bf16 *sd = p.st + so * D * D;
        float *zd = p.stz + so * D;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int tile = w + 4 * u;
            if (NT % 4 != 0 && tile >= NT) break;
            int ta, tb;
            walk_tile<NA>(w, u, ta, tb);
            const int a = 16 * ta + r;
            if (tb < NA) {
                bf16x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = f2bf(acc[u][e]);
                *reinterpret_cast<bf16x4 *>(sd + a * D + 16 * tb + 4 * g) = o;
            } else {
                // hi + lo in lane r of group 0; the row's four lanes store the same value
                zd[a] = __shfl(acc[u][0] + acc[u][1], r, 64);
            }
        }
        // decay across the chunk, then add its tokens: S^T[b][a] += sum_j Y_j[b] X'_j[a]
        const float dec = KIND == kMaskD ? fast_exp2((float)n * lg)
                                         : KIND == kMaskS ? fast_exp2(cum(b)[CT]) : 1.f;
#pragma unroll
        for (int u = 0; u < NU; ++u) acc[u] *= dec;
        const __bf16 *xb = Xt(b), *yb = Yt(b);
        const float *czb = cz(b);
#pragma unroll
        for (int h = 0; h < CT / kKB; ++h) {
            // the last column's tile: row 0 the hi part, row 1 the lo part (keys: 1), at the tokens of
            // the transposed fragments' slots (4 g + e and 16 + 4 g + e of the sub-block)
            bf16x8 zf;
            if constexpr (KEYS) {
#pragma unroll
                for (int e = 0; e < 8; ++e) zf[e] = f2bf(r == 0 ? 1.f : 0.f);
            } else {
                const f32x4 c0 = *reinterpret_cast<const f32x4 *>(czb + h * kKB + 4 * g);
                const f32x4 c1 = *reinterpret_cast<const f32x4 *>(czb + h * kKB + 16 + 4 * g);
                // selected in fp32: lane r = 0 rounds c (the hi part), r = 1 the rest (the lo part)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float r0 = c0[e] - (float)f2bf(c0[e]), r1 = c1[e] - (float)f2bf(c1[e]);
                    zf[e] = f2bf(r == 0 ? c0[e] : (r == 1 ? r0 : 0.f));
                    zf[4 + e] = f2bf(r == 0 ? c1[e] : (r == 1 ? r1 : 0.f));
                }
            }
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int tile = w + 4 * u;
                if (NT % 4 != 0 && tile >= NT) break;
                int ta, tb;
                walk_tile<NA>(w, u, ta, tb);
                const bf16x8 af = tb < NA ? tr_frag<D>(yb, h, tb, r, g) : zf;
                acc[u] = mfma_bf16(af, tr_frag<D>(xb, h, ta, r, g), acc[u]);
            }
        }
        // stage the next chunk into the other buffer (its last readers finished before the previous
        // step's barrier)
        if (step + 1 < p.nch) {
            const int nb = b ^ 1, n1 = rows_of(step + 1);
            if constexpr (KIND == kMaskS) {
                if (w == 0) walk_scan<D, CT, KEYS>(cum(nb), R1, n1, lane);
                __syncthreads();
            }
            walk_commit<D, KIND, CT, KEYS>(Xt(nb), Yt(nb), cum(nb), cz(nb), n1, dir, lg, R1);
        }
        __syncthreads();   // the next chunk's buffer is written; this one's readers are done
    };
#pragma unroll 1
    for (int step = 0; step < p.nch; step += 2) {
        one_step(step, 0, RA, RB);
        if (step + 1 < p.nch) one_step(step + 1, 1, RB, RA);
    }
}

template <int D, int KIND, int CT>
__global__ void __launch_bounds__(kWalkThreads) mb_walk_kernel(MbParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int ns = p.causal ? 2 : 4;
    const int bh = blockIdx.x / ns, s = blockIdx.x % ns;
    // causal: s = 0 keys from the left, s = 1 queries from the right; else s = 2 dir + (queries)
    const int dir = p.causal ? s : s >> 1;
    const bool keys = p.causal ? s == 0 : (s & 1) == 0;
    if (keys) walk<D, KIND, CT, true>(p, smem, bh, dir);
    else walk<D, KIND, CT, false>(p, smem, bh, dir);
}

// ================================ main ===============================================================
// Four bf16 values of row `row`, channels c .. c + 3 (c a multiple of 4), of a staged tile.
template <int D>
__device__ __forceinline__ bf16x4 row4(const __bf16 *tile, int row, int c) {
    return *reinterpret_cast<const bf16x4 *>(tile + RowTile<D, __bf16>::off(row, c));
}

// Tiles per wave (two at C = 256, which would otherwise need 32 waves) and threads per workgroup.
constexpr int main_tpw(int ct) { return ct > 128 ? 2 : 1; }
constexpr int main_threads(int ct) { return ct * 8 / main_tpw(ct); }

template <int D, int CT, bool SPLIT = false>
struct MainLds {
    static constexpr int TILE = CT * D;                        // bf16 elements per token tile
    static constexpr size_t TOK = (size_t)(SPLIT ? 2 : 4) * TILE * 2;   // phi(q), phi(k), v, dy (one side's two)
    static constexpr size_t F32 = (size_t)(CT + 4) + 2 * CT + 4 * D;   // cum, 1/den, delta, last columns
    static constexpr size_t BYTES = TOK + F32 * 4;
    static constexpr int NSF = 2 * CT / D < 4 ? 2 * CT / D : 4;  // states staged at once (value + dy tiles' space)
};

// The workgroup has 2 C / 16 waves (C / 16 at C = 256, each wave taking two tiles, one from each end, in
// turn): the first half take the query side of their query tiles (dphi(q) and the row half of dA), the
// second half the key side of their key tiles (dphi(k), dv and the column half).  Each side keeps only
// its own accumulators, and the two run as separate code paths (with the same barriers), so a wave's
// registers hold one side's work.
// SPLIT (a lone chunk, no states): the two sides go to two workgroups of C / 16 waves, blocks b and b + 8
// of each 16 (one XCD, so the second read of the rows hits its L2); each stages only the two tiles its
// side reads across (keys and values for the query side, queries and dy for the key side) and loads the
// fragments of its own rows from memory, so two such workgroups share a compute unit.
template <int D, int KIND, int CT, bool SPLIT = false>
__global__ void __launch_bounds__(SPLIT ? main_threads(CT) / 2 : main_threads(CT))
    __attribute__((amdgpu_waves_per_eu(SPLIT ? 4 : 1))) mb_main_kernel(MbParams p) {
    using RT = RowTile<D, __bf16>;
    using ML = MainLds<D, CT, SPLIT>;
    constexpr int NS = D / 32, NCT = D / 16, SPR = D / 8, NW = CT / 16, TPW = main_tpw(CT), NQW = NW / TPW;
    constexpr int NWG = SPLIT ? NQW : 2 * NQW, NT = 64 * NWG;
    extern __shared__ __align__(16) unsigned char smem[];
    // (split: the query side's phi(k), v tiles and the key side's phi(q), dy tiles share the space)
    __bf16 *Qt = reinterpret_cast<__bf16 *>(smem);
    __bf16 *Kt = SPLIT ? Qt : Qt + ML::TILE, *Vt = Kt + ML::TILE, *Gt = SPLIT ? Vt : Vt + ML::TILE;
    float *cum = reinterpret_cast<float *>(Gt + ML::TILE);
    float *inv = cum + CT + 4, *dl = inv + CT, *zst = dl + CT;

    const int bid = blockIdx.x;
    const int bh = SPLIT ? (bid >> 4) * 8 + (bid & 7) : bid / p.nch, c = SPLIT ? 0 : bid % p.nch;
    if (SPLIT && bh >= p.nbh) return;   // the grid is rounded up to whole groups of 16 (workgroup-uniform)
    const int n = min(CT, p.L - c * CT);
    const int tid = threadIdx.x, w = uniform(tid >> 6), lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int wq = w % NQW;          // this wave's tiles: wq and, with two per wave, NW - 1 - wq
    const bool qside = SPLIT ? ((bid >> 3) & 1) == 0 : w < NQW;   // wave-uniform
    const size_t row0 = (size_t)bh * p.L + (size_t)c * CT;
    const bool causal = p.causal != 0;

    // the entering states this chunk needs (none left of the first chunk or right of the last; causal,
    // not the keys' state from the right nor the queries' from the left)
    // (a list of 4-bit state indices rather than an array, which a dynamic index would put in scratch)
    unsigned sts = 0;
    int nst = 0;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const bool right = st >= 2, keys = (st & 1) == 0;
        if (!((right ? c == p.nch - 1 : c == 0) || (causal && keys == right))) sts |= (unsigned)st << (4 * nst++);
    }
    auto st_at = [&](int k) { return (int)((sts >> (4 * k)) & 15u); };

    // ---- stage the chunk: phi(q), phi(k), v, dy as bf16 rows (zero past n); 1/den and delta per row
    {
        constexpr int NSL = CT * SPR, NIT = (NSL + NT - 1) / NT;
        bf16x8 rq[NIT], rk[NIT], rv[NIT], rg[NIT], ry[NIT];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int sl = min(it * NT + tid, NSL - 1);
            const int row = sl / SPR, cs = (sl % SPR) * 8;
            const size_t gi = (row0 + min(row, n - 1)) * D + cs;
            if (!SPLIT || !qside) rq[it] = __builtin_bit_cast(bf16x8, ld16(p.q + gi));
            if (!SPLIT || qside) {
                rk[it] = __builtin_bit_cast(bf16x8, ld16(p.k + gi));
                rv[it] = __builtin_bit_cast(bf16x8, ld16(p.v + gi));
            }
            rg[it] = __builtin_bit_cast(bf16x8, ld16(p.dy + gi));
            ry[it] = __builtin_bit_cast(bf16x8, ld16(p.y + gi));
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int sl = it * NT + tid;   // slots past NSL (d = 32) repeat the last one and store nothing
            const int row = min(sl, NSL - 1) / SPR, cs = (sl % SPR) * 8;
            const bool ok = row < n;
            float fq[8], fk[8], ssq = 0.f, ssk = 0.f, part = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                fq[e] = !SPLIT || !qside ? phi_pre<KIND>((float)rq[it][e]) : 0.f;
                fk[e] = !SPLIT || qside ? phi_pre<KIND>((float)rk[it][e]) : 0.f;
                ssq += fq[e] * fq[e];
                ssk += fk[e] * fk[e];
                part += (float)rg[it][e] * (float)ry[it][e];
            }
            float sq = ok ? 1.f : 0.f, sk = sq;
            if constexpr (KIND == kMaskS) {
                sq *= inv_norm(group_sum<SPR>(ssq));
                sk *= inv_norm(group_sum<SPR>(ssk));
            }
            part = group_sum<SPR>(part);
            bf16x8 oq, ok8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                oq[e] = f2bf(fq[e] * sq);
                ok8[e] = f2bf(fk[e] * sk);
            }
            if (NSL % NT == 0 || sl < NSL) {
                const int at = RT::off(row, cs);
                if (!SPLIT || !qside) {
                    *reinterpret_cast<bf16x8 *>(Qt + at) = oq;
                    *reinterpret_cast<u32x4 *>(Gt + at) = keep_if(rg[it], ok);
                }
                if (!SPLIT || qside) {
                    *reinterpret_cast<bf16x8 *>(Kt + at) = ok8;
                    *reinterpret_cast<u32x4 *>(Vt + at) = keep_if(rv[it], ok);
                }
                if (sl % SPR == 0) {
                    const float iv = ok ? 1.f / p.den[row0 + row] : 0.f;
                    inv[row] = iv;
                    dl[row] = part * iv;
                }
            }
        }
    }
    if (w == 0) chunk_cum<KIND, CT>(cum, p.ll, KIND == kMaskS ? p.ll + row0 : nullptr, bh % p.H, n, lane);
    for (int t = tid; t < nst * D; t += NT) {
        const int st = st_at(t / D);
        zst[st * D + t % D] = p.stz[(((size_t)bh * p.nch + c) * 4 + st) * D + t % D];
    }
    __syncthreads();
    const float tot = cum[CT];

    // The entering states, staged NSF at a time into the value and dy tiles' space as bf16 d x d row
    // tiles; apply(S, z, st) runs for each (both sides pass through the same barriers).
    auto rounds = [&](auto &&apply) {
        if (SPLIT || nst == 0) return;   // a lone chunk (workgroup-uniform)
        __syncthreads();   // every wave is done with the value and dy tiles
        __bf16 *Sb = Vt;
#pragma unroll 1
        for (int k0 = 0; k0 < nst; k0 += ML::NSF) {
            const int kn = min(ML::NSF, nst - k0);
            for (int k = 0; k < kn; ++k)
                stage_rows<D, __bf16>(Sb + k * D * D, p.st + (((size_t)bh * p.nch + c) * 4 + st_at(k0 + k)) * D * D, 0,
                                      D, D, w, NWG, lane);
            wait_vm_all();
            __syncthreads();
#pragma unroll 1
            for (int k = 0; k < kn; ++k) {
                const int st = st_at(k0 + k);
                apply(Sb + k * D * D, zst + st * D, st);
            }
            __syncthreads();   // before the next states overwrite these
        }
    };
    const bool gb = p.g_bf16 != 0;
    // LION-D with dll_part: this lane's share of sum_t t dA_t (a lone chunk, so t is the tile row)
    const bool fuse_dll = KIND == kMaskD && p.dll_part != nullptr;   // workgroup-uniform
    double tsum = 0.0;

    if (qside) {
#pragma unroll 1
        for (int kt = 0; kt < TPW; ++kt) {
            const int tw = kt == 0 ? wq : NW - 1 - wq;   // tiles paired from both ends: the causal pair counts balance
            const int i_me = 16 * tw + r;   // this lane's row of the tile
            const float cum_me = cum[i_me];
            const size_t rowg = row0 + i_me;
            const bool live = 16 * tw < n;   // wave-uniform; a tile wholly past the chunk's end computes nothing
            // ---- query side: dphi(Q)^T (channel 16 ct + 4 g + e, query i_me) against the chunk's keys
            bf16x8 qf[NS], df[NS];
            if constexpr (SPLIT) {
                const size_t rc = row0 + min(i_me, n - 1);
                row_frags<D, KIND, true>(p.q + rc * D, i_me < n, qf);
                row_frags<D, KIND, false>(p.dy + rc * D, i_me < n, df);
            } else {
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    qf[st] = rows_frag<D>(Qt, tw >> 1, tw & 1, st, r, g);
                    df[st] = rows_frag<D>(Gt, tw >> 1, tw & 1, st, r, g);
                }
            }
            const float inv_me = inv[i_me], dl_me = dl[i_me];
            f32x4 aq[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) aq[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            float rowterm = 0.f;
            // Separable mask for key sub-blocks wholly before or after the tile's rows (first row r0, last
            // rl; the prefix sums decrease along the chunk): M_ij = exp2(c_i - c_r0) exp2(c_r0 - c_j) for keys
            // before, exp2(c_rl - c_i) exp2(c_j - c_rl) for keys after, every factor at most 1; the key's factor
            // comes by DPP row broadcast.  The sub-block the tile sits in keeps one exponential per score.
            const float e_first = uniform(cum[16 * tw]), e_last = uniform(cum[16 * tw + 15]);
            const float rowf_b = KIND != kMaskLit ? fast_exp2(cum_me - e_first) : 1.f;
            const float rowf_a = KIND != kMaskLit ? fast_exp2(e_last - cum_me) : 1.f;
#pragma unroll 1
            for (int h = 0; h < CT / kKB; ++h) {
                if (!live || h * kKB >= n) break;   // keys past the chunk's end are zero rows
                if (causal && h * kKB > 16 * tw + 15) break;   // every key after every query of the tile
                // 0: overlap, 1: every key before the tile's rows, 2: every key after them (wave-uniform)
                const int region = h * kKB + kKB - 1 < 16 * tw ? 1 : h * kKB > 16 * tw + 15 ? 2 : 0;
                float cl = 1.f;
                if (KIND != kMaskLit && region != 0) {
                    const float ej = cum[h * kKB + 16 * ((r >> 2) & 1) + 4 * g + (r & 3)];
                    cl = fast_exp2(region == 1 ? e_first - ej : ej - e_last);
                }
                f32x4 sacc[2], dpacc[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    sacc[t] = dpacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < NS; ++st) {
                        sacc[t] = mfma_bf16(rows_frag<D>(Kt, h, t, st, r, g), qf[st], sacc[t]);
                        dpacc[t] = mfma_bf16(rows_frag<D>(Vt, h, t, st, r, g), df[st], dpacc[t]);
                    }
                }
                // element (t, e): key j = 32 h + 16 t + 4 g + e, query i_me
                bf16x8 dsf;
                if (region == 0) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const f32x4 cj = *reinterpret_cast<const f32x4 *>(cum + h * kKB + 16 * t + 4 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int j = h * kKB + 16 * t + 4 * g + e;
                            float m = KIND != kMaskLit ? fast_exp2(-__builtin_fabsf(cum_me - cj[e])) : 1.f;
                            if (causal && j > i_me) m = 0.f;
                            const float dp = dpacc[t][e] * inv_me - dl_me;
                            const float wv = dp * (sacc[t][e] * m);
                            rowterm += j < i_me ? wv : (j > i_me ? -wv : 0.f);
                            dsf[4 * t + e] = f2bf(dp * m);
                        }
                    }
                } else {
                    const float rowf = region == 1 ? rowf_b : rowf_a;
                    float wsum = 0.f;
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float m = KIND != kMaskLit ? bwd_bcast16(cl, 4 * t + e) * rowf : 1.f;
                            const float dp = dpacc[t][e] * inv_me - dl_me;
                            wsum += dp * (sacc[t][e] * m);
                            dsf[4 * t + e] = f2bf(dp * m);
                        }
                    rowterm += region == 1 ? wsum : -wsum;
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) aq[ct] = mfma_bf16(tr_frag<D>(Kt, h, ct, r, g), dsf, aq[ct]);
            }
            // the keys' states: dphi(q) += f (F dy / den - F_d delta), F rows as A and dy of the query row as
            // B; the row half of dA takes phi(q) . that (phi(q) at the output layout's channels)
            rounds([&](const __bf16 *S, const float *z, int st) {
                if (st & 1) return;   // a queries' state: the key side's
                const bool right = st >= 2;
                const float f = KIND == kMaskLit ? 1.f : fast_exp2(right ? tot - cum_me : cum_me);
                float part = 0.f;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st2 = 0; st2 < NS; ++st2) o = mfma_bf16(rows_frag<D>(S, ct >> 1, ct & 1, st2, r, g), df[st2], o);
                    const f32x4 zc = *reinterpret_cast<const f32x4 *>(z + 16 * ct + 4 * g);
                    const bf16x4 q4 = row4<D>(Qt, i_me, 16 * ct + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float oe = o[e] * inv_me - zc[e] * dl_me;
                        aq[ct][e] += f * oe;
                        part += (float)q4[e] * oe;
                    }
                }
                rowterm += (right ? -f : f) * part;
            });
            rowterm += __shfl_xor(rowterm, 16, 64);
            rowterm += __shfl_xor(rowterm, 32, 64);
            if (i_me < n) {
                if constexpr (KIND != kMaskD) {
                    float xq[NCT][4];
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        const bf16x4 q4 = *reinterpret_cast<const bf16x4 *>(p.q + rowg * D + 16 * ct + 4 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e) xq[ct][e] = (float)q4[e];
                    }
                    phi_backward<D, KIND>(xq, aq);
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) store4(p.dq, gb, rowg * D + 16 * ct + 4 * g, aq[ct]);
                if constexpr (KIND != kMaskLit) {
                    if (g == 0) {
                        if (fuse_dll) tsum += (double)i_me * (double)rowterm;
                        else p.da_row[rowg] = rowterm;
                    }
                }
            }
        }
    } else {
#pragma unroll 1
        for (int kt = 0; kt < TPW; ++kt) {
            const int tw = kt == 0 ? wq : NW - 1 - wq;   // as the query side
            const int i_me = 16 * tw + r;   // this lane's row of the tile
            const float cum_me = cum[i_me];
            const size_t rowg = row0 + i_me;
            const bool live = 16 * tw < n;   // wave-uniform; a tile wholly past the chunk's end computes nothing
            // ---- key side: dV^T and dphi(K)^T (channel 16 ct + 4 g + e, key i_me) against the chunk's queries
            bf16x8 kf[NS], vf[NS];
            if constexpr (SPLIT) {
                const size_t rc = row0 + min(i_me, n - 1);
                row_frags<D, KIND, true>(p.k + rc * D, i_me < n, kf);
                row_frags<D, KIND, false>(p.v + rc * D, i_me < n, vf);
            } else {
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    kf[st] = rows_frag<D>(Kt, tw >> 1, tw & 1, st, r, g);
                    vf[st] = rows_frag<D>(Vt, tw >> 1, tw & 1, st, r, g);
                }
            }
            f32x4 ak[NCT], av[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) ak[ct] = av[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            float colterm = 0.f;
            // Separable mask for query sub-blocks wholly before or after the tile's keys (first key k0, last
            // kl): M_ij = exp2(c_j - c_k0) exp2(c_k0 - c_i) for queries before, exp2(c_kl - c_j) exp2(c_i - c_kl)
            // for queries after; the query's factor comes by DPP row broadcast.
            const float e_first = uniform(cum[16 * tw]), e_last = uniform(cum[16 * tw + 15]);
            const float keyf_b = KIND != kMaskLit ? fast_exp2(cum_me - e_first) : 1.f;
            const float keyf_a = KIND != kMaskLit ? fast_exp2(e_last - cum_me) : 1.f;
#pragma unroll 1
            for (int h = 0; h < CT / kKB; ++h) {
                if (!live || h * kKB >= n) break;   // queries past the chunk's end are zero rows
                if (causal && h * kKB + kKB - 1 < 16 * tw) continue;   // every query before every key of the tile
                // 0: overlap, 1: every query before the tile's keys, 2: every query after them (wave-uniform)
                const int region = h * kKB + kKB - 1 < 16 * tw ? 1 : h * kKB > 16 * tw + 15 ? 2 : 0;
                float cl = 1.f;
                if (KIND != kMaskLit && region != 0) {
                    const float ei = cum[h * kKB + 16 * ((r >> 2) & 1) + 4 * g + (r & 3)];
                    cl = fast_exp2(region == 1 ? e_first - ei : ei - e_last);
                }
                f32x4 sacc[2], dpacc[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    sacc[t] = dpacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < NS; ++st) {
                        sacc[t] = mfma_bf16(rows_frag<D>(Qt, h, t, st, r, g), kf[st], sacc[t]);
                        dpacc[t] = mfma_bf16(rows_frag<D>(Gt, h, t, st, r, g), vf[st], dpacc[t]);
                    }
                }
                // element (t, e): query i = 32 h + 16 t + 4 g + e, key i_me
                bf16x8 pf, dsf;
                const float keyf = region == 1 ? keyf_b : keyf_a;
                float wsum = 0.f;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int ib = h * kKB + 16 * t + 4 * g;
                    const f32x4 iv = *reinterpret_cast<const f32x4 *>(inv + ib);
                    const f32x4 dv4 = *reinterpret_cast<const f32x4 *>(dl + ib);
                    if (region == 0) {
                        const f32x4 ci = *reinterpret_cast<const f32x4 *>(cum + ib);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int i = ib + e;
                            float m = KIND != kMaskLit ? fast_exp2(-__builtin_fabsf(ci[e] - cum_me)) : 1.f;
                            if (causal && i_me > i) m = 0.f;
                            const float pm = sacc[t][e] * m;
                            const float dp = dpacc[t][e] * iv[e] - dv4[e];
                            const float wv = dp * pm;
                            colterm += i < i_me ? wv : (i > i_me ? -wv : 0.f);
                            pf[4 * t + e] = f2bf(pm * iv[e]);
                            dsf[4 * t + e] = f2bf(dp * m);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float m = KIND != kMaskLit ? bwd_bcast16(cl, 4 * t + e) * keyf : 1.f;
                            const float pm = sacc[t][e] * m;
                            const float dp = dpacc[t][e] * iv[e] - dv4[e];
                            wsum += dp * pm;
                            pf[4 * t + e] = f2bf(pm * iv[e]);
                            dsf[4 * t + e] = f2bf(dp * m);
                        }
                    }
                }
                if (region != 0) colterm += region == 1 ? wsum : -wsum;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    av[ct] = mfma_bf16(tr_frag<D>(Gt, h, ct, r, g), pf, av[ct]);
                    ak[ct] = mfma_bf16(tr_frag<D>(Qt, h, ct, r, g), dsf, ak[ct]);
                }
            }
            // phi(k) of the key row at channels 32 hh + 16 t + 4 g + e: the transposed-slot B operand of dv
            // and, with ct = 2 hh + t, the output layout's channels 16 ct + 4 g + e
            bf16x8 kT[NS];
            if constexpr (SPLIT) {
                // from memory: phi, and LION-S's normalisation over the row's four lane groups
                const __bf16 *kr = p.k + (row0 + min(i_me, n - 1)) * D;
                float x[NS][8], ss = 0.f;
#pragma unroll
                for (int hh = 0; hh < NS; ++hh) {
                    const bf16x4 k0 = *reinterpret_cast<const bf16x4 *>(kr + 32 * hh + 4 * g);
                    const bf16x4 k1 = *reinterpret_cast<const bf16x4 *>(kr + 32 * hh + 16 + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[hh][e] = phi_pre<KIND>((float)k0[e]);
                        x[hh][4 + e] = phi_pre<KIND>((float)k1[e]);
                        ss += x[hh][e] * x[hh][e] + x[hh][4 + e] * x[hh][4 + e];
                    }
                }
                float sc = i_me < n ? 1.f : 0.f;
                if constexpr (KIND == kMaskS) {
                    ss += __shfl_xor(ss, 16, 64);
                    ss += __shfl_xor(ss, 32, 64);
                    sc *= inv_norm(ss);
                }
#pragma unroll
                for (int hh = 0; hh < NS; ++hh)
#pragma unroll
                    for (int e = 0; e < 8; ++e) kT[hh][e] = f2bf(x[hh][e] * sc);
            } else {
#pragma unroll
                for (int hh = 0; hh < NS; ++hh) {
                    const bf16x4 k0 = row4<D>(Kt, i_me, 32 * hh + 4 * g), k1 = row4<D>(Kt, i_me, 32 * hh + 16 + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kT[hh][e] = k0[e];
                        kT[hh][4 + e] = k1[e];
                    }
                }
            }
            // the queries' states: dphi(k) += f (G v + G_d), G rows as A and v of the key row as B; dv += f G^T
            // phi(k), G read transposed as A; the column half of dA takes phi(k) . (G v + G_d)
            rounds([&](const __bf16 *S, const float *z, int st) {
                if (!(st & 1)) return;   // a keys' state: the query side's
                const bool right = st >= 2;
                const float f = KIND == kMaskLit ? 1.f : fast_exp2(right ? tot - cum_me : cum_me);
                float part = 0.f;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    f32x4 o = {0.f, 0.f, 0.f, 0.f}, ov = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st2 = 0; st2 < NS; ++st2) {
                        o = mfma_bf16(rows_frag<D>(S, ct >> 1, ct & 1, st2, r, g), vf[st2], o);
                        ov = mfma_bf16(tr_frag<D>(S, st2, ct, r, g), kT[st2], ov);
                    }
                    const f32x4 zc = *reinterpret_cast<const f32x4 *>(z + 16 * ct + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float oe = o[e] + zc[e];
                        ak[ct][e] += f * oe;
                        av[ct][e] += f * ov[e];
                        part += (float)kT[ct >> 1][4 * (ct & 1) + e] * oe;
                    }
                }
                colterm += (right ? -f : f) * part;
            });
            colterm += __shfl_xor(colterm, 16, 64);
            colterm += __shfl_xor(colterm, 32, 64);
            if (i_me < n) {
                if constexpr (KIND != kMaskD) {
                    float xk[NCT][4];
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        const bf16x4 k4 = *reinterpret_cast<const bf16x4 *>(p.k + rowg * D + 16 * ct + 4 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e) xk[ct][e] = (float)k4[e];
                    }
                    phi_backward<D, KIND>(xk, ak);
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    store4(p.dk, gb, rowg * D + 16 * ct + 4 * g, ak[ct]);
                    store4(p.dv, gb, rowg * D + 16 * ct + 4 * g, av[ct]);
                }
                if constexpr (KIND != kMaskLit) {
                    if (g == 0) {
                        if (fuse_dll) tsum += (double)i_me * (double)colterm;
                        else p.da_col[rowg] = colterm;
                    }
                }
            }
        }
    }
    if constexpr (KIND == kMaskD) {
        if (fuse_dll) {
            // each side's waves add their shares in fp64 (the states' last-column space is free: no
            // states) and the side's first wave leaves the sum as a hi/lo float pair
            double *red = reinterpret_cast<double *>(zst);
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) tsum += __shfl_xor(tsum, o, 64);
            if (lane == 0) red[w] = tsum;
            __syncthreads();
            if (lane == 0 && (w == 0 || (!SPLIT && w == NQW))) {
                double sum = 0.0;
                for (int k = 0; k < NQW; ++k) sum += red[w + k];
                const float hi = (float)sum;
                float *dst = p.dll_part + ((size_t)bh * 2 + (qside ? 0 : 1)) * 2;
                dst[0] = hi;
                dst[1] = (float)(sum - (double)hi);
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

struct MbLayout {
    size_t st, stz, da, bytes;   // byte offsets into the workspace
};

MbLayout mb_layout(int B, int H, int L, int d, int C) {
    const size_t bh = (size_t)B * H, nch = (size_t)((L + C - 1) / C);
    MbLayout w;
    w.st = 0;
    w.stz = w.st + bh * nch * 4 * (size_t)d * d * 2;
    w.da = w.stz + bh * nch * 4 * (size_t)d * 4;
    w.bytes = w.da + 2 * (((bh * L) + 3) / 4) * 4 * 4;
    return w;
}

size_t mb_main_lds(int d, int C) {
    const size_t f32 = (size_t)(C + 4) + 2 * (size_t)C + 4 * (size_t)d;
    return (size_t)4 * C * d * 2 + f32 * 4;
}

MbParams mb_params(const BwdArgs &a, int C) {
    MbParams p{};
    p.q = reinterpret_cast<const __bf16 *>(a.q);
    p.k = reinterpret_cast<const __bf16 *>(a.k);
    p.v = reinterpret_cast<const __bf16 *>(a.v);
    p.y = reinterpret_cast<const __bf16 *>(a.y);
    p.dy = reinterpret_cast<const __bf16 *>(a.dy);
    p.den = a.den;
    p.ll = a.log_lambda;
    p.H = a.H;
    p.L = a.L;
    p.nch = (a.L + C - 1) / C;
    p.causal = a.causal ? 1 : 0;
    p.dq = a.dq;
    p.dk = a.dk;
    p.dv = a.dv;
    p.g_bf16 = a.g_bf16 ? 1 : 0;
    p.nbh = a.B * a.H;
    return p;
}

template <int D, int KIND, int CT, bool SPLIT = false>
hipError_t launch_main_dll(const MbParams &p, const BwdArgs &a, hipStream_t stream) {
    constexpr size_t lm = MainLds<D, CT, SPLIT>::BYTES;
    allow_lds(&mb_main_kernel<D, KIND, CT, SPLIT>, lm);
    const int grid = SPLIT ? 16 * ((a.B * a.H + 7) / 8) : a.B * a.H * p.nch;
    const int nt = SPLIT ? main_threads(CT) / 2 : main_threads(CT);
    hipLaunchKernelGGL((mb_main_kernel<D, KIND, CT, SPLIT>), dim3(grid), dim3(nt), lm, stream, p);
    if (KIND != kMaskLit) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (p.dll_part != nullptr) return launch_dll_parts(p.dll_part, a.dll, a.B, a.H, stream);
        return launch_dll(KIND, p.da_row, p.da_col, a.dll, a.B, a.H, a.L, stream);
    }
    return hipGetLastError();
}

template <int D, int KIND, int CT>
hipError_t launch_mb_t(const BwdArgs &a, hipStream_t stream) {
    const MbLayout w = mb_layout(a.B, a.H, a.L, a.d, CT);
    unsigned char *ws = reinterpret_cast<unsigned char *>(a.workspace);
    MbParams p = mb_params(a, CT);
    p.st = reinterpret_cast<__bf16 *>(ws + w.st);
    p.stz = reinterpret_cast<float *>(ws + w.stz);
    const size_t n = (size_t)a.B * a.H * a.L;
    p.da_row = reinterpret_cast<float *>(ws + w.da);
    p.da_col = p.da_row + ((n + 3) / 4) * 4;
    if (p.nch > 1) {
        constexpr size_t lw = WalkLds<D, CT>::BYTES;
        allow_lds(&mb_walk_kernel<D, KIND, CT>, lw);
        hipLaunchKernelGGL((mb_walk_kernel<D, KIND, CT>), dim3(a.B * a.H * (a.causal ? 2 : 4)), dim3(kWalkThreads), lw,
                           stream, p);
    }
    return launch_main_dll<D, KIND, CT>(p, a, stream);
}

// The whole sequence as one chunk (no walk, no states).  The two sides go to workgroups of their own
// (two per compute unit) unless one workgroup per (batch, head) fills a single round of the 256 compute
// units while the split would put two on some of them (128 < B H <= 256); LION-D's heavier mask work
// makes the split pay there as well.  The dA halves go to the full form's workspace (3 B H L floats, of
// which the last two thirds).
constexpr size_t kComputeUnits = 256;

template <int D, int KIND, int CT>
hipError_t launch_single_c(const MbParams &p, const BwdArgs &a, hipStream_t stream) {
    const size_t pairs = (size_t)a.B * a.H;
    const bool one_round = pairs > kComputeUnits / 2 && pairs <= kComputeUnits;
    if (KIND == kMaskD || !one_round) return launch_main_dll<D, KIND, CT, true>(p, a, stream);
    return launch_main_dll<D, KIND, CT, false>(p, a, stream);
}

template <int D, int KIND>
hipError_t launch_single_t(const BwdArgs &a, hipStream_t stream) {
    const int C = a.L <= 64 ? 64 : a.L <= 128 ? 128 : 256;
    MbParams p = mb_params(a, C);
    const size_t n = (size_t)a.B * a.H * a.L;
    p.da_row = reinterpret_cast<float *>(a.workspace) + n;
    p.da_col = p.da_row + n;
    // LION-D, L >= 4: the token sums of dA are formed in the kernel, into the first third (4 B H floats)
    if (KIND == kMaskD && a.L >= 4) p.dll_part = reinterpret_cast<float *>(a.workspace);
    if (C == 64) return launch_single_c<D, KIND, 64>(p, a, stream);
    if (C == 128) return launch_single_c<D, KIND, 128>(p, a, stream);
    return launch_single_c<D, KIND, 256>(p, a, stream);
}

template <int D>
hipError_t launch_single_kind(const BwdArgs &a, hipStream_t stream) {
    switch (a.kind) {
    case kMaskLit: return launch_single_t<D, kMaskLit>(a, stream);
    case kMaskD: return launch_single_t<D, kMaskD>(a, stream);
    default: return launch_single_t<D, kMaskS>(a, stream);
    }
}

template <int D, int KIND>
hipError_t launch_mb_c(const BwdArgs &a, hipStream_t stream) {
    if (a.C == 64) return launch_mb_t<D, KIND, 64>(a, stream);
    if constexpr (D != 128) return launch_mb_t<D, KIND, 128>(a, stream);
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_mb_kind(const BwdArgs &a, hipStream_t stream) {
    switch (a.kind) {
    case kMaskLit: return launch_mb_c<D, kMaskLit>(a, stream);
    case kMaskD: return launch_mb_c<D, kMaskD>(a, stream);
    default: return launch_mb_c<D, kMaskS>(a, stream);
    }
}

}  // namespace

Plan plan_chunk_bwd_mfma(const BwdArgs &a) {
    Plan p;
    const bool dims = a.d == 32 || a.d == 64 || a.d == 128;
    const bool cs = a.C == 64 || (a.C == 128 && a.d != 128);
    p.ok = dims && cs && mb_main_lds(a.d, a.C) <= kLdsPerWorkgroup;
    p.workspace = p.ok ? mb_layout(a.B, a.H, a.L, a.d, a.C).bytes : 0;
    return p;
}

bool single_chunk_bwd_ok(const BwdArgs &a) { return (a.d == 32 || a.d == 64) && a.L >= 1 && a.L <= 256; }

hipError_t launch_single_chunk_bwd(const BwdArgs &a, hipStream_t stream) {
    return a.d == 32 ? launch_single_kind<32>(a, stream) : launch_single_kind<64>(a, stream);
}

hipError_t launch_chunk_bwd_mfma(const BwdArgs &a, hipStream_t stream) {
    switch (a.d) {
    case 32: return launch_mb_kind<32>(a, stream);
    case 64: return launch_mb_kind<64>(a, stream);
    default: return launch_mb_kind<128>(a, stream);
    }
}

}  // namespace lion
