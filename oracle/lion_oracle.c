/*
 * lion_oracle.c -- plain fp64 CPU oracle of LION bidirectional masked linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
 * bench.py may load this library.  It shares no code, header, table or helper with the GPU
 * library; neither side includes or imports the other.
 *
 * Sources (the pages this file is written from):
 *   [RB] "LION: A bidirectional framework that trains like a Transformer and infers like an RNN",
 *        author-reviewer discussion (paperhub copy of the ICLR 2025 forum).
 *   [OR] the same title, OpenReview forum header (TL;DR and abstract).
 *
 * What is computed is the full-form definition, written out term by term with no blocking,
 * fusion or reordering:
 *
 *   y_i = sum_j M_ij (phi(q_i) . phi(k_j)) v_j  /  ( sum_j M_ij (phi(q_i) . phi(k_j)) + eps )
 *
 *   - the attention form Y = SCALE(Q K^T (.) M) V                 [RB, reply "Concern 1", Theorem 3.3 Eq. 25]
 *   - SCALE divides each row by its own sum, as in linear attention y_i = q_i^T S_i / q_i^T z_i
 *                                                                 [RB, reply "1: Recurrence Form of Linear Attention"]
 *   - phi = elu()+1 for LION-LIT, silu normalised for LION-S     [RB, item 4 "Default non-linearity", Table 8]
 *   - LION-LIT has lambda_i = 1, a mask of all ones               [RB, item 5 "Equations 109 and 112"]
 *   - LION-RETNET (LION-D) a fixed per-head decay, LION-S an input-dependent lambda_i
 *                                                                 [RB, reply "(3) ... two distinct methodological contributions"]
 *   - heads are independent problems                              [RB, "Concern 2", item 3 (multi-head attention)]
 *
 * Readings where the pages leave a step open (each is listed with its reason in the design notes):
 *   - the mask entry M_ij is the product of the decays lambda_t for t strictly after min(i,j) up to
 *     and including max(i,j); M is symmetric with a unit diagonal.  This is the mask the forward
 *     recurrence S_i = lambda_i S_{i-1} + k_i v_i^T unrolls to below the diagonal, mirrored above it.
 *     Here it is formed as that product, directly, without logarithms or prefix sums.
 *   - eps is added to the row sum only.
 *   - the L2 normalisation of silu has no epsilon; an all-zero silu vector maps to phi = 0.
 *   - LION-D uses phi = identity.
 *
 * The causal (unidirectional) variant, mask_kind | ORACLE_CAUSAL, keeps only the keys at or before
 * the query: M_ij = 0 for j > i.  What remains is the forward recurrence alone -- causal linear
 * attention S_i = S_{i-1} + k_i v_i^T, z_i = z_{i-1} + k_i, y_i = q_i^T S_i / q_i^T z_i [RB, reply "1:
 * Recurrence Form of Linear Attention", Eq. 4a-4c] with the kind's decay, which the pages use for
 * single-directional generation (LION-S 1D) [RB, item 5 "Is this method limited to bidirectional
 * models?"].
 *
 * All arithmetic is IEEE double; build with plain -O2 (no fast-math), so the order of every sum is
 * the loop order written here.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MASK_LIT 0
#define ORACLE_MASK_D 1
#define ORACLE_MASK_S 2
#define ORACLE_CAUSAL 4

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

/* phi of one token's d channels.
 *   LIT:      elu(x) + 1  =  x + 1 for x > 0,  exp(x) otherwise        [RB, item 4]
 *   D:        identity
 *   S:        s = silu(x) = x * sigmoid(x) = x / (1 + exp(-x)), then s / ||s||_2 over the d channels [RB, item 4]
 */
static void phi_row(int kind, const double *x, int d, double *out)
{
    int c;
    if (kind == ORACLE_MASK_LIT) {
        for (c = 0; c < d; ++c)
            out[c] = x[c] > 0.0 ? x[c] + 1.0 : exp(x[c]);
    } else if (kind == ORACLE_MASK_D) {
        for (c = 0; c < d; ++c)
            out[c] = x[c];
    } else {
        double ss = 0.0, nrm;
        for (c = 0; c < d; ++c) {
            out[c] = x[c] / (1.0 + exp(-x[c]));
            ss += out[c] * out[c];
        }
        nrm = sqrt(ss);
        for (c = 0; c < d; ++c)
            out[c] = nrm > 0.0 ? out[c] / nrm : 0.0;
    }
}

/* Row i of the mask from the per-token decays lam[0..L-1] of one (batch, head):
 *   M_ii = 1,   M_ij = lam[i+1] * ... * lam[j]   (j > i),   M_ij = lam[j+1] * ... * lam[i]   (j < i).
 * lam[0] never enters.  Built as running products walking outward from the diagonal.  Causal:
 * M_ij = 0 for j > i. */
static void mask_row(const double *lam, int L, int i, int causal, double *m)
{
    int j;
    m[i] = 1.0;
    for (j = i + 1; j < L; ++j)
        m[j] = causal ? 0.0 : m[j - 1] * lam[j];
    for (j = i - 1; j >= 0; --j)
        m[j] = m[j + 1] * lam[j + 1];
}

/* One output row of one (batch, head): phq_i [d], phk/v [L, d], mask row m [L].
 * Writes y_i [d], the divisor den_i + eps, and (if asked) the absolute-value sums used by the
 * condition-aware parity gate:  absnum_c = sum_j Pbar_ij |v_jc|,  absden = sum_j Pbar_ij,
 * with Pbar_ij = M_ij * sum_c |phq_ic| |phk_jc|. */
static void attn_row(const double *phq_i, const double *phk, const double *v, const double *m, int L, int d,
                     double eps, double *num, double *anum, double *y_i, double *den_i, double *absnum_i,
                     double *absden_i)
{
    int j, c;
    double den = 0.0, aden = 0.0, s, sa, p, pa, div;
    for (c = 0; c < d; ++c) {
        num[c] = 0.0;
        anum[c] = 0.0;
    }
    for (j = 0; j < L; ++j) {
        const double *kj = phk + (size_t)j * d;
        const double *vj = v + (size_t)j * d;
        s = 0.0;
        sa = 0.0;
        for (c = 0; c < d; ++c) {
            s += phq_i[c] * kj[c];
            sa += fabs(phq_i[c]) * fabs(kj[c]);
        }
        p = s * m[j];
        pa = sa * m[j];
        den += p;
        aden += pa;
        for (c = 0; c < d; ++c) {
            num[c] += p * vj[c];
            anum[c] += pa * fabs(vj[c]);
        }
    }
    div = den + eps;
    for (c = 0; c < d; ++c)
        y_i[c] = num[c] / div;
    if (den_i)
        *den_i = div;
    if (absnum_i)
        for (c = 0; c < d; ++c)
            absnum_i[c] = anum[c];
    if (absden_i)
        *absden_i = aden;
}

/* phi over n rows of d channels. */
int lion_oracle_phi_f64(int kind, const double *x, long n, int d, double *out)
{
    long r;
    if (!x || !out || n < 0 || d < 1 || kind < ORACLE_MASK_LIT || kind > ORACLE_MASK_S)
        return ORACLE_EINVAL;
    for (r = 0; r < n; ++r)
        phi_row(kind, x + (size_t)r * d, d, out + (size_t)r * d);
    return ORACLE_OK;
}

/* The whole L x L mask of one sequence of decays lam[0..L-1] (test access to the mask itself). */
int lion_oracle_mask_f64(const double *lam, int L, double *M)
{
    int i;
    if (!lam || !M || L < 1)
        return ORACLE_EINVAL;
    for (i = 0; i < L; ++i)
        mask_row(lam, L, i, 0, M + (size_t)i * L);
    return ORACLE_OK;
}

/* Masked, row-normalised attention on inputs phi has already been applied to.
 *   phq, phk, v: [B, H, L, d]   lam: per-token decays [B, H, L]   eps >= 0
 *   y: [B, H, L, d]   den (nullable): [B, H, L] = row sum + eps
 *   absnum (nullable): [B, H, L, d]   absden (nullable): [B, H, L]
 * Independent (batch, head) problems are spread over OpenMP threads; each row's sums run in
 * index order. */
static int attn_all(const double *phq, const double *phk, const double *v, const double *lam, double eps, int causal,
                    int B, int H, int L, int d, double *y, double *den, double *absnum, double *absden)
{
    long bh, nbh;
    int err = 0;
    nbh = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (bh = 0; bh < nbh; ++bh) {
        double *m = (double *)malloc(sizeof(double) * (size_t)L);
        double *num = (double *)malloc(sizeof(double) * (size_t)d);
        double *anum = (double *)malloc(sizeof(double) * (size_t)d);
        size_t base = (size_t)bh * L;
        int i;
        if (!m || !num || !anum) {
            err |= 1;
        } else {
            for (i = 0; i < L; ++i) {
                size_t row = base + (size_t)i;
                mask_row(lam + base, L, i, causal, m);
                attn_row(phq + row * d, phk + base * d, v + base * d, m, L, d, eps, num, anum, y + row * d,
                         den ? den + row : NULL, absnum ? absnum + row * d : NULL, absden ? absden + row : NULL);
            }
        }
        free(m);
        free(num);
        free(anum);
    }
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}

int lion_oracle_attn_f64(const double *phq, const double *phk, const double *v, const double *lam, double eps, int B,
                         int H, int L, int d, double *y, double *den, double *absnum, double *absden)
{
    if (!phq || !phk || !v || !lam || !y || B < 1 || H < 1 || L < 1 || d < 1 || !(eps >= 0.0))
        return ORACLE_EINVAL;
    return attn_all(phq, phk, v, lam, eps, 0, B, H, L, d, y, den, absnum, absden);
}

/* Per-token decays of one (batch, head) from the log-decay argument as the GPU library takes it:
 *   LIT: lambda = 1 (log_lambda unused);  D: lambda_t = exp(log_lambda[h]);  S: lambda_t = exp(log_lambda[b,h,t]). */
static void decays(int kind, const double *log_lambda, int H, int L, long bh, double *lam)
{
    int t;
    for (t = 0; t < L; ++t) {
        if (kind == ORACLE_MASK_LIT)
            lam[t] = 1.0;
        else if (kind == ORACLE_MASK_D)
            lam[t] = exp(log_lambda[bh % H]);
        else
            lam[t] = exp(log_lambda[(size_t)bh * L + t]);
    }
}

/* The full definition from raw q, k, v:
 *   q, k, v: [B, H, L, d];  log_lambda: NULL (LIT), [H] (D) or [B, H, L] (S), every entry <= 0 and finite.
 *   Outputs as in lion_oracle_attn_f64. */
int lion_oracle_full_f64(const double *q, const double *k, const double *v, const double *log_lambda, int mask_kind,
                         double eps, int B, int H, int L, int d, double *y, double *den, double *absnum,
                         double *absden)
{
    size_t n, nt;
    double *phq, *phk, *lam;
    long bh;
    int rc;
    int causal = (mask_kind & ORACLE_CAUSAL) != 0;
    mask_kind &= ~ORACLE_CAUSAL;
    if (!q || !k || !v || !y || B < 1 || H < 1 || L < 1 || d < 1 || !(eps >= 0.0) ||
        mask_kind < ORACLE_MASK_LIT || mask_kind > ORACLE_MASK_S || (mask_kind != ORACLE_MASK_LIT && !log_lambda))
        return ORACLE_EINVAL;
    nt = (size_t)B * H * L;
    n = nt * d;
    phq = (double *)malloc(sizeof(double) * n);
    phk = (double *)malloc(sizeof(double) * n);
    lam = (double *)malloc(sizeof(double) * nt);
    if (!phq || !phk || !lam) {
        free(phq);
        free(phk);
        free(lam);
        return ORACLE_ENOMEM;
    }
    lion_oracle_phi_f64(mask_kind, q, (long)nt, d, phq);
    lion_oracle_phi_f64(mask_kind, k, (long)nt, d, phk);
    for (bh = 0; bh < (long)B * H; ++bh)
        decays(mask_kind, log_lambda, H, L, bh, lam + (size_t)bh * L);
    rc = attn_all(phq, phk, v, lam, eps, causal, B, H, L, d, y, den, absnum, absden);
    free(phq);
    free(phk);
    free(lam);
    return rc;
}

/* The same definition evaluated only at selected rows (for checks at sizes where every row would
 * take too long).  rows[r] = bh * L + i, in any order.  Outputs are packed per requested row:
 *   y: [nrows, d], den/absden: [nrows], absnum: [nrows, d]. */
int lion_oracle_rows_f64(const double *q, const double *k, const double *v, const double *log_lambda, int mask_kind,
                         double eps, int B, int H, int L, int d, const long *rows, long nrows, double *y, double *den,
                         double *absnum, double *absden)
{
    long r;
    int err = 0;
    int causal = (mask_kind & ORACLE_CAUSAL) != 0;
    mask_kind &= ~ORACLE_CAUSAL;
    if (!q || !k || !v || !y || !rows || nrows < 0 || B < 1 || H < 1 || L < 1 || d < 1 || !(eps >= 0.0) ||
        mask_kind < ORACLE_MASK_LIT || mask_kind > ORACLE_MASK_S || (mask_kind != ORACLE_MASK_LIT && !log_lambda))
        return ORACLE_EINVAL;
    for (r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= (long)B * H * L)
            return ORACLE_EINVAL;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (r = 0; r < nrows; ++r) {
        long bh = rows[r] / L;
        int i = (int)(rows[r] % L), j;
        size_t base = (size_t)bh * L;
        double *phk = (double *)malloc(sizeof(double) * (size_t)L * d);
        double *phq = (double *)malloc(sizeof(double) * (size_t)d);
        double *lam = (double *)malloc(sizeof(double) * (size_t)L);
        double *m = (double *)malloc(sizeof(double) * (size_t)L);
        double *num = (double *)malloc(sizeof(double) * (size_t)d);
        double *anum = (double *)malloc(sizeof(double) * (size_t)d);
        if (!phk || !phq || !lam || !m || !num || !anum) {
            err |= 1;
        } else {
            for (j = 0; j < L; ++j)
                phi_row(mask_kind, k + (base + j) * d, d, phk + (size_t)j * d);
            phi_row(mask_kind, q + (base + i) * d, d, phq);
            decays(mask_kind, log_lambda, H, L, bh, lam);
            mask_row(lam, L, i, causal, m);
            attn_row(phq, phk, v + base * d, m, L, d, eps, num, anum, y + (size_t)r * d, den ? den + r : NULL,
                     absnum ? absnum + (size_t)r * d : NULL, absden ? absden + r : NULL);
        }
        free(phk);
        free(phq);
        free(lam);
        free(m);
        free(num);
        free(anum);
    }
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}
