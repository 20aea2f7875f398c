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

/* ---- backward pass of the full form ------------------------------------------------------------------
 * The pages train the attention form ([OR] abstract and title; [RB] reply "Concern 1", Theorem 3.3
 * Eq. 25), so the gradient of the definition above is what training needs.  Nothing on
 * the pages spells it out; it is the chain rule applied to the definition, step by step, for a loss
 * whose gradient with respect to y is dy:
 *
 *   s_ij = phi(q_i).phi(k_j)      p_ij = M_ij s_ij      den_i = sum_j p_ij + eps      y_i = sum_j p_ij v_j / den_i
 *   g_i  = dy_i / den_i           delta_i = g_i . y_i
 *   dp_ij = g_i . v_j - delta_i                         (through the numerator and through den_i)
 *   dv_j = sum_i p_ij g_i
 *   dphi(q_i) = sum_j M_ij dp_ij phi(k_j)               dphi(k_j) = sum_i M_ij dp_ij phi(q_i)
 *   dq_i, dk_j = the Jacobian of phi at q_i, k_j (transposed) applied to those
 *   dM_ij = dp_ij s_ij
 *   M_ij = prod_{t = min(i,j)+1}^{max(i,j)} lambda_t, so d M_ij / d log(lambda_t) = M_ij for t in that
 *   range: dlog(lambda_t) = sum over the pairs (i, j) whose range holds t of dM_ij M_ij.  The range sums
 *   are taken with a difference array (add at min+1, subtract after max, then one running sum), the
 *   standard exact way to add a value over an index range.
 *   LION-D: every lambda_t of a head is exp(log_lambda[h]), so dlog_lambda[h] = the sum of those over
 *   every batch entry and token.  Causal: M_ij = 0 for j > i is a constant, contributing nothing.
 *
 * Optional absolute-value companions (for the condition-aware parity gate, like absnum/absden of the
 * forward): the same steps with every term replaced by its magnitude and every difference by a sum.
 * The divisor and y come from the forward, whose first-order error (relative u per term) is at most
 * u sum_j pbar_ij for den_i and u (sum_j pbar_ij |v_j| + |y_i| sum_j pbar_ij) / |den_i| for y_i
 * (pbar_ij = M_ij sum_c |phi(q_i)_c| |phi(k_j)_c|, aden_i = sum_j pbar_ij), so those enter as
 *   ag_i = |dy_i| (|den_i| + aden_i) / den_i^2,   ay_i = |y_i| + (sum_j pbar_ij |v_j| + |y_i| aden_i) / |den_i|,
 *   adelta_i = sum_c ag_ic ay_ic,   adp_ij = sum_c ag_ic |v_jc| + adelta_i,   adv_j = sum_i pbar_ij ag_i,
 *   adphi(q_i) = sum_j M_ij adp_ij |phi(k_j)|,   adphi(k_j) = sum_i M_ij adp_ij |phi(q_i)|,
 *   then phi's Jacobian in absolute values, and adlog(lambda_t) = the range sums of adp_ij pbar_ij.
 * A relative error of u in every term (and in den and y as above) moves each gradient by at most about
 * u times its companion: the first-order bound, as in the forward's gate. */

/* The Jacobian of phi at x, transposed, applied to g (one token's d channels).
 *   LIT: d(elu(x)+1)/dx = 1 for x > 0, exp(x) otherwise.   D: identity.
 *   S: phi = s / ||s|| with s = silu(x): dphi/ds = (I - phi phi^T) / ||s||, and
 *      dsilu/dx = sigmoid(x) (1 + x (1 - sigmoid(x))).  ||s|| = 0 gives 0 (phi is 0 there). */
static void phi_grad_row(int kind, const double *x, const double *g, int d, double *dx);

/* |Jacobian of phi|^T applied to a non-negative vector a (the companion of phi_grad_row):
 *   LIT |phi'| a;  D a;  S |silu'| (a + |phi| (|phi| . a)) / ||silu(x)||. */
static void phi_grad_abs_row(int kind, const double *x, const double *a, int d, double *out)
{
    int c;
    if (kind == ORACLE_MASK_LIT) {
        for (c = 0; c < d; ++c)
            out[c] = a[c] * (x[c] > 0.0 ? 1.0 : exp(x[c]));
    } else if (kind == ORACLE_MASK_D) {
        for (c = 0; c < d; ++c)
            out[c] = a[c];
    } else {
        double ss = 0.0, nrm, pa = 0.0;
        for (c = 0; c < d; ++c) {
            const double sv = x[c] / (1.0 + exp(-x[c]));
            ss += sv * sv;
        }
        nrm = sqrt(ss);
        for (c = 0; c < d; ++c) {
            const double sv = x[c] / (1.0 + exp(-x[c]));
            pa += (nrm > 0.0 ? fabs(sv) / nrm : 0.0) * a[c];
        }
        for (c = 0; c < d; ++c) {
            const double sig = 1.0 / (1.0 + exp(-x[c]));
            const double ph = nrm > 0.0 ? fabs(x[c] * sig) / nrm : 0.0;
            out[c] = nrm > 0.0 ? fabs(sig * (1.0 + x[c] * (1.0 - sig))) * (a[c] + ph * pa) / nrm : 0.0;
        }
    }
}

static void phi_grad_row(int kind, const double *x, const double *g, int d, double *dx)
{
    int c;
    if (kind == ORACLE_MASK_LIT) {
        for (c = 0; c < d; ++c)
            dx[c] = g[c] * (x[c] > 0.0 ? 1.0 : exp(x[c]));
    } else if (kind == ORACLE_MASK_D) {
        for (c = 0; c < d; ++c)
            dx[c] = g[c];
    } else {
        double ss = 0.0, nrm, pg = 0.0;
        for (c = 0; c < d; ++c) {
            const double sv = x[c] / (1.0 + exp(-x[c]));
            ss += sv * sv;
        }
        nrm = sqrt(ss);
        for (c = 0; c < d; ++c) {
            const double sv = x[c] / (1.0 + exp(-x[c]));
            pg += (nrm > 0.0 ? sv / nrm : 0.0) * g[c];
        }
        for (c = 0; c < d; ++c) {
            const double sig = 1.0 / (1.0 + exp(-x[c]));
            const double ph = nrm > 0.0 ? x[c] * sig / nrm : 0.0;
            dx[c] = nrm > 0.0 ? sig * (1.0 + x[c] * (1.0 - sig)) * (g[c] - ph * pg) / nrm : 0.0;
        }
    }
}

/* Gradients of the full definition.
 *   q, k, v, dy: [B, H, L, d];  log_lambda as for lion_oracle_full_f64;  mask_kind may carry ORACLE_CAUSAL.
 *   dq, dk, dv: [B, H, L, d];  dll: NULL for LIT, [H] for D, [B, H, L] for S (entry t = 0 is always 0:
 *   lambda_0 never enters the mask). */
int lion_oracle_full_bwd_f64(const double *q, const double *k, const double *v, const double *log_lambda,
                             int mask_kind, double eps, int B, int H, int L, int d, const double *dy, double *dq,
                             double *dk, double *dv, double *dll, double *adq, double *adk, double *adv,
                             double *adll)
{
    long bh, nbh = (long)B * H;
    int err = 0, kind, causal, want_abs = adq && adk && adv;
    double *dll_tok, *adll_tok;
    causal = (mask_kind & ORACLE_CAUSAL) != 0;
    kind = mask_kind & ~ORACLE_CAUSAL;
    if (!q || !k || !v || !dy || !dq || !dk || !dv || B < 1 || H < 1 || L < 1 || d < 1 || !(eps >= 0.0) ||
        kind < ORACLE_MASK_LIT || kind > ORACLE_MASK_S || (kind != ORACLE_MASK_LIT && (!log_lambda || !dll)))
        return ORACLE_EINVAL;
    dll_tok = (double *)calloc((size_t)nbh * L, sizeof(double));
    adll_tok = (double *)calloc((size_t)nbh * L, sizeof(double));
    if (!dll_tok || !adll_tok) {
        free(dll_tok);
        free(adll_tok);
        return ORACLE_ENOMEM;
    }
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (bh = 0; bh < nbh; ++bh) {
        size_t base = (size_t)bh * L;
        double *phq = (double *)malloc(sizeof(double) * (size_t)L * d);
        double *phk = (double *)malloc(sizeof(double) * (size_t)L * d);
        double *dphq = (double *)calloc((size_t)L * d, sizeof(double));
        double *dphk = (double *)calloc((size_t)L * d, sizeof(double));
        double *lam = (double *)malloc(sizeof(double) * (size_t)L);
        double *m = (double *)malloc(sizeof(double) * (size_t)L);
        double *s = (double *)malloc(sizeof(double) * (size_t)L);
        double *y = (double *)malloc(sizeof(double) * (size_t)d);
        double *g = (double *)malloc(sizeof(double) * (size_t)d);
        double *diff = (double *)calloc((size_t)L + 1, sizeof(double));
        double *aphq = (double *)calloc((size_t)L * d, sizeof(double));
        double *aphk = (double *)calloc((size_t)L * d, sizeof(double));
        double *adiff = (double *)calloc((size_t)L + 1, sizeof(double));
        double *ag = (double *)malloc(sizeof(double) * (size_t)d);
        double *apv = (double *)malloc(sizeof(double) * (size_t)d);
        int i, j, c;
        if (!phq || !phk || !dphq || !dphk || !lam || !m || !s || !y || !g || !diff || !aphq || !aphk || !adiff ||
            !ag || !apv) {
            err |= 1;
        } else {
            for (j = 0; j < L; ++j) {
                phi_row(kind, q + (base + j) * d, d, phq + (size_t)j * d);
                phi_row(kind, k + (base + j) * d, d, phk + (size_t)j * d);
            }
            decays(kind, log_lambda, H, L, bh, lam);
            for (c = 0; c < L * d; ++c) {
                dv[base * d + c] = 0.0;
                if (want_abs)
                    adv[base * d + c] = 0.0;
            }
            for (i = 0; i < L; ++i) {
                const double *pq = phq + (size_t)i * d;
                const double *dyi = dy + (base + i) * d;
                double den = 0.0, delta = 0.0;
                mask_row(lam, L, i, causal, m);
                /* forward row: scores, row sum, output */
                for (c = 0; c < d; ++c)
                    y[c] = 0.0;
                for (j = 0; j < L; ++j) {
                    double sc = 0.0;
                    for (c = 0; c < d; ++c)
                        sc += pq[c] * phk[(size_t)j * d + c];
                    s[j] = sc;
                    den += m[j] * sc;
                    for (c = 0; c < d; ++c)
                        y[c] += m[j] * sc * v[(base + j) * d + c];
                }
                den += eps;
                for (c = 0; c < d; ++c) {
                    y[c] /= den;
                    g[c] = dyi[c] / den;
                    delta += g[c] * y[c];
                }
                if (want_abs) {
                    /* the absolute-value companion of this row (see the comment above) */
                    double adelta = 0.0, aden = 0.0;
                    for (c = 0; c < d; ++c)
                        apv[c] = 0.0;
                    for (j = 0; j < L; ++j) {
                        double pbar = 0.0;
                        for (c = 0; c < d; ++c)
                            pbar += fabs(pq[c]) * fabs(phk[(size_t)j * d + c]);
                        pbar *= m[j];
                        aden += pbar;
                        for (c = 0; c < d; ++c)
                            apv[c] += pbar * fabs(v[(base + j) * d + c]);
                    }
                    for (c = 0; c < d; ++c) {
                        const double ay = fabs(y[c]) + (apv[c] + fabs(y[c]) * aden) / fabs(den);
                        ag[c] = fabs(dyi[c]) * (fabs(den) + aden) / (den * den);
                        adelta += ag[c] * ay;
                    }
                    for (j = 0; j < L; ++j) {
                        double agv = 0.0, pbar = 0.0, adp;
                        for (c = 0; c < d; ++c) {
                            agv += ag[c] * fabs(v[(base + j) * d + c]);
                            pbar += fabs(pq[c]) * fabs(phk[(size_t)j * d + c]);
                        }
                        pbar *= m[j];
                        adp = agv + adelta;
                        for (c = 0; c < d; ++c) {
                            adv[(base + j) * d + c] += pbar * ag[c];
                            aphq[(size_t)i * d + c] += m[j] * adp * fabs(phk[(size_t)j * d + c]);
                            aphk[(size_t)j * d + c] += m[j] * adp * fabs(pq[c]);
                        }
                        if (j != i) {
                            const int lo = i < j ? i : j, hi = i < j ? j : i;
                            adiff[lo + 1] += adp * pbar;
                            adiff[hi + 1] -= adp * pbar;
                        }
                    }
                }
                /* backward row */
                for (j = 0; j < L; ++j) {
                    double gv = 0.0, dp, ds;
                    for (c = 0; c < d; ++c)
                        gv += g[c] * v[(base + j) * d + c];
                    dp = gv - delta;
                    for (c = 0; c < d; ++c)
                        dv[(base + j) * d + c] += m[j] * s[j] * g[c];
                    ds = m[j] * dp;
                    for (c = 0; c < d; ++c) {
                        dphq[(size_t)i * d + c] += ds * phk[(size_t)j * d + c];
                        dphk[(size_t)j * d + c] += ds * pq[c];
                    }
                    /* dlog(lambda_t) += dM_ij M_ij for min(i,j) < t <= max(i,j) */
                    if (j != i) {
                        const double w = dp * s[j] * m[j];
                        const int lo = i < j ? i : j, hi = i < j ? j : i;
                        diff[lo + 1] += w;
                        diff[hi + 1] -= w;
                    }
                }
            }
            for (j = 0; j < L; ++j) {
                phi_grad_row(kind, q + (base + j) * d, dphq + (size_t)j * d, d, dq + (base + j) * d);
                phi_grad_row(kind, k + (base + j) * d, dphk + (size_t)j * d, d, dk + (base + j) * d);
                if (want_abs) {
                    phi_grad_abs_row(kind, q + (base + j) * d, aphq + (size_t)j * d, d, adq + (base + j) * d);
                    phi_grad_abs_row(kind, k + (base + j) * d, aphk + (size_t)j * d, d, adk + (base + j) * d);
                }
            }
            {
                double run = 0.0, arun = 0.0;
                for (j = 0; j < L; ++j) {
                    run += diff[j];
                    dll_tok[base + j] = run;
                    arun += adiff[j];
                    adll_tok[base + j] = arun;
                }
            }
        }
        free(phq);
        free(phk);
        free(dphq);
        free(dphk);
        free(lam);
        free(m);
        free(s);
        free(y);
        free(g);
        free(diff);
        free(aphq);
        free(aphk);
        free(adiff);
        free(ag);
        free(apv);
    }
    if (!err && kind == ORACLE_MASK_S) {
        memcpy(dll, dll_tok, sizeof(double) * (size_t)nbh * L);
        if (adll)
            memcpy(adll, adll_tok, sizeof(double) * (size_t)nbh * L);
    } else if (!err && kind == ORACLE_MASK_D) {
        int h, t;
        long b2;
        for (h = 0; h < H; ++h) {
            double acc = 0.0, aacc = 0.0;
            for (b2 = 0; b2 < B; ++b2)
                for (t = 0; t < L; ++t) {
                    acc += dll_tok[((size_t)b2 * H + h) * L + t];
                    aacc += adll_tok[((size_t)b2 * H + h) * L + t];
                }
            dll[h] = acc;
            if (adll)
                adll[h] = aacc;
        }
    }
    free(dll_tok);
    free(adll_tok);
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}

/* ---- selectivity prologue of LION-S ------------------------------------------------------------------
 * LION-S takes an input-dependent decay lambda_i, the scalar version of Mamba-2's state matrix [RB,
 * reply "1. Some equations/notations are not clear enough", Eq. 5a], and the pages derive its two
 * coefficients from zero-order-hold discretisation: exp(a_i) multiplies the state and exp(a_i) - 1 scales
 * the input on the key path [RB, reply "Concern 8"].  Reading (the pages print neither formula): per head
 * h, a_i = log(lambda_i) = log sigmoid(x_i . w_h + b_h) for the layer input x_i, so lambda_i = exp(a_i);
 * the key scale is exp(a_i) - 1 = lambda_i - 1 = -sigmoid(-(x_i . w_h + b_h)), applied to the raw key
 * (the attention then takes the scaled key as its k).
 *   x: [B, L, Dm];  w: [H, Dm];  bias: [H]
 *   log_lambda: [B, H, L];  key_scale (nullable): [B, H, L];
 *   k, k_out (both or neither): [B, H, L, d], k_out = key_scale * k. */
int lion_oracle_selectivity_f64(const double *x, const double *w, const double *bias, int B, int L, int H, int Dm,
                                int d, const double *k, double *log_lambda, double *key_scale, double *k_out)
{
    long b;
    if (!x || !w || !bias || !log_lambda || B < 1 || L < 1 || H < 1 || Dm < 1 || (!k != !k_out) ||
        (k && d < 1))
        return ORACLE_EINVAL;
    for (b = 0; b < B; ++b) {
        int h, i, c;
        for (h = 0; h < H; ++h)
            for (i = 0; i < L; ++i) {
                const double *xi = x + ((size_t)b * L + i) * Dm;
                const size_t row = ((size_t)b * H + h) * L + i;
                double z = bias[h], ll, ks;
                for (c = 0; c < Dm; ++c)
                    z += xi[c] * w[(size_t)h * Dm + c];
                /* log sigmoid(z) = -log(1 + exp(-z)), written so that exp never overflows */
                ll = z >= 0.0 ? -log1p(exp(-z)) : z - log1p(exp(z));
                /* lambda - 1 = sigmoid(z) - 1 = -sigmoid(-z) */
                ks = -1.0 / (1.0 + exp(z));
                log_lambda[row] = ll;
                if (key_scale)
                    key_scale[row] = ks;
                if (k)
                    for (c = 0; c < d; ++c)
                        k_out[row * d + c] = ks * k[row * d + c];
            }
    }
    return ORACLE_OK;
}

/* ---- two token orders, averaged masks (patch-reordered LION-D / LION-S) -------------------------------
 * For images the pages average the masks of two patch orders instead of choosing one: M = (M_b + M_c) / 2
 * [RB, reply "P2: Comparison against vision SSMs", item 1, Figure 7 b and c; "LION-D natural / LION-S
 * natural" rows of the ImageNet table].  Reading (the figure is not on the pages): M_b is the mask of the
 * tokens' own order and M_c the same product-of-decays mask taken along a second order of the same
 * tokens, order[p] = the token at position p of it (for an image: the column-major raster of the patch
 * grid); each token keeps its own decay, so (M_c)_ij multiplies the decays of the tokens strictly after
 * min(pos(i), pos(j)) up to and including max(pos(i), pos(j)) in that order.
 *   order: [L], a permutation of 0 .. L-1 shared by every (batch, head); other arguments as
 *   lion_oracle_full_f64 (mask_kind LIT, D or S; no causal flag). */
int lion_oracle_full2_f64(const double *q, const double *k, const double *v, const double *log_lambda, int mask_kind,
                          double eps, const long *order, int B, int H, int L, int d, double *y, double *den,
                          double *absnum, double *absden)
{
    long bh, nbh = (long)B * H;
    int err = 0, t;
    char *seen;
    if (!q || !k || !v || !y || !order || B < 1 || H < 1 || L < 1 || d < 1 || !(eps >= 0.0) ||
        mask_kind < ORACLE_MASK_LIT || mask_kind > ORACLE_MASK_S || (mask_kind != ORACLE_MASK_LIT && !log_lambda))
        return ORACLE_EINVAL;
    seen = (char *)calloc((size_t)L, 1);
    if (!seen)
        return ORACLE_ENOMEM;
    for (t = 0; t < L; ++t) {
        if (order[t] < 0 || order[t] >= L || seen[order[t]])
            err = 1;
        else
            seen[order[t]] = 1;
    }
    free(seen);
    if (err)
        return ORACLE_EINVAL;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (bh = 0; bh < nbh; ++bh) {
        size_t base = (size_t)bh * L;
        double *phq = (double *)malloc(sizeof(double) * (size_t)L * d);
        double *phk = (double *)malloc(sizeof(double) * (size_t)L * d);
        double *lam = (double *)malloc(sizeof(double) * (size_t)L);
        double *lamc = (double *)malloc(sizeof(double) * (size_t)L);
        double *mb = (double *)malloc(sizeof(double) * (size_t)L);
        double *mc = (double *)malloc(sizeof(double) * (size_t)L);
        double *m = (double *)malloc(sizeof(double) * (size_t)L);
        long *pos = (long *)malloc(sizeof(long) * (size_t)L);
        double *num = (double *)malloc(sizeof(double) * (size_t)d);
        double *anum = (double *)malloc(sizeof(double) * (size_t)d);
        int i, j, p;   /* private to this (batch, head) */
        if (!phq || !phk || !lam || !lamc || !mb || !mc || !m || !pos || !num || !anum) {
            err |= 1;
        } else {
            for (j = 0; j < L; ++j) {
                const size_t tok = base + (size_t)j;
                phi_row(mask_kind, q + tok * d, d, phq + (size_t)j * d);
                phi_row(mask_kind, k + tok * d, d, phk + (size_t)j * d);
            }
            decays(mask_kind, log_lambda, H, L, bh, lam);
            /* the decays listed along the second order, and each token's position in it */
            for (p = 0; p < L; ++p) {
                lamc[p] = lam[order[p]];
                pos[order[p]] = p;
            }
            for (i = 0; i < L; ++i) {
                mask_row(lam, L, i, 0, mb);
                mask_row(lamc, L, (int)pos[i], 0, mc);   /* indexed by position in the second order */
                for (j = 0; j < L; ++j)
                    m[j] = 0.5 * (mb[j] + mc[pos[j]]);
                attn_row(phq + (size_t)i * d, phk, v + base * d, m, L, d, eps, num, anum, y + (base + i) * d,
                         den ? den + base + i : NULL, absnum ? absnum + (base + i) * d : NULL,
                         absden ? absden + base + i : NULL);
            }
        }
        free(phq);
        free(phk);
        free(lam);
        free(lamc);
        free(mb);
        free(mc);
        free(m);
        free(pos);
        free(num);
        free(anum);
    }
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}
