/*
 * sinkhorn_oracle.c -- plain double-precision CPU oracle for entropic optimal
 * transport between point clouds under squared-Euclidean cost.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously-correct reference the
 * GPU library is checked against.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load it; the library itself never does, and the
 * two share no code (no headers, helpers, tables or constants).
 *
 * Sources, cited by page and section:
 *   [FS]  "FlashSinkhorn: IO-bewuste Entropische Optimale Transport op GPU"
 *         (gist.science technical summary, Dutch).
 *   [AP]  "From Theory to Throughput: CUDA-Optimized APML for Large-Batch 3D
 *         Learning" (newx.sg paper page).
 *
 * What is computed, per pair b of a batch (pairs are independent):
 *   C_ij = ||x_i - y_j||^2                                   [FS Probleemstelling,
 *                                                             Methodologie intro]
 *   f_i <- -eps * LSE_j[(g_j - C_ij)/eps + log b_j]          [FS Methodologie 1,
 *                                                             Propositie 1]
 *   g_j <- -eps * LSE_i[(f_i - C_ij)/eps + log a_i]          (mirror of the f-update;
 *                                                             the page names its bias
 *                                                             gamma but prints only f)
 *   LSE_k z_k = M + log sum_k exp(z_k - M),  M = max_k z_k   (stabilised log domain)
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - g starts at 0 and f is updated first; one "iteration" is one f-update
 *     followed by one g-update that already uses the new f; no early stop.
 *   - an eps schedule is a list of stages (eps_s, iters_s) run back to back,
 *     potentials carried over (warm start) from stage to stage.
 *   - the plan at the final eps is
 *       log P_ij = (f_i + g_j - C_ij)/eps + log a_i + log b_j.
 *   - transport cost = sum_ij P_ij C_ij (primal), computed with compensated
 *     summation; the dual <a,f> + <b,g> is reported beside it.
 *   - the sparse plan [AP Abstract, Innovation] keeps
 *       P_ij >= rel_thr * max_kl P_kl  (max over the pair), decided in the log
 *     domain, stored row-major (pair, row, col) without duplicates.
 *   - loss on the stored support: L_b = sum_S P_ij C_ij (no renormalisation);
 *     dL/dx_i = sum_{j:(i,j) in S} 2 P_ij (x_i - y_j)   (P held fixed).
 *   - a zero weight gives log 0 = -inf and drops that term from the other
 *     side's LSE.
 *
 * Attention form [FS Methodologie 1, Propositie 1]: with hat potentials
 *   fh = f - ||x||^2, gh = g - ||y||^2, Q = sqrt(2) X, K = sqrt(2) Y,
 *   delta = eps log b, gamma = eps log a:
 *     fh_i <- -eps * LSE_j[(Q_i . K_j + gh_j + delta_j)/eps]
 *     gh_j <- -eps * LSE_i[(Q_i . K_j + fh_i + gamma_i)/eps]
 *   It is the same recurrence written differently; it lives here only so that
 *   the two forms can be checked against each other.
 *
 * Layout: all arrays are double, row-major, batch-major: X[B][n][d],
 * Y[B][m][d], a[B][n], b[B][m], f[B][n], g[B][m].  No function allocates
 * anything the caller has to free.  Rows are spread over threads with OpenMP;
 * the arithmetic of each row is sequential and in the order written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Half-updates smaller than this many entries run on one thread (a parallel
 * region per tiny update costs more than the update). */
#define PARALLEL_MIN_WORK 65536L

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static double sq_dist(const double *x, const double *y, int d)
{
    double s = 0.0;
    for (int k = 0; k < d; ++k) {
        double t = x[k] - y[k];
        s += t * t;
    }
    return s;
}

static double dot(const double *x, const double *y, int d)
{
    double s = 0.0;
    for (int k = 0; k < d; ++k)
        s += x[k] * y[k];
    return s;
}

/* Stabilised log-sum-exp of z[0..len): max, then log of the shifted sum. */
static double log_sum_exp(const double *z, int len)
{
    double M = -INFINITY;
    for (int k = 0; k < len; ++k)
        if (z[k] > M)
            M = z[k];
    if (M == -INFINITY)
        return -INFINITY;
    double s = 0.0;
    for (int k = 0; k < len; ++k)
        s += exp(z[k] - M);
    return M + log(s);
}

/*
 * One half-update of the direct (cost) form, for the rows of P against the
 * points of Q [FS Methodologie 1]:
 *     out_r = -eps * LSE_j[(pot_j - ||p_r - q_j||^2)/eps + logw_j]
 * pot / logw belong to Q.  With P = X, Q = Y this is the f-update; with
 * P = Y, Q = X it is the g-update.  rows == NULL means every row 0..np-1,
 * otherwise the nrows listed rows (out has nrows entries in that order).
 */
void oracle_half_update(const double *P, int np, const double *Q, int nq, int d,
                        const double *pot, const double *logw, double eps,
                        const int *rows, int nrows, double *out)
{
    int count = rows ? nrows : np;
#pragma omp parallel if ((long)count * nq >= PARALLEL_MIN_WORK)
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)(nq > 0 ? nq : 1));
#pragma omp for schedule(static)
        for (int t = 0; t < count; ++t) {
            int r = rows ? rows[t] : t;
            const double *p = P + (size_t)r * d;
            for (int j = 0; j < nq; ++j)
                z[j] = (pot[j] - sq_dist(p, Q + (size_t)j * d, d)) / eps + logw[j];
            out[t] = -eps * log_sum_exp(z, nq);
        }
        free(z);
    }
}

/*
 * One half-update of the attention form [FS Methodologie 1, Propositie 1]:
 *     out_r = -eps * LSE_j[(sqrt2 p_r . sqrt2 q_j + hat_j + bias_j)/eps]
 * hat = hat potential of Q, bias = eps * log w of Q.
 */
static void half_update_attention(const double *P, int np, const double *Q, int nq, int d,
                                  const double *hat, const double *bias, double eps,
                                  double *out)
{
    const double r2 = sqrt(2.0);
#pragma omp parallel if ((long)np * nq >= PARALLEL_MIN_WORK)
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)(nq > 0 ? nq : 1));
        double *qrow = (double *)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
        double *krow = (double *)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
#pragma omp for schedule(static)
        for (int r = 0; r < np; ++r) {
            for (int k = 0; k < d; ++k)
                qrow[k] = r2 * P[(size_t)r * d + k];
            for (int j = 0; j < nq; ++j) {
                for (int k = 0; k < d; ++k)
                    krow[k] = r2 * Q[(size_t)j * d + k];
                z[j] = (dot(qrow, krow, d) + hat[j] + bias[j]) / eps;
            }
            out[r] = -eps * log_sum_exp(z, nq);
        }
        free(krow);
        free(qrow);
        free(z);
    }
}

static void log_weights(const double *w, int len, double *lw)
{
    for (int k = 0; k < len; ++k)
        lw[k] = log(w[k]); /* log 0 = -inf: the point drops out of the other LSE */
}

/*
 * Full solve.  eps[s], iters[s] for s < n_stages; iters counts full
 * iterations (f-update then g-update).  form 0 = direct, 1 = attention.
 * warm != 0: g (and f) hold starting potentials; otherwise g starts at 0.
 * Returns 0, or -1 on bad arguments.
 */
int oracle_potentials(const double *X, const double *Y, const double *a, const double *b,
                      int B, int n, int m, int d,
                      const double *eps, const int *iters, int n_stages,
                      int form, int warm, double *f, double *g)
{
    if (B < 0 || n < 1 || m < 1 || d < 1 || n_stages < 0)
        return -1;
    double *la = (double *)malloc(sizeof(double) * (size_t)n);
    double *lb = (double *)malloc(sizeof(double) * (size_t)m);
    double *nx = (double *)malloc(sizeof(double) * (size_t)n);
    double *ny = (double *)malloc(sizeof(double) * (size_t)m);
    double *fh = (double *)malloc(sizeof(double) * (size_t)n);
    double *gh = (double *)malloc(sizeof(double) * (size_t)m);
    double *ga = (double *)malloc(sizeof(double) * (size_t)n);
    double *de = (double *)malloc(sizeof(double) * (size_t)m);

    for (int p = 0; p < B; ++p) {
        const double *Xp = X + (size_t)p * n * d;
        const double *Yp = Y + (size_t)p * m * d;
        double *fp = f + (size_t)p * n;
        double *gp = g + (size_t)p * m;
        log_weights(a + (size_t)p * n, n, la);
        log_weights(b + (size_t)p * m, m, lb);
        if (!warm) {
            for (int j = 0; j < m; ++j)
                gp[j] = 0.0;
            for (int i = 0; i < n; ++i)
                fp[i] = 0.0;
        }
        if (form == 0) {
            for (int s = 0; s < n_stages; ++s)
                for (int it = 0; it < iters[s]; ++it) {
                    oracle_half_update(Xp, n, Yp, m, d, gp, lb, eps[s], NULL, 0, fp);
                    oracle_half_update(Yp, m, Xp, n, d, fp, la, eps[s], NULL, 0, gp);
                }
        } else {
            for (int i = 0; i < n; ++i) {
                nx[i] = dot(Xp + (size_t)i * d, Xp + (size_t)i * d, d);
                fh[i] = fp[i] - nx[i];
            }
            for (int j = 0; j < m; ++j) {
                ny[j] = dot(Yp + (size_t)j * d, Yp + (size_t)j * d, d);
                gh[j] = gp[j] - ny[j];
            }
            for (int s = 0; s < n_stages; ++s) {
                for (int i = 0; i < n; ++i)
                    ga[i] = eps[s] * la[i];
                for (int j = 0; j < m; ++j)
                    de[j] = eps[s] * lb[j];
                for (int it = 0; it < iters[s]; ++it) {
                    half_update_attention(Xp, n, Yp, m, d, gh, de, eps[s], fh);
                    half_update_attention(Yp, m, Xp, n, d, fh, ga, eps[s], gh);
                }
            }
            for (int i = 0; i < n; ++i)
                fp[i] = fh[i] + nx[i];
            for (int j = 0; j < m; ++j)
                gp[j] = gh[j] + ny[j];
        }
    }
    free(la); free(lb); free(nx); free(ny); free(fh); free(gh); free(ga); free(de);
    return 0;
}

/* Neumaier compensated accumulator. */
typedef struct { double s, c; } acc_t;
static void acc_add(acc_t *a, double v)
{
    double t = a->s + v;
    if (fabs(a->s) >= fabs(v))
        a->c += (a->s - t) + v;
    else
        a->c += (v - t) + a->s;
    a->s = t;
}
static double acc_get(const acc_t *a) { return a->s + a->c; }

/* log P_ij = (f_i + g_j - C_ij)/eps + log a_i + log b_j.  The two log weights
 * are added to each other first, so every rounding is symmetric in the two
 * sides and the plan of (Y, X) is exactly the transpose of the plan of (X, Y),
 * values included. */
static double log_plan(const double *x, const double *y, int d, double fi, double gj,
                       double lai, double lbj, double eps)
{
    return (fi + gj - sq_dist(x, y, d)) / eps + (lai + lbj);
}

/*
 * Statistics of the plan at eps, per pair (out has 5 values per pair):
 *   out[0] = sum_ij P_ij C_ij                  (transport cost, primal)
 *   out[1] = sum_i a_i f_i + sum_j b_j g_j      (dual value)
 *   out[2] = sum_i |sum_j P_ij - a_i|           (row-marginal L1 error)
 *   out[3] = sum_j |sum_i P_ij - b_j|           (column-marginal L1 error)
 *   out[4] = sum_ij P_ij log(P_ij / (a_i b_j))  (KL of P to a (x) b)
 * Row quantities are summed per row (compensated), then over rows in order;
 * column sums are a second pass over the plan, one column at a time.
 */
void oracle_plan_stats(const double *X, const double *Y, const double *a, const double *b,
                       const double *f, const double *g, double eps,
                       int B, int n, int m, int d, double *out)
{
    double *la = (double *)malloc(sizeof(double) * (size_t)n);
    double *lb = (double *)malloc(sizeof(double) * (size_t)m);
    double *row_cost = (double *)malloc(sizeof(double) * (size_t)n);
    double *row_kl = (double *)malloc(sizeof(double) * (size_t)n);
    double *row_mass = (double *)malloc(sizeof(double) * (size_t)n);
    double *col_mass = (double *)malloc(sizeof(double) * (size_t)m);
    for (int p = 0; p < B; ++p) {
        const double *Xp = X + (size_t)p * n * d, *Yp = Y + (size_t)p * m * d;
        const double *ap = a + (size_t)p * n, *bp = b + (size_t)p * m;
        const double *fp = f + (size_t)p * n, *gp = g + (size_t)p * m;
        log_weights(ap, n, la);
        log_weights(bp, m, lb);
#pragma omp parallel for schedule(static)
        for (int i = 0; i < n; ++i) {
            acc_t cost = {0, 0}, kl = {0, 0}, mass = {0, 0};
            for (int j = 0; j < m; ++j) {
                const double *x = Xp + (size_t)i * d, *y = Yp + (size_t)j * d;
                double lp = log_plan(x, y, d, fp[i], gp[j], la[i], lb[j], eps);
                double P = exp(lp);
                if (P > 0.0) {
                    acc_add(&cost, P * sq_dist(x, y, d));
                    acc_add(&kl, P * (lp - la[i] - lb[j]));
                }
                acc_add(&mass, P);
            }
            row_cost[i] = acc_get(&cost);
            row_kl[i] = acc_get(&kl);
            row_mass[i] = acc_get(&mass);
        }
#pragma omp parallel for schedule(static)
        for (int j = 0; j < m; ++j) {
            acc_t mass = {0, 0};
            for (int i = 0; i < n; ++i)
                acc_add(&mass, exp(log_plan(Xp + (size_t)i * d, Yp + (size_t)j * d, d, fp[i],
                                            gp[j], la[i], lb[j], eps)));
            col_mass[j] = acc_get(&mass);
        }
        acc_t cost = {0, 0}, dual = {0, 0}, row_err = {0, 0}, col_err = {0, 0}, kl = {0, 0};
        for (int i = 0; i < n; ++i) {
            acc_add(&cost, row_cost[i]);
            acc_add(&kl, row_kl[i]);
            acc_add(&row_err, fabs(row_mass[i] - ap[i]));
            if (ap[i] > 0.0)
                acc_add(&dual, ap[i] * fp[i]);
        }
        for (int j = 0; j < m; ++j) {
            acc_add(&col_err, fabs(col_mass[j] - bp[j]));
            if (bp[j] > 0.0)
                acc_add(&dual, bp[j] * gp[j]);
        }
        out[5 * p + 0] = acc_get(&cost);
        out[5 * p + 1] = acc_get(&dual);
        out[5 * p + 2] = acc_get(&row_err);
        out[5 * p + 3] = acc_get(&col_err);
        out[5 * p + 4] = acc_get(&kl);
    }
    free(la); free(lb); free(row_cost); free(row_kl); free(row_mass); free(col_mass);
}

/* Largest log P_ij of one pair and the number of entries at or above
 * that maximum + log rel_thr. */
static void pair_max_count(const double *Xp, const double *Yp, const double *la,
                           const double *lb, const double *fp, const double *gp, double eps,
                           double log_thr, int n, int m, int d, double *max_out,
                           int64_t *count_out)
{
    double M = -INFINITY;
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < m; ++j) {
            double lp = log_plan(Xp + (size_t)i * d, Yp + (size_t)j * d, d, fp[i], gp[j],
                                 la[i], lb[j], eps);
            if (lp > M)
                M = lp;
        }
    int64_t c = 0;
    if (M > -INFINITY)
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < m; ++j)
                if (log_plan(Xp + (size_t)i * d, Yp + (size_t)j * d, d, fp[i], gp[j], la[i],
                             lb[j], eps) >= M + log_thr)
                    ++c;
    *max_out = M;
    *count_out = c;
}

/*
 * Thresholded sparse plan in COO form [AP Abstract, Innovation]: per pair,
 * M = max_ij log P_ij and the stored set is {(i,j) : log P_ij >= M + log rel_thr},
 * enumerated row-major.  pair_offsets[B+1] is always written.  The entries are
 * written only when capacity >= total; the return value is the total number of
 * kept entries (the required capacity), or -1 on bad arguments.
 */
int64_t oracle_plan_coo(const double *X, const double *Y, const double *a, const double *b,
                        const double *f, const double *g, double eps, double rel_thr,
                        int B, int n, int m, int d, int64_t capacity,
                        int32_t *rows, int32_t *cols, double *vals, int64_t *pair_offsets)
{
    if (!(rel_thr > 0.0 && rel_thr <= 1.0) || !(eps > 0.0) || B < 0 || n < 1 || m < 1)
        return -1;
    double log_thr = log(rel_thr);
    double *maxes = (double *)malloc(sizeof(double) * (size_t)(B > 0 ? B : 1));
    int64_t *counts = (int64_t *)malloc(sizeof(int64_t) * (size_t)(B > 0 ? B : 1));
#pragma omp parallel
    {
        double *la = (double *)malloc(sizeof(double) * (size_t)n);
        double *lb = (double *)malloc(sizeof(double) * (size_t)m);
#pragma omp for schedule(dynamic, 1)
        for (int p = 0; p < B; ++p) {
            log_weights(a + (size_t)p * n, n, la);
            log_weights(b + (size_t)p * m, m, lb);
            pair_max_count(X + (size_t)p * n * d, Y + (size_t)p * m * d, la, lb,
                           f + (size_t)p * n, g + (size_t)p * m, eps, log_thr, n, m, d,
                           &maxes[p], &counts[p]);
        }
        free(la);
        free(lb);
    }
    pair_offsets[0] = 0;
    for (int p = 0; p < B; ++p)
        pair_offsets[p + 1] = pair_offsets[p] + counts[p];
    int64_t total = pair_offsets[B];
    if (total <= capacity) {
#pragma omp parallel
        {
            double *la = (double *)malloc(sizeof(double) * (size_t)n);
            double *lb = (double *)malloc(sizeof(double) * (size_t)m);
#pragma omp for schedule(dynamic, 1)
            for (int p = 0; p < B; ++p) {
                const double *Xp = X + (size_t)p * n * d, *Yp = Y + (size_t)p * m * d;
                const double *fp = f + (size_t)p * n, *gp = g + (size_t)p * m;
                log_weights(a + (size_t)p * n, n, la);
                log_weights(b + (size_t)p * m, m, lb);
                int64_t k = pair_offsets[p];
                if (maxes[p] > -INFINITY)
                    for (int i = 0; i < n; ++i)
                        for (int j = 0; j < m; ++j) {
                            double lp = log_plan(Xp + (size_t)i * d, Yp + (size_t)j * d, d,
                                                 fp[i], gp[j], la[i], lb[j], eps);
                            if (lp >= maxes[p] + log_thr) {
                                rows[k] = i;
                                cols[k] = j;
                                vals[k] = exp(lp);
                                ++k;
                            }
                        }
            }
            free(la);
            free(lb);
        }
    }
    free(maxes);
    free(counts);
    return total;
}

/*
 * Loss and gradient on the stored support (P held fixed):
 *   loss[p]    = sum_{k in pair p} vals_k * ||x_{rows_k} - y_{cols_k}||^2
 *   dX[p][i]   = sum_{k in pair p, rows_k = i} 2 vals_k (x_i - y_{cols_k})
 * Entries may come in any order.  Returns 0, or -1 on an index out of range.
 */
int oracle_loss_grad(const double *X, const double *Y, int B, int n, int m, int d,
                     const int32_t *rows, const int32_t *cols, const double *vals,
                     const int64_t *pair_offsets, double *loss, double *dX)
{
    for (size_t t = 0; t < (size_t)B * n * d; ++t)
        dX[t] = 0.0;
    for (int p = 0; p < B; ++p) {
        const double *Xp = X + (size_t)p * n * d, *Yp = Y + (size_t)p * m * d;
        double *dXp = dX + (size_t)p * n * d;
        acc_t L = {0, 0};
        for (int64_t k = pair_offsets[p]; k < pair_offsets[p + 1]; ++k) {
            int i = rows[k], j = cols[k];
            if (i < 0 || i >= n || j < 0 || j >= m)
                return -1;
            const double *x = Xp + (size_t)i * d, *y = Yp + (size_t)j * d;
            acc_add(&L, vals[k] * sq_dist(x, y, d));
            for (int c = 0; c < d; ++c)
                dXp[(size_t)i * d + c] += 2.0 * vals[k] * (x[c] - y[c]);
        }
        loss[p] = acc_get(&L);
    }
    return 0;
}

/*
 * Dense transport application at eps [FS Methodologie 3, "Toepassing van
 * Transportmatrix": the barycentric projection and the gradient are weighted
 * averages over the plan, streamed like the update].  For each selected row i
 * of the X side of pair p, with P from the given potentials:
 *   r_i  = sum_j P_ij                              (row mass)
 *   dX_i = sum_j 2 P_ij (x_i - y_j)                (gradient of <P,C> in x_i,
 *                                                   P held fixed)
 *   T_i  = sum_j P_ij y_j / r_i                    (barycentric projection;
 *                                                   0 where r_i = 0)
 * Every sum is compensated and runs over j in order.  sel lists flat row
 * indices p * n + i (NULL: all B * n rows in order); outputs are indexed by
 * position in that list: r[k], dX[k][d], T[k][d] (any of them may be NULL).
 * The Y side is the same call with the roles of (X, a, f) and (Y, b, g)
 * exchanged, since log P is symmetric in them.
 */
void oracle_dense_grad(const double *X, const double *Y, const double *a, const double *b,
                       const double *f, const double *g, double eps, int B, int n, int m, int d,
                       const int64_t *sel, int64_t nsel, double *r, double *dX, double *T)
{
    const int64_t count = sel ? nsel : (int64_t)B * n;
#pragma omp parallel
    {
        double *lb = (double *)malloc(sizeof(double) * (size_t)m);
        acc_t *G = (acc_t *)malloc(sizeof(acc_t) * (size_t)d);
        acc_t *V = (acc_t *)malloc(sizeof(acc_t) * (size_t)d);
        int cur = -1;
#pragma omp for schedule(dynamic, 16)
        for (int64_t k = 0; k < count; ++k) {
            const int64_t flat = sel ? sel[k] : k;
            const int p = (int)(flat / n), i = (int)(flat % n);
            if (p != cur) {
                log_weights(b + (size_t)p * m, m, lb);
                cur = p;
            }
            const double *x = X + ((size_t)p * n + i) * d;
            const double *Yp = Y + (size_t)p * m * d;
            const double ai = a[(size_t)p * n + i];
            const double lai = ai > 0.0 ? log(ai) : -INFINITY;
            const double fi = f[(size_t)p * n + i];
            acc_t mass = {0, 0};
            for (int c = 0; c < d; ++c) {
                G[c].s = G[c].c = 0.0;
                V[c].s = V[c].c = 0.0;
            }
            for (int j = 0; j < m; ++j) {
                const double *y = Yp + (size_t)j * d;
                const double P = exp(log_plan(x, y, d, fi, g[(size_t)p * m + j], lai, lb[j], eps));
                acc_add(&mass, P);
                for (int c = 0; c < d; ++c) {
                    acc_add(&G[c], 2.0 * P * (x[c] - y[c]));
                    acc_add(&V[c], P * y[c]);
                }
            }
            const double rm = acc_get(&mass);
            if (r)
                r[k] = rm;
            for (int c = 0; c < d; ++c) {
                if (dX)
                    dX[(size_t)k * d + c] = acc_get(&G[c]);
                if (T)
                    T[(size_t)k * d + c] = rm > 0.0 ? acc_get(&V[c]) / rm : 0.0;
            }
        }
        free(lb);
        free(G);
        free(V);
    }
}

/*
 * Cosine cost on normalised vectors [FS Betekenis en Claims: the approach
 * applies to the cosine distance after normalisation].  For unit vectors
 * 2 - 2 xh . yh = ||xh - yh||^2, so the squared-Euclidean routines above give
 * the cosine-cost problem on the normalised points.
 *   out_i = x_i / ||x_i||, norms_i = ||x_i||   (out_i = 0 for a zero vector)
 */
void oracle_normalize(const double *X, int64_t count, int d, double *out, double *norms)
{
    for (int64_t i = 0; i < count; ++i) {
        const double *x = X + (size_t)i * d;
        double s = 0.0;
        for (int k = 0; k < d; ++k)
            s += x[k] * x[k];
        const double r = sqrt(s);
        norms[i] = r;
        for (int k = 0; k < d; ++k)
            out[(size_t)i * d + k] = r > 0.0 ? x[k] / r : 0.0;
    }
}

/*
 * Chain rule through the normalisation: with G the gradient with respect to
 * the normalised point xh = x / ||x||,
 *   dX_i = (G_i - xh_i (xh_i . G_i)) / ||x_i||     (0 for a zero vector),
 * the Jacobian of x / ||x|| being (I - xh xh^T) / ||x||.
 */
void oracle_normalize_backward(const double *Xh, const double *norms, const double *G,
                               int64_t count, int d, double *dX)
{
    for (int64_t i = 0; i < count; ++i) {
        const double *xh = Xh + (size_t)i * d, *g = G + (size_t)i * d;
        double dot = 0.0;
        for (int k = 0; k < d; ++k)
            dot += xh[k] * g[k];
        for (int k = 0; k < d; ++k)
            dX[(size_t)i * d + k] = norms[i] > 0.0 ? (g[k] - xh[k] * dot) / norms[i] : 0.0;
    }
}

/*
 * Sinkhorn normalisation of a sparse plan on its stored support [AP Abstract,
 * Innovation: Sinkhorn normalisation run directly in COO form].  For each pair
 * p, with the entries k of the pair (any order, no duplicates) and
 * lv_k = log vals_k, scalings alpha (rows) and beta (columns) start at 0 and
 * each of `iters` rounds sets, in this order,
 *   alpha_i = log a_i - LSE_{k in row i} (lv_k + beta_{col k})
 *   beta_j  = log b_j - LSE_{k in col j} (lv_k + alpha_{row k})
 * (a row or column with no entries, or whose LSE is -inf, keeps scaling 0);
 * then vals_k <- exp(lv_k + alpha_{row k} + beta_{col k}).  Afterwards
 * err[2p] = sum_i |row sum_i - a_i| and err[2p+1] = sum_j |col sum_j - b_j|
 * over the rows and columns of the pair.  Returns 0, or -1 on an index out of
 * range.
 */
int oracle_coo_normalize(const int32_t *rows, const int32_t *cols, double *vals,
                         const int64_t *pair_offsets, const double *a, const double *b,
                         int B, int n, int m, int iters, double *err)
{
    double *al = (double *)malloc(sizeof(double) * (size_t)n);
    double *be = (double *)malloc(sizeof(double) * (size_t)m);
    double *mx_r = (double *)malloc(sizeof(double) * (size_t)n);
    double *sm_r = (double *)malloc(sizeof(double) * (size_t)n);
    double *mx_c = (double *)malloc(sizeof(double) * (size_t)m);
    double *sm_c = (double *)malloc(sizeof(double) * (size_t)m);
    int rc = 0;
    for (int p = 0; p < B && rc == 0; ++p) {
        const int64_t k0 = pair_offsets[p], k1 = pair_offsets[p + 1];
        const double *ap = a + (size_t)p * n, *bp = b + (size_t)p * m;
        for (int64_t k = k0; k < k1; ++k)
            if (rows[k] < 0 || rows[k] >= n || cols[k] < 0 || cols[k] >= m)
                rc = -1;
        if (rc)
            break;
        for (int i = 0; i < n; ++i)
            al[i] = 0.0;
        for (int j = 0; j < m; ++j)
            be[j] = 0.0;
        for (int it = 0; it < iters; ++it) {
            /* rows */
            for (int i = 0; i < n; ++i) {
                mx_r[i] = -INFINITY;
                sm_r[i] = 0.0;
            }
            for (int64_t k = k0; k < k1; ++k) {
                const double z = log(vals[k]) + be[cols[k]];
                if (z > mx_r[rows[k]])
                    mx_r[rows[k]] = z;
            }
            for (int64_t k = k0; k < k1; ++k)
                if (mx_r[rows[k]] > -INFINITY)
                    sm_r[rows[k]] += exp(log(vals[k]) + be[cols[k]] - mx_r[rows[k]]);
            for (int i = 0; i < n; ++i)
                al[i] = mx_r[i] > -INFINITY ? log(ap[i]) - (mx_r[i] + log(sm_r[i])) : 0.0;
            /* columns */
            for (int j = 0; j < m; ++j) {
                mx_c[j] = -INFINITY;
                sm_c[j] = 0.0;
            }
            for (int64_t k = k0; k < k1; ++k) {
                const double z = log(vals[k]) + al[rows[k]];
                if (z > mx_c[cols[k]])
                    mx_c[cols[k]] = z;
            }
            for (int64_t k = k0; k < k1; ++k)
                if (mx_c[cols[k]] > -INFINITY)
                    sm_c[cols[k]] += exp(log(vals[k]) + al[rows[k]] - mx_c[cols[k]]);
            for (int j = 0; j < m; ++j)
                be[j] = mx_c[j] > -INFINITY ? log(bp[j]) - (mx_c[j] + log(sm_c[j])) : 0.0;
        }
        for (int64_t k = k0; k < k1; ++k)
            vals[k] = exp(log(vals[k]) + al[rows[k]] + be[cols[k]]);
        if (err) {
            for (int i = 0; i < n; ++i)
                sm_r[i] = 0.0;
            for (int j = 0; j < m; ++j)
                sm_c[j] = 0.0;
            for (int64_t k = k0; k < k1; ++k) {
                sm_r[rows[k]] += vals[k];
                sm_c[cols[k]] += vals[k];
            }
            double er = 0.0, ec = 0.0;
            for (int i = 0; i < n; ++i)
                er += fabs(sm_r[i] - ap[i]);
            for (int j = 0; j < m; ++j)
                ec += fabs(sm_c[j] - bp[j]);
            err[2 * p] = er;
            err[2 * p + 1] = ec;
        }
    }
    free(al); free(be); free(mx_r); free(sm_r); free(mx_c); free(sm_c);
    return rc;
}

/*
 * Hessian-vector product of the entropic OT value in X [FS Methodologie 3,
 * Hessiaan-Vector Producten], at the plan of the given potentials (meant to be
 * converged):  HV = d/dt grad_X OT(X + t V) at t = 0, where
 *   grad_i = sum_j 2 P_ij (x_i - y_j)          (the envelope gradient)
 * and P moves with X through C and through the potentials, which keep the
 * plan's marginals.  Differentiating P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps):
 *   dP_ij = P_ij (df_i + dg_j - dC_ij) / eps,   dC_ij = 2 (x_i - y_j) . v_i,
 * and the marginals stay fixed, sum_j dP_ij = 0 and sum_i dP_ij = 0:
 *   ma_i df_i + (P dg)_i = r_i = sum_j P_ij dC_ij,
 *   (P^T df)_j + mb_j dg_j = c_j = sum_i P_ij dC_ij,
 * with ma, mb the plan's row and column sums.  Eliminating df gives
 *   (diag(mb) - P^T diag(1/ma) P) dg = c - P^T (r / ma),
 * singular only along the constant vector (df + t, dg - t leave dP unchanged);
 * here dg = 0 on the first column with plan mass fixes it and the rest is solved
 * by Cholesky.  A column without plan mass (zero weight: its row and column of
 * the system are 0) keeps dg = 0 and stays out of the solve; it enters nothing
 * else, as P is 0 on it.  Then
 *   HV_i = sum_j 2 dP_ij (x_i - y_j) + 2 ma_i v_i.
 * Dense in n x m: for the small cases the tests use.  Returns 0, or -1 when a
 * system is not positive definite.
 */
int oracle_hvp(const double *X, const double *Y, const double *a, const double *b,
               const double *f, const double *g, double eps, int B, int n, int m, int d,
               const double *V, double *HV)
{
    double *P = (double *)malloc(sizeof(double) * (size_t)n * m);
    double *dC = (double *)malloc(sizeof(double) * (size_t)n * m);
    double *S = (double *)malloc(sizeof(double) * (size_t)m * m);
    double *ma = (double *)malloc(sizeof(double) * (size_t)n);
    double *mb = (double *)malloc(sizeof(double) * (size_t)m);
    double *r = (double *)malloc(sizeof(double) * (size_t)n);
    double *c = (double *)malloc(sizeof(double) * (size_t)m);
    double *rhs = (double *)malloc(sizeof(double) * (size_t)m);
    double *dg = (double *)malloc(sizeof(double) * (size_t)m);
    double *df = (double *)malloc(sizeof(double) * (size_t)n);
    double *la = (double *)malloc(sizeof(double) * (size_t)n);
    double *lb = (double *)malloc(sizeof(double) * (size_t)m);
    int *idx = (int *)malloc(sizeof(int) * (size_t)m);
    int rc = 0;
    for (int p = 0; p < B && rc == 0; ++p) {
        const double *Xp = X + (size_t)p * n * d, *Yp = Y + (size_t)p * m * d;
        const double *Vp = V + (size_t)p * n * d;
        double *Hp = HV + (size_t)p * n * d;
        log_weights(a + (size_t)p * n, n, la);
        log_weights(b + (size_t)p * m, m, lb);
        for (int i = 0; i < n; ++i) {
            ma[i] = 0.0;
            r[i] = 0.0;
        }
        for (int j = 0; j < m; ++j) {
            mb[j] = 0.0;
            c[j] = 0.0;
        }
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < m; ++j) {
                const double *x = Xp + (size_t)i * d, *y = Yp + (size_t)j * d;
                const double pij = exp(log_plan(x, y, d, f[(size_t)p * n + i],
                                                g[(size_t)p * m + j], la[i], lb[j], eps));
                double dot = 0.0;
                for (int k = 0; k < d; ++k)
                    dot += (x[k] - y[k]) * Vp[(size_t)i * d + k];
                P[(size_t)i * m + j] = pij;
                dC[(size_t)i * m + j] = 2.0 * dot;
                ma[i] += pij;
                mb[j] += pij;
                r[i] += pij * 2.0 * dot;
                c[j] += pij * 2.0 * dot;
            }
        /* S = diag(mb) - P^T diag(1/ma) P,  rhs = c - P^T (r / ma) */
        for (int j = 0; j < m; ++j) {
            double s = c[j];
            for (int i = 0; i < n; ++i)
                if (ma[i] > 0.0)
                    s -= P[(size_t)i * m + j] * r[i] / ma[i];
            rhs[j] = s;
            for (int l = 0; l < m; ++l) {
                double t = (j == l) ? mb[j] : 0.0;
                for (int i = 0; i < n; ++i)
                    if (ma[i] > 0.0)
                        t -= P[(size_t)i * m + j] * P[(size_t)i * m + l] / ma[i];
                S[(size_t)j * m + l] = t;
            }
        }
        /* dg = 0 on the pinned column and on columns without mass; Cholesky of
           S over the other columns (idx) */
        int q = 0, pin = -1;
        for (int j = 0; j < m; ++j) {
            dg[j] = 0.0;
            if (mb[j] > 0.0) {
                if (pin < 0)
                    pin = j;
                else
                    idx[q++] = j;
            }
        }
        for (int j = 0; j < q && rc == 0; ++j) {
            const size_t rj = (size_t)idx[j] * m;
            for (int l = 0; l <= j; ++l) {
                const size_t rl = (size_t)idx[l] * m;
                double s = S[rj + idx[l]];
                for (int k = 0; k < l; ++k)
                    s -= S[rj + idx[k]] * S[rl + idx[k]];
                if (j == l) {
                    if (!(s > 0.0)) {
                        rc = -1;
                        break;
                    }
                    S[rj + idx[j]] = sqrt(s);
                } else {
                    S[rj + idx[l]] = s / S[rl + idx[l]];
                }
            }
        }
        if (rc)
            break;
        for (int j = 0; j < q; ++j) {   /* L y = rhs */
            const size_t rj = (size_t)idx[j] * m;
            double s = rhs[idx[j]];
            for (int k = 0; k < j; ++k)
                s -= S[rj + idx[k]] * dg[idx[k]];
            dg[idx[j]] = s / S[rj + idx[j]];
        }
        for (int j = q - 1; j >= 0; --j) {   /* L^T dg = y */
            double s = dg[idx[j]];
            for (int k = j + 1; k < q; ++k)
                s -= S[(size_t)idx[k] * m + idx[j]] * dg[idx[k]];
            dg[idx[j]] = s / S[(size_t)idx[j] * m + idx[j]];
        }
        for (int i = 0; i < n; ++i) {
            double s = r[i];
            for (int j = 0; j < m; ++j)
                s -= P[(size_t)i * m + j] * dg[j];
            df[i] = ma[i] > 0.0 ? s / ma[i] : 0.0;
        }
        for (int i = 0; i < n; ++i) {
            const double *x = Xp + (size_t)i * d;
            for (int k = 0; k < d; ++k)
                Hp[(size_t)i * d + k] = 2.0 * ma[i] * Vp[(size_t)i * d + k];
            for (int j = 0; j < m; ++j) {
                const double *y = Yp + (size_t)j * d;
                const double dp = P[(size_t)i * m + j] *
                                  (df[i] + dg[j] - dC[(size_t)i * m + j]) / eps;
                for (int k = 0; k < d; ++k)
                    Hp[(size_t)i * d + k] += 2.0 * dp * (x[k] - y[k]);
            }
        }
    }
    free(P); free(dC); free(S); free(ma); free(mb); free(r); free(c); free(rhs); free(dg);
    free(df); free(la); free(lb); free(idx);
    return rc;
}
