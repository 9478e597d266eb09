/*
 * oracle.c -- plain float64 CPU oracle of the stabilised log-domain Sinkhorn
 * iteration for entropic optimal transport with squared-Euclidean cost.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code with the HIP library: it never forms the
 * dot-product (attention) form of the update, never rounds operands, never
 * centres the clouds and never streams tiles.  It is the textbook iteration,
 * written out so that it can be checked against the pages by eye.
 *
 * Source of every formula: "FlashSinkhorn: IO-Aware Entropic Optimal
 * Transport on GPU" (gist.science explainer of arXiv 2602.03067), section
 * "Method", part 1 ("attention-form reformulation"): the stabilised update
 *     f_i <- -eps * LSE_j [ (g_j - C_ij)/eps + log b_j ]
 * for squared-Euclidean cost C_ij = |x_i - y_j|^2, and its mirror for g with
 * the log-weights of the other side.  Readings where the page is silent:
 *   - alternating (Gauss-Seidel) order: one iteration = f-update, then a
 *     g-update that already uses the new f; g starts at 0;
 *   - C has no 1/2 factor (the page's Q = sqrt2 X, K = sqrt2 Y gives
 *     Q K^T = 2 X Y^T, i.e. C = |x|^2 + |y|^2 - 2 x.y);
 *   - the plan is P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps), the only plan
 *     whose row sums equal a exactly after an f-update of this form;
 *   - annealed runs use eps_s = eps0 (eps_end/eps0)^(s/(S-1)), s = 0..S-1,
 *     with f and g carried from stage to stage;
 *   - the marginal residual is the L1 error of both marginals of P.
 * Section "Method", part 3 (differentiation): the barycentric projection and
 * the gradient are weighted averages under the plan.  The gradient here is
 * that of the dual objective
 *     D = <a,f> + <b,g> - eps sum_ij a_i b_j (exp((f_i + g_j - C_ij)/eps) - 1)
 * with respect to the points at fixed (f, g): d/dx_i = sum_j P_ij dC_ij/dx_i
 * = 2 sum_j P_ij (x_i - y_j), and symmetrically for y_j; each summed as its
 * definition reads, pair by pair.
 * Natural log/exp from libm, two-pass log-sum-exp (max, then sum), costs by
 * direct coordinate differences, OpenMP over the output index only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_VERSION 2

int oracle_version(void) { return ORACLE_VERSION; }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* C_ij = sum_t (x_t - y_t)^2, by direct differences. */
static double sq_dist(const double* x, const double* y, int32_t d) {
    double c = 0.0;
    for (int32_t t = 0; t < d; ++t) {
        const double u = x[t] - y[t];
        c += u * u;
    }
    return c;
}

/*
 * One soft-min over the other cloud:
 *   out = -eps * log sum_k w_k exp((pot_k - C(p, q_k))/eps)
 *       = -eps * LSE_k [ (pot_k - C(p, q_k))/eps + log w_k ].
 * Two passes over the k axis: the first stores z_k and finds their maximum,
 * the second sums exp(z_k - max).  `z` is caller scratch of length cnt.
 */
static double soft_min(const double* p, const double* q, const double* w,
                       const double* pot, int64_t cnt, int32_t d, double eps,
                       double* z) {
    double zmax = -INFINITY;
    for (int64_t k = 0; k < cnt; ++k) {
        const double c = sq_dist(p, q + k * (int64_t)d, d);
        z[k] = (pot[k] - c) / eps + log(w[k]);
        if (z[k] > zmax) zmax = z[k];
    }
    double s = 0.0;
    for (int64_t k = 0; k < cnt; ++k) s += exp(z[k] - zmax);
    return -eps * (zmax + log(s));
}

/*
 * Soft-min for a list of output indices `idx` (or all of 0..cnt_out-1 when
 * idx is NULL): out[r] = soft-min of point P[idx[r]] against cloud Q with
 * weights w and potential pot.  The f-update is (P,Q,w,pot) = (X,Y,b,g); the
 * g-update is (Y,X,a,f).
 */
static int soft_min_many(const double* P, const double* Q, const double* w,
                         const double* pot, int64_t cnt_out, int64_t cnt_in,
                         int32_t d, double eps, const int64_t* idx, double* out) {
    int err = 0;
#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)(cnt_in > 0 ? cnt_in : 1));
        if (!z) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < cnt_out; ++r) {
                const int64_t i = idx ? idx[r] : r;
                out[r] = soft_min(P + i * (int64_t)d, Q, w, pot, cnt_in, d, eps, z);
            }
            free(z);
        }
    }
    return err;
}

/* f_i <- -eps LSE_j[(g_j - C_ij)/eps + log b_j], all rows (f-update). */
int oracle_f_update(const double* X, const double* Y, const double* b,
                    const double* g, int64_t n, int64_t m, int32_t d, double eps,
                    double* f_out) {
    return soft_min_many(X, Y, b, g, n, m, d, eps, NULL, f_out);
}

/* g_j <- -eps LSE_i[(f_i - C_ij)/eps + log a_i], all columns (g-update). */
int oracle_g_update(const double* X, const double* Y, const double* a,
                    const double* f, int64_t n, int64_t m, int32_t d, double eps,
                    double* g_out) {
    return soft_min_many(Y, X, a, f, m, n, d, eps, NULL, g_out);
}

/* The f-update evaluated only at rows rows[0..nrows-1] (spot checks). */
int oracle_f_update_rows(const double* X, const double* Y, const double* b,
                         const double* g, int64_t m, int32_t d, double eps,
                         const int64_t* rows, int64_t nrows, double* out) {
    return soft_min_many(X, Y, b, g, nrows, m, d, eps, rows, out);
}

/* The g-update evaluated only at columns cols[0..ncols-1]. */
int oracle_g_update_cols(const double* X, const double* Y, const double* a,
                         const double* f, int64_t n, int32_t d, double eps,
                         const int64_t* cols, int64_t ncols, double* out) {
    return soft_min_many(Y, X, a, f, ncols, n, d, eps, cols, out);
}

/*
 * L1 marginal residual of the plan P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps):
 *   r = sum_i |sum_j P_ij - a_i| + sum_j |sum_i P_ij - b_j|,
 * both sums formed directly.  row_err/col_err (nullable) receive the two terms.
 */
double oracle_marginal_residual(const double* X, const double* Y, const double* a,
                                const double* b, const double* f, const double* g,
                                int64_t n, int64_t m, int32_t d, double eps,
                                double* row_err, double* col_err) {
    double rsum = 0.0, csum = 0.0;
#pragma omp parallel for schedule(static) reduction(+ : rsum)
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            const double c = sq_dist(X + i * (int64_t)d, Y + j * (int64_t)d, d);
            s += a[i] * b[j] * exp((f[i] + g[j] - c) / eps);
        }
        rsum += fabs(s - a[i]);
    }
#pragma omp parallel for schedule(static) reduction(+ : csum)
    for (int64_t j = 0; j < m; ++j) {
        double s = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            const double c = sq_dist(X + i * (int64_t)d, Y + j * (int64_t)d, d);
            s += a[i] * b[j] * exp((f[i] + g[j] - c) / eps);
        }
        csum += fabs(s - b[j]);
    }
    if (row_err) *row_err = rsum;
    if (col_err) *col_err = csum;
    return rsum + csum;
}

/* eps of stage s of an S-stage geometric schedule from eps0 to eps_end. */
double oracle_stage_eps(int32_t s, int32_t n_stages, double eps0, double eps_end) {
    if (n_stages <= 1) return eps_end;
    return eps0 * pow(eps_end / eps0, (double)s / (double)(n_stages - 1));
}

/*
 * The alternating solve.  g (length m) holds the starting g on entry (zeros
 * for a cold start) and the final g on exit; f (length n) receives the final
 * f.  Each stage runs iters_per_stage iterations (f-update, then g-update).
 * With tol > 0 the residual of the current (f, g) is evaluated after every
 * check_every-th iteration and the solve stops at the first one <= tol.
 * dual_log (nullable, length 2 * total iterations) receives <a,f> + <b,g>
 * after every half-step.  Returns 0, or nonzero on allocation failure.
 */
int oracle_sinkhorn(const double* X, const double* Y, const double* a, const double* b,
                    int64_t n, int64_t m, int32_t d, int32_t n_stages, double eps0,
                    double eps_end, int32_t iters_per_stage, double tol,
                    int32_t check_every, double* f, double* g, double* dual_log,
                    double* resid_out, int32_t* iters_done) {
    int32_t done = 0;
    double resid = -1.0;
    int stop = 0;
    if (check_every < 1) check_every = 1;
    for (int32_t s = 0; s < n_stages && !stop; ++s) {
        const double eps = oracle_stage_eps(s, n_stages, eps0, eps_end);
        for (int32_t it = 0; it < iters_per_stage; ++it) {
            if (oracle_f_update(X, Y, b, g, n, m, d, eps, f)) return 1;
            if (dual_log) {
                double D = 0.0;
                for (int64_t i = 0; i < n; ++i) D += a[i] * f[i];
                for (int64_t j = 0; j < m; ++j) D += b[j] * g[j];
                dual_log[2 * done] = D;
            }
            if (oracle_g_update(X, Y, a, f, n, m, d, eps, g)) return 1;
            if (dual_log) {
                double D = 0.0;
                for (int64_t i = 0; i < n; ++i) D += a[i] * f[i];
                for (int64_t j = 0; j < m; ++j) D += b[j] * g[j];
                dual_log[2 * done + 1] = D;
            }
            ++done;
            if (tol > 0.0 && done % check_every == 0) {
                resid = oracle_marginal_residual(X, Y, a, b, f, g, n, m, d, eps, NULL, NULL);
                if (resid <= tol) { stop = 1; break; }
            }
        }
    }
    if (iters_done) *iters_done = done;
    if (resid_out) *resid_out = resid;
    return 0;
}

/*
 * Transport application U_i = sum_j P_ij V_j (V is m x dv, U is n x dv), with
 * P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps).  divide_by_a != 0 returns the
 * barycentric projection U_i / a_i instead, formed as sum_j b_j exp(...) V_j.
 * rows (nullable) restricts the output to rows[0..nrows-1]; U then has nrows
 * rows.  Method section, part 3: projections and gradients as weighted
 * averages under the plan.
 */
int oracle_transport(const double* X, const double* Y, const double* a, const double* b,
                     const double* f, const double* g, const double* V, int64_t n,
                     int64_t m, int32_t d, int32_t dv, double eps, int32_t divide_by_a,
                     const int64_t* rows, int64_t nrows, double* U) {
    const int64_t cnt = rows ? nrows : n;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < cnt; ++r) {
        const int64_t i = rows ? rows[r] : r;
        double* u = U + r * (int64_t)dv;
        for (int32_t t = 0; t < dv; ++t) u[t] = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            const double c = sq_dist(X + i * (int64_t)d, Y + j * (int64_t)d, d);
            double p = b[j] * exp((f[i] + g[j] - c) / eps);
            if (!divide_by_a) p *= a[i];
            const double* v = V + j * (int64_t)dv;
            for (int32_t t = 0; t < dv; ++t) u[t] += p * v[t];
        }
    }
    return 0;
}

/* grad_x_i = 2 sum_j P_ij (x_i - y_j) (n x d) and grad_y_j = 2 sum_i P_ij
 * (y_j - x_i) (m x d), P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps); either
 * output may be NULL. */
int oracle_gradient(const double* X, const double* Y, const double* a, const double* b,
                    const double* f, const double* g, int64_t n, int64_t m, int32_t d,
                    double eps, double* gX, double* gY) {
    if (gX) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            double* gi = gX + i * (int64_t)d;
            const double* xi = X + i * (int64_t)d;
            for (int32_t t = 0; t < d; ++t) gi[t] = 0.0;
            for (int64_t j = 0; j < m; ++j) {
                const double* yj = Y + j * (int64_t)d;
                const double p = a[i] * b[j] * exp((f[i] + g[j] - sq_dist(xi, yj, d)) / eps);
                for (int32_t t = 0; t < d; ++t) gi[t] += 2.0 * p * (xi[t] - yj[t]);
            }
        }
    }
    if (gY) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < m; ++j) {
            double* gj = gY + j * (int64_t)d;
            const double* yj = Y + j * (int64_t)d;
            for (int32_t t = 0; t < d; ++t) gj[t] = 0.0;
            for (int64_t i = 0; i < n; ++i) {
                const double* xi = X + i * (int64_t)d;
                const double p = a[i] * b[j] * exp((f[i] + g[j] - sq_dist(xi, yj, d)) / eps);
                for (int32_t t = 0; t < d; ++t) gj[t] += 2.0 * p * (yj[t] - xi[t]);
            }
        }
    }
    return 0;
}

/* The dual objective D above, with its exponential term summed pair by pair. */
double oracle_dual_objective(const double* X, const double* Y, const double* a,
                             const double* b, const double* f, const double* g, int64_t n,
                             int64_t m, int32_t d, double eps) {
    double lin = 0.0, ex = 0.0;
    for (int64_t i = 0; i < n; ++i) lin += a[i] * f[i];
    for (int64_t j = 0; j < m; ++j) lin += b[j] * g[j];
#pragma omp parallel for schedule(static) reduction(+ : ex)
    for (int64_t i = 0; i < n; ++i) {
        for (int64_t j = 0; j < m; ++j) {
            const double c = sq_dist(X + i * (int64_t)d, Y + j * (int64_t)d, d);
            ex += a[i] * b[j] * (exp((f[i] + g[j] - c) / eps) - 1.0);
        }
    }
    return lin - eps * ex;
}
