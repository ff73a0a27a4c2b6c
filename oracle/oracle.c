/*
 * oracle.c -- plain, slow, fp64 reference for the differentiable sparse solve.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no header, helper or table with the HIP
 * library.
 *
 * What it computes (torch-sla explainer pages on gist.science, "Technical
 * summary"):
 *   - Methodology section 1 ("unified backend") names CG and BiCGStab as the
 *     iterative solvers and Significance/limitations says the PyTorch-native
 *     backend uses a Jacobi preconditioner;
 *   - Methodology section 2 ("adjoint differentiation framework"), linear
 *     systems: the backward pass solves one adjoint system A^T lambda = dL/dx
 *     and the matrix gradient on the sparsity pattern is -lambda_i x_j.
 * Iteration steps are the textbook ones: preconditioned CG as in Saad,
 * "Iterative Methods for Sparse Linear Systems", Algorithm 9.1 (Jacobi M =
 * diag(A)); BiCGStab as in van der Vorst, SIAM J. Sci. Stat. Comput. 13 (1992).
 *
 * Conventions: all arithmetic is fp64, compiled without FMA contraction; dot
 * products are plain left-to-right sums; row_ptr is int64; col is int32.  The
 * optional OpenMP pragmas only split independent rows/elements across threads,
 * so every result is bitwise identical to the single-threaded run.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
    ORC_OK = 0,
    ORC_NOT_CONVERGED = 1,
    ORC_BREAKDOWN = 2,
    ORC_ERR_ARG = -1,
    ORC_ERR_PATTERN = -2,
    ORC_ERR_ZERO_DIAG = -3,
    ORC_ERR_NO_MEMORY = -4
};

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the OpenMP loops from now on (for a timed serial run). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* y_i = sum over stored k of row i: val[k] * x[col[k]] */
void orc_spmv(int64_t n, const int64_t *row_ptr, const int32_t *col,
              const double *val, const double *x, double *y)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
            s += val[k] * x[col[k]];
        y[i] = s;
    }
}

double orc_dot(int64_t n, const double *a, const double *b)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i)
        s += a[i] * b[i];
    return s;
}

/*
 * Pattern check: row_ptr[0] = 0, non-decreasing, row_ptr[n] = nnz; every
 * column in [0, n); columns strictly ascending in each row; the diagonal is
 * stored.  Writes diagpos[i] = position of (i, i) when diagpos != NULL.
 */
int orc_check_pattern(int64_t n, int64_t nnz, const int64_t *row_ptr,
                      const int32_t *col, int64_t *diagpos)
{
    if (n < 0 || nnz < 0)
        return ORC_ERR_ARG;
    if (row_ptr[0] != 0 || row_ptr[n] != nnz)
        return ORC_ERR_PATTERN;
    for (int64_t i = 0; i < n; ++i) {
        if (row_ptr[i + 1] < row_ptr[i])
            return ORC_ERR_PATTERN;
        int64_t dpos = -1;
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
            if (col[k] < 0 || col[k] >= n)
                return ORC_ERR_PATTERN;
            if (k > row_ptr[i] && col[k] <= col[k - 1])
                return ORC_ERR_PATTERN;
            if (col[k] == i)
                dpos = k;
        }
        if (dpos < 0)
            return ORC_ERR_PATTERN;
        if (diagpos)
            diagpos[i] = dpos;
    }
    return ORC_OK;
}

/*
 * Transpose of the pattern by a counting sort on columns.  Entries of a column
 * are taken in increasing row order, so each row of A^T is sorted.
 * Outputs: row_ptr_t[n+1], col_t[nnz] (= row of the source entry), perm[nnz]
 * (= source position: A^T value at kt is A's value at perm[kt]).
 */
int orc_transpose(int64_t n, int64_t nnz, const int64_t *row_ptr,
                  const int32_t *col, int64_t *row_ptr_t, int32_t *col_t,
                  int64_t *perm)
{
    int64_t *next = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    if (!next)
        return ORC_ERR_NO_MEMORY;
    for (int64_t j = 0; j <= n; ++j)
        row_ptr_t[j] = 0;
    for (int64_t k = 0; k < nnz; ++k)
        row_ptr_t[col[k] + 1] += 1;
    for (int64_t j = 0; j < n; ++j)
        row_ptr_t[j + 1] += row_ptr_t[j];
    for (int64_t j = 0; j < n; ++j)
        next[j] = row_ptr_t[j];
    for (int64_t i = 0; i < n; ++i) {
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
            int64_t dst = next[col[k]]++;
            col_t[dst] = (int32_t)i;
            perm[dst] = k;
        }
    }
    free(next);
    return ORC_OK;
}

static int inv_diag(int64_t n, const int64_t *row_ptr, const int32_t *col,
                    const double *val, double *dinv)
{
    for (int64_t i = 0; i < n; ++i) {
        double d = 0.0;
        int found = 0;
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
            if (col[k] == i) {
                d = val[k];
                found = 1;
            }
        if (!found)
            return ORC_ERR_PATTERN;
        if (d == 0.0)
            return ORC_ERR_ZERO_DIAG;
        dinv[i] = 1.0 / d;
    }
    return ORC_OK;
}

/*
 * Preconditioned conjugate gradients with M = diag(A) (precond = 1) or M = I
 * (precond = 0), started from x = 0.
 *
 *   r = b, z = M^-1 r, p = z, rho = r.z
 *   repeat: q = A p; alpha = rho / (p.q); x += alpha p; r -= alpha q;
 *           stop when ||r|| <= tol ||b||;
 *           z = M^-1 r; rho' = r.z; beta = rho'/rho; p = z + beta p
 *
 * p.q <= 0 means A is not positive definite along p: status BREAKDOWN.
 * The stopping test uses the recurrence residual.  b = 0 returns x = 0 with
 * zero iterations.  hist (optional, maxit+1 entries) receives ||r_k||/||b||.
 */
int orc_cg(int64_t n, const int64_t *row_ptr, const int32_t *col,
           const double *val, const double *b, double *x, double tol,
           int64_t maxit, int precond, int64_t *iters, double *relres,
           double *hist)
{
    int status = ORC_NOT_CONVERGED;
    int64_t it = 0;
    double *r = (double *)malloc(sizeof(double) * (size_t)n);
    double *z = (double *)malloc(sizeof(double) * (size_t)n);
    double *p = (double *)malloc(sizeof(double) * (size_t)n);
    double *q = (double *)malloc(sizeof(double) * (size_t)n);
    double *dinv = precond ? (double *)malloc(sizeof(double) * (size_t)n) : NULL;
    if (!r || !z || !p || !q || (precond && !dinv)) {
        status = ORC_ERR_NO_MEMORY;
        goto out;
    }
    if (precond) {
        int e = inv_diag(n, row_ptr, col, val, dinv);
        if (e != ORC_OK) {
            status = e;
            goto out;
        }
    }
    for (int64_t i = 0; i < n; ++i)
        x[i] = 0.0;
    double bnorm = sqrt(orc_dot(n, b, b));
    if (relres)
        *relres = 0.0;
    if (hist)
        hist[0] = bnorm > 0.0 ? 1.0 : 0.0;
    if (bnorm == 0.0) {
        status = ORC_OK;
        goto out;
    }
    memcpy(r, b, sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; ++i)
        z[i] = precond ? dinv[i] * r[i] : r[i];
    memcpy(p, z, sizeof(double) * (size_t)n);
    double rho = orc_dot(n, r, z);
    double rnorm = bnorm;
    for (it = 0; it < maxit; ++it) {
        orc_spmv(n, row_ptr, col, val, p, q);
        double pq = orc_dot(n, p, q);
        if (!(pq > 0.0)) {
            status = ORC_BREAKDOWN;
            break;
        }
        double alpha = rho / pq;
        int64_t i;
#pragma omp parallel for schedule(static)
        for (i = 0; i < n; ++i) {
            x[i] += alpha * p[i];
            r[i] -= alpha * q[i];
        }
        rnorm = sqrt(orc_dot(n, r, r));
        if (hist)
            hist[it + 1] = rnorm / bnorm;
        if (rnorm <= tol * bnorm) {
            status = ORC_OK;
            ++it;
            break;
        }
#pragma omp parallel for schedule(static)
        for (i = 0; i < n; ++i)
            z[i] = precond ? dinv[i] * r[i] : r[i];
        double rho_new = orc_dot(n, r, z);
        double beta = rho_new / rho;
#pragma omp parallel for schedule(static)
        for (i = 0; i < n; ++i)
            p[i] = z[i] + beta * p[i];
        rho = rho_new;
    }
    if (relres)
        *relres = rnorm / bnorm;
out:
    if (iters)
        *iters = it;
    free(r);
    free(z);
    free(p);
    free(q);
    free(dinv);
    return status;
}

/*
 * Unpreconditioned BiCGStab from x = 0 (van der Vorst 1992):
 *
 *   r = b, rhat = b, rho_prev = alpha = omega = 1, v = p = 0
 *   for k = 1..maxit:
 *     rho = rhat.r                      (0 or NaN: BREAKDOWN)
 *     beta = (rho/rho_prev)(alpha/omega); p = r + beta (p - omega v)
 *     v = A p; alpha = rho / (rhat.v)   (rhat.v = 0 or NaN: BREAKDOWN)
 *     s = r - alpha v
 *     if ||s|| <= tol ||b||: x += alpha p, stop (half step; spmv = 2k-1)
 *     t = A s; omega = (t.s)/(t.t)      (t.t or t.s = 0 or NaN: BREAKDOWN)
 *     x += alpha p + omega s; r = s - omega t; rho_prev = rho
 *     if ||r|| <= tol ||b||: stop (spmv = 2k)
 *
 * iters counts started iterations k; *spmv counts products with A.
 */
int orc_bicgstab(int64_t n, const int64_t *row_ptr, const int32_t *col,
                 const double *val, const double *b, double *x, double tol,
                 int64_t maxit, int64_t *iters, int64_t *spmv, double *relres,
                 double *hist)
{
    int status = ORC_NOT_CONVERGED;
    int64_t k = 0, nmv = 0;
    double *r = (double *)malloc(sizeof(double) * (size_t)n);
    double *rh = (double *)malloc(sizeof(double) * (size_t)n);
    double *p = (double *)calloc((size_t)n, sizeof(double));
    double *v = (double *)calloc((size_t)n, sizeof(double));
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double *t = (double *)malloc(sizeof(double) * (size_t)n);
    if (!r || !rh || !p || !v || !s || !t) {
        status = ORC_ERR_NO_MEMORY;
        goto out;
    }
    for (int64_t i = 0; i < n; ++i)
        x[i] = 0.0;
    double bnorm = sqrt(orc_dot(n, b, b));
    if (relres)
        *relres = 0.0;
    if (hist)
        hist[0] = bnorm > 0.0 ? 1.0 : 0.0;
    if (bnorm == 0.0) {
        status = ORC_OK;
        goto out;
    }
    memcpy(r, b, sizeof(double) * (size_t)n);
    memcpy(rh, b, sizeof(double) * (size_t)n);
    double rho_prev = 1.0, alpha = 1.0, omega = 1.0, rnorm = bnorm;
    for (k = 1; k <= maxit; ++k) {
        int64_t i;
        double rho = orc_dot(n, rh, r);
        if (!(fabs(rho) > 0.0)) {
            status = ORC_BREAKDOWN;
            --k;
            break;
        }
        double beta = (rho / rho_prev) * (alpha / omega);
#pragma omp parallel for schedule(static)
        for (i = 0; i < n; ++i)
            p[i] = r[i] + beta * (p[i] - omega * v[i]);
        orc_spmv(n, row_ptr, col, val, p, v);
        ++nmv;
        double rv = orc_dot(n, rh, v);
        if (!(fabs(rv) > 0.0)) {
            status = ORC_BREAKDOWN;
            --k;
            break;
        }
        alpha = rho / rv;
#pragma omp parallel for schedule(static)
        for (i = 0; i < n; ++i)
            s[i] = r[i] - alpha * v[i];
        double snorm = sqrt(orc_dot(n, s, s));
        if (snorm <= tol * bnorm) {
#pragma omp parallel for schedule(static)
            for (i = 0; i < n; ++i)
                x[i] += alpha * p[i];
            rnorm = snorm;
            if (hist)
                hist[k] = rnorm / bnorm;
            status = ORC_OK;
            break;
        }
        orc_spmv(n, row_ptr, col, val, s, t);
        ++nmv;
        double tt = orc_dot(n, t, t);
        double ts = orc_dot(n, t, s);
        if (!(fabs(tt) > 0.0) || !(fabs(ts) > 0.0)) {
            status = ORC_BREAKDOWN;
            --k;
            break;
        }
        omega = ts / tt;
#pragma omp parallel for schedule(static)
        for (i = 0; i < n; ++i) {
            x[i] += alpha * p[i] + omega * s[i];
            r[i] = s[i] - omega * t[i];
        }
        rho_prev = rho;
        rnorm = sqrt(orc_dot(n, r, r));
        if (hist)
            hist[k] = rnorm / bnorm;
        if (rnorm <= tol * bnorm) {
            status = ORC_OK;
            break;
        }
    }
    if (k > maxit)
        k = maxit;
    if (relres)
        *relres = rnorm / bnorm;
out:
    if (iters)
        *iters = k;
    if (spmv)
        *spmv = nmv;
    free(r);
    free(rh);
    free(p);
    free(v);
    free(s);
    free(t);
    return status;
}

/*
 * grad_val[k] = -lambda[row(k)] * x[col[k]] for every stored entry k, in CSR
 * order (the matrix gradient on the pattern, adjoint framework, linear case).
 */
void orc_grad_on_pattern(int64_t n, const int64_t *row_ptr, const int32_t *col,
                         const double *lam, const double *x, double *grad_val)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
            grad_val[k] = -(lam[i] * x[col[k]]);
}

/*
 * Vector-Jacobian product of the differentiable product y = A x (the
 * autograd-aware .matvec of the unified API, Methodology section 1): for an
 * upstream gradient gy = dL/dy,
 *   grad_x[j]   = sum over stored entries (i, j) of A_ij gy[i]   (A^T gy),
 *                 accumulated in increasing row i;
 *   grad_val[k] = gy[row(k)] * x[col(k)]                          (dL/dA_ij).
 * Either output may be NULL.
 */
void orc_matvec_vjp(int64_t n, const int64_t *row_ptr, const int32_t *col,
                    const double *val, const double *x, const double *gy,
                    double *grad_x, double *grad_val)
{
    int64_t i;
    if (grad_x) {
        for (i = 0; i < n; ++i)
            grad_x[i] = 0.0;
        for (i = 0; i < n; ++i)
            for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
                grad_x[col[k]] += val[k] * gy[i];
    }
    if (grad_val) {
#pragma omp parallel for schedule(static)
        for (i = 0; i < n; ++i)
            for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
                grad_val[k] = gy[i] * x[col[k]];
    }
}

/*
 * Adjoint of x = A^-1 b for a loss gradient g = dL/dx:
 *   solve A^T lambda = g (x0 = 0, same method/tol/maxit, tol relative to ||g||),
 *   grad_b = lambda, grad_val[k] = -lambda[row(k)] x[col(k)].
 * method 0 (CG) presumes a symmetric A and uses A itself; method 1
 * (BiCGStab) builds A^T with orc_transpose and gathers its values.
 */
int orc_adjoint(int64_t n, int64_t nnz, const int64_t *row_ptr,
                const int32_t *col, const double *val, const double *x,
                const double *g, int method, int precond, double tol,
                int64_t maxit, double *grad_b, double *grad_val,
                int64_t *iters, int64_t *spmv, double *relres)
{
    int status;
    if (method == 0) {
        status = orc_cg(n, row_ptr, col, val, g, grad_b, tol, maxit, precond,
                        iters, relres, NULL);
        if (spmv)
            *spmv = iters ? *iters : 0;
    } else {
        int64_t *rpt = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n + 1));
        int32_t *ct = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
        int64_t *perm = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nnz > 0 ? nnz : 1));
        double *vt = (double *)malloc(sizeof(double) * (size_t)(nnz > 0 ? nnz : 1));
        if (!rpt || !ct || !perm || !vt) {
            free(rpt);
            free(ct);
            free(perm);
            free(vt);
            return ORC_ERR_NO_MEMORY;
        }
        status = orc_transpose(n, nnz, row_ptr, col, rpt, ct, perm);
        if (status == ORC_OK) {
            for (int64_t k = 0; k < nnz; ++k)
                vt[k] = val[perm[k]];
            status = orc_bicgstab(n, rpt, ct, vt, g, grad_b, tol, maxit, iters,
                                  spmv, relres, NULL);
        }
        free(rpt);
        free(ct);
        free(perm);
        free(vt);
    }
    if (status < 0)
        return status;
    orc_grad_on_pattern(n, row_ptr, col, grad_b, x, grad_val);
    return status;
}
