/*
 * sla_oracle.c -- plain, slow, sequential CPU oracle for the sparse CG solve and
 * its adjoint backward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The product path (the HIP library and
 * its Python binding) never calls it and shares no code with it.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC (see oracle/build.py).
 * Contraction is off so every product is rounded before it is added: the row
 * sums of the SpMV below are plain sequential fp64 sums in ascending entry order,
 * with no fused multiply-add.  Inner products are the exact sums rounded once (to
 * within a unit in the last place; see orc_dot), so that the reference does not
 * carry the rounding error of one particular summation order.
 *
 * Sources (torch-sla: Differentiable Sparse Linear Algebra with Adjoint Solvers
 * and Sparse Tensor Parallelism for PyTorch):
 *   - CG (Hestenes and Stiefel) as the pytorch-native iterative backend:
 *     paperpeel page, section 1 "Introduction" and section 3.1 "Five backends
 *     and auto-dispatch"; one SpMV and the inner products <r,r>, <p,Ap> per
 *     iteration: section 3.3 "Distributed Krylov solvers".
 *   - Linear adjoint: for A x = b the backward pass solves A^T lambda = dL/dx and
 *     the matrix gradient is -lambda_i x_j on the sparsity pattern only:
 *     gist.science Hindi and Japanese summaries, Methodology item 2
 *     ("Adjoint Differentiation Framework"), linear-systems bullet.
 *     dL/db = lambda follows from x = A^{-1} b (implicit function theorem,
 *     paperpeel section 3.2 "Adjoint Differentiation Framework").
 *   - BiCGStab (van der Vorst, 1992) for nonsymmetric systems, the pages' second
 *     iterative method (paperpeel section 1; section 3.1 "Five backends and
 *     auto-dispatch"), with the same adjoint on A^T.
 *   - Stopping tests, breakdown and iteration counting are not printed on the
 *     pages; the readings used here are listed with the parity tests.
 *
 * Parity pins (tests/test_oracle_pins.py, tests/test_oracle_bicgstab.py): dense LU
 * solves on small grids, the closed-form eigenpairs of the 5-point Laplacian,
 * manufactured solutions,
 * one-iteration convergence on an eigenvector, homogeneity invariants of the
 * gradients, central finite differences, scipy.sparse products and transposes,
 * and exact rational solutions of a 2 x 2 grid (tests/golden).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Per-system outcome codes; the HIP library uses the same numbers. */
enum { ORC_CONVERGED = 0, ORC_MAX_ITER = 1, ORC_NOT_SPD = 2, ORC_NAN = 3, ORC_BREAKDOWN = 4 };

/* y = A x, one row at a time; row i sums val[k] * x[col[k]] for k ascending. */
void orc_spmv(int64_t n_rows, const int64_t* row_ptr, const int32_t* col,
              const double* val, const double* x, double* y)
{
    for (int64_t i = 0; i < n_rows; ++i) {
        double s = 0.0;
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
            double t = val[k] * x[col[k]];
            s = s + t;
        }
        y[i] = s;
    }
}

/* y = A^T x by scattering each row: y[col[k]] += val[k] * x[i], rows ascending. */
void orc_spmv_transposed(int64_t n_rows, int64_t n_cols, const int64_t* row_ptr,
                         const int32_t* col, const double* val, const double* x, double* y)
{
    for (int64_t j = 0; j < n_cols; ++j) y[j] = 0.0;
    for (int64_t i = 0; i < n_rows; ++i) {
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
            double t = val[k] * x[i];
            y[col[k]] = y[col[k]] + t;
        }
    }
}

/*
 * Inner product <a, b> = sum_i a_i b_i, computed as the exact sum rounded once to
 * fp64, up to the last bit: the compensated dot product "Dot2" of Ogita, Rump and
 * Oishi (Accurate sum and dot product, SIAM J. Sci. Comput. 26(6), 2005), whose result
 * is as accurate as if it had been accumulated in twice the working precision and
 * then rounded.  Every product is split exactly into its rounded value h and the
 * remainder r (r by fma, which rounds a_i b_i - h once, and that is exact), every
 * running addition exactly into its rounded sum and remainder q (Knuth's two-sum),
 * and the remainders are added up beside the main sum.
 */
double orc_dot(int64_t n, const double* a, const double* b)
{
    double s = 0.0, c = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double h = a[i] * b[i];
        double r = fma(a[i], b[i], -h);          /* a_i b_i = h + r exactly */
        double t = s + h;
        double z = t - s;
        double q = (s - (t - z)) + (h - z);      /* s + h = t + q exactly */
        s = t;
        c = c + (q + r);
    }
    return s + c;
}

/*
 * Conjugate gradients for A x = b with x0 = 0, no preconditioner.
 *
 *   r = b, p = r, rho = <r,r>, threshold = max(rtol * |b|, atol)
 *   repeat:  q = A p;  sigma = <p,q>;  alpha = rho / sigma
 *            x = x + alpha p;  r = r - alpha q;  rho' = <r,r>
 *            stop when |r| <= threshold (|r| from the recurrence, no extra SpMV)
 *            beta = rho' / rho;  p = r + beta p
 *
 * The iteration count is the number of products A p (b = 0 stops at 0).
 * sigma <= 0 stops with NOT_SPD, a NaN sigma with NAN; x is left as it was
 * before that iteration.  max_iter reached: MAX_ITER with the last x.  With
 * fixed != 0 the residual test is skipped and exactly max_iter iterations run
 * (unless a breakdown stops them first).
 *
 * work: 3 * n doubles (r, p, q).  hist (nullable, max_iter + 1 entries) receives
 * |r_k| for k = 0 .. iterations.
 */
int orc_cg(int64_t n, const int64_t* row_ptr, const int32_t* col, const double* val,
           const double* b, double* x, double rtol, double atol, int64_t max_iter,
           int fixed, double* work, int64_t* iters_out, double* res_out,
           double* rhs_out, double* hist)
{
    double* r = work;
    double* p = work + n;
    double* q = work + 2 * n;
    for (int64_t i = 0; i < n; ++i) { x[i] = 0.0; r[i] = b[i]; p[i] = b[i]; }
    double rho = orc_dot(n, r, r);
    double bnorm = sqrt(rho);
    double thr = rtol * bnorm;
    if (atol > thr) thr = atol;
    *rhs_out = bnorm;
    if (hist) hist[0] = bnorm;
    int64_t k = 0;
    int state = ORC_MAX_ITER;
    if (!fixed && sqrt(rho) <= thr) { state = ORC_CONVERGED; goto done; }
    while (k < max_iter) {
        orc_spmv(n, row_ptr, col, val, p, q);
        double sigma = orc_dot(n, p, q);
        if (!(sigma > 0.0)) { state = (sigma != sigma) ? ORC_NAN : ORC_NOT_SPD; goto done; }
        double alpha = rho / sigma;
        for (int64_t i = 0; i < n; ++i) {
            double t = alpha * p[i];
            x[i] = x[i] + t;
        }
        for (int64_t i = 0; i < n; ++i) {
            double t = alpha * q[i];
            r[i] = r[i] - t;
        }
        double rho1 = orc_dot(n, r, r);
        k = k + 1;
        if (hist) hist[k] = sqrt(rho1);
        if (!fixed && sqrt(rho1) <= thr) { rho = rho1; state = ORC_CONVERGED; goto done; }
        double beta = rho1 / rho;
        for (int64_t i = 0; i < n; ++i) {
            double t = beta * p[i];
            p[i] = r[i] + t;
        }
        rho = rho1;
    }
done:
    *iters_out = k;
    *res_out = sqrt(rho);
    return state;
}

/*
 * Jacobi-preconditioned conjugate gradients, M = diag(A), x0 = 0 (the pages'
 * pytorch-native backend: paperpeel page, section 4.1, Table 3, which runs CG with
 * a Jacobi preconditioner):
 *
 *   r = b, z = M^{-1} r, p = z, rho = <r,z>, threshold = max(rtol * |b|, atol)
 *   repeat:  q = A p;  sigma = <p,q>;  alpha = rho / sigma
 *            x = x + alpha p;  r = r - alpha q;  z = M^{-1} r;  rho' = <r,z>
 *            stop when |r| <= threshold (|r| = sqrt(<r,r>) of the recurrence
 *            residual, the same test as orc_cg)
 *            beta = rho' / rho;  p = z + beta p
 *
 * M^{-1} r is the solution of the diagonal system: z_i = r_i / a_ii (a division,
 * not a multiplication by a stored reciprocal).  a_ii is the stored entry (i, i);
 * a row without one has a_ii = 0.  If some a_ii is NaN the solve stops with NAN, if
 * some a_ii <= 0 (M is not positive definite) with NOT_SPD, both before any
 * iteration with x = 0.  Iteration count, budget, fixed mode and breakdowns as in
 * orc_cg.  work: 5 n doubles (r, z, p, q, diagonal).
 */
int orc_pcg_jacobi(int64_t n, const int64_t* row_ptr, const int32_t* col, const double* val,
                   const double* b, double* x, double rtol, double atol, int64_t max_iter,
                   int fixed, double* work, int64_t* iters_out, double* res_out,
                   double* rhs_out, double* hist)
{
    double* r = work;
    double* z = work + n;
    double* p = work + 2 * n;
    double* q = work + 3 * n;
    double* d = work + 4 * n;
    int bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        d[i] = 0.0;
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
            if (col[k] == i) d[i] = val[k];
        if (d[i] != d[i]) bad |= 2;
        else if (!(d[i] > 0.0)) bad |= 1;
    }
    for (int64_t i = 0; i < n; ++i) x[i] = 0.0;
    double rr = orc_dot(n, b, b);
    double bnorm = sqrt(rr);
    double thr = rtol * bnorm;
    if (atol > thr) thr = atol;
    *rhs_out = bnorm;
    if (hist) hist[0] = bnorm;
    int64_t k = 0;
    int state = ORC_MAX_ITER;
    double rho = 0.0;
    if (!fixed && bnorm <= thr) { state = ORC_CONVERGED; goto done; }
    if (bad) { state = (bad & 2) ? ORC_NAN : ORC_NOT_SPD; goto done; }
    for (int64_t i = 0; i < n; ++i) { r[i] = b[i]; z[i] = r[i] / d[i]; p[i] = z[i]; }
    rho = orc_dot(n, r, z);
    while (k < max_iter) {
        orc_spmv(n, row_ptr, col, val, p, q);
        double sigma = orc_dot(n, p, q);
        if (!(sigma > 0.0)) { state = (sigma != sigma) ? ORC_NAN : ORC_NOT_SPD; goto done; }
        double alpha = rho / sigma;
        for (int64_t i = 0; i < n; ++i) {
            double t = alpha * p[i];
            x[i] = x[i] + t;
        }
        for (int64_t i = 0; i < n; ++i) {
            double t = alpha * q[i];
            r[i] = r[i] - t;
            z[i] = r[i] / d[i];
        }
        rr = orc_dot(n, r, r);
        double rho1 = orc_dot(n, r, z);
        k = k + 1;
        if (hist) hist[k] = sqrt(rr);
        if (!fixed && sqrt(rr) <= thr) { state = ORC_CONVERGED; goto done; }
        double beta = rho1 / rho;
        for (int64_t i = 0; i < n; ++i) {
            double t = beta * p[i];
            p[i] = z[i] + t;
        }
        rho = rho1;
    }
done:
    *iters_out = k;
    *res_out = sqrt(rr);
    return state;
}

/*
 * BiCGStab (van der Vorst, Bi-CGSTAB: a fast and smoothly converging variant of Bi-CG
 * for the solution of nonsymmetric linear systems, SIAM J. Sci. Stat. Comput. 13(2),
 * 1992; cited by the paperpeel page, section 1, and listed there in section 3.1 as
 * the second iterative method of the scipy, eigen and pytorch-native backends) for
 * A x = b with x0 = 0, no preconditioner, shadow residual rh = r0 = b:
 *
 *   r = b, p = r, rho = <rh, r>, threshold = max(rtol * |b|, atol)
 *   iteration k = 0, 1, ...:
 *     stop when |r| <= threshold (recurrence residual), or at the budget
 *     k > 0:  rho' = <rh, r>;  beta = (rho' / rho) (alpha / omega);
 *             p = r + beta (p - omega v);  rho = rho'
 *     v = A p;  alpha = rho / <rh, v>
 *     s = r - alpha v
 *     t = A s;  omega = <t, s> / <t, t>
 *     if |s| <= threshold: x = x + alpha p, stop (converged half-way, k + 1)
 *     x = x + alpha p + omega s;  r = s - omega t
 *
 * The half-way test on s is the customary safeguard (Barrett et al., Templates for
 * the Solution of Linear Systems, 1994, section 2.3.8): without it an exactly
 * converged s gives t = 0 and omega = 0 / 0.  t = A s is formed before that test.
 * The iteration count is the number of products A p.  Breakdowns stop the solve with
 * x as it was before the failing iteration: <rh, v> = 0 or <t, t> = 0 (BREAKDOWN),
 * either of them or <t, s> NaN (NAN), and rho' = 0 or omega = 0 at the start of an
 * iteration (BREAKDOWN: beta would divide by zero).  The tests run in the order
 * written: residual, budget, then the breakdowns.  With fixed != 0 neither residual
 * test runs and exactly max_iter iterations are made unless a breakdown stops them.
 *
 * work: 5 n doubles (r, p, v, s, t).  hist (nullable, max_iter + 1 entries) receives
 * |r_k| for k = 0 .. iterations (|s| for a half-way stop).
 */
int orc_bicgstab(int64_t n, const int64_t* row_ptr, const int32_t* col, const double* val,
                 const double* b, double* x, double rtol, double atol, int64_t max_iter,
                 int fixed, double* work, int64_t* iters_out, double* res_out,
                 double* rhs_out, double* hist)
{
    double* r = work;
    double* p = work + n;
    double* v = work + 2 * n;
    double* s = work + 3 * n;
    double* t = work + 4 * n;
    const double* rh = b;
    for (int64_t i = 0; i < n; ++i) { x[i] = 0.0; r[i] = b[i]; p[i] = b[i]; v[i] = 0.0; }
    double rr = orc_dot(n, r, r);
    double bnorm = sqrt(rr);
    double thr = rtol * bnorm;
    if (atol > thr) thr = atol;
    *rhs_out = bnorm;
    double rho = orc_dot(n, rh, r);
    double alpha = 0.0, omega = 0.0, res = bnorm;
    int64_t k = 0;
    int state;
    for (;;) {
        res = sqrt(rr);
        if (hist) hist[k] = res;
        if (!fixed && res <= thr) { state = ORC_CONVERGED; break; }
        if (k >= max_iter) { state = ORC_MAX_ITER; break; }
        if (k > 0) {
            double rho1 = orc_dot(n, rh, r);
            if (rho1 == 0.0 || omega == 0.0) { state = ORC_BREAKDOWN; break; }
            double beta = (rho1 / rho) * (alpha / omega);
            for (int64_t i = 0; i < n; ++i) {
                double tv = omega * v[i];
                double d = p[i] - tv;
                double tb = beta * d;
                p[i] = r[i] + tb;
            }
            rho = rho1;
        }
        orc_spmv(n, row_ptr, col, val, p, v);
        double rv = orc_dot(n, rh, v);
        if (rv != rv) { state = ORC_NAN; break; }
        if (rv == 0.0) { state = ORC_BREAKDOWN; break; }
        alpha = rho / rv;
        for (int64_t i = 0; i < n; ++i) {
            double tv = alpha * v[i];
            s[i] = r[i] - tv;
        }
        double ss = orc_dot(n, s, s);
        orc_spmv(n, row_ptr, col, val, s, t);
        double ts = orc_dot(n, t, s);
        double tt = orc_dot(n, t, t);
        if (!fixed && sqrt(ss) <= thr) {
            for (int64_t i = 0; i < n; ++i) {
                double tp = alpha * p[i];
                x[i] = x[i] + tp;
            }
            k = k + 1;
            res = sqrt(ss);
            if (hist) hist[k] = res;
            state = ORC_CONVERGED;
            break;
        }
        if (tt != tt || ts != ts) { state = ORC_NAN; break; }
        if (tt == 0.0) { state = ORC_BREAKDOWN; break; }
        omega = ts / tt;
        for (int64_t i = 0; i < n; ++i) {
            double tp = alpha * p[i];
            double x1 = x[i] + tp;
            double ts_ = omega * s[i];
            x[i] = x1 + ts_;
            double tt_ = omega * t[i];
            r[i] = s[i] - tt_;
        }
        rr = orc_dot(n, r, r);
        k = k + 1;
    }
    *iters_out = k;
    *res_out = res;
    return state;
}

/*
 * Transpose of an n_rows x n_cols CSR pattern by a stable counting sort on the
 * column index.  Row j of A^T lists the entries of column j of A in ascending
 * row order; perm[kT] is the position in A of entry kT of A^T, so
 * valT[kT] = val[perm[kT]].  row_ptr_t has n_cols + 1 entries.
 */
void orc_transpose(int64_t n_rows, int64_t n_cols, const int64_t* row_ptr, const int32_t* col,
                   int64_t* row_ptr_t, int32_t* col_t, int64_t* perm)
{
    int64_t nnz = row_ptr[n_rows];
    for (int64_t j = 0; j <= n_cols; ++j) row_ptr_t[j] = 0;
    for (int64_t k = 0; k < nnz; ++k) row_ptr_t[col[k] + 1] += 1;
    for (int64_t j = 0; j < n_cols; ++j) row_ptr_t[j + 1] += row_ptr_t[j];
    int64_t* next = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_cols > 0 ? n_cols : 1));
    for (int64_t j = 0; j < n_cols; ++j) next[j] = row_ptr_t[j];
    for (int64_t i = 0; i < n_rows; ++i) {
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
            int64_t dst = next[col[k]]++;
            col_t[dst] = (int32_t)i;
            perm[dst] = k;
        }
    }
    free(next);
}

/* gvals[k] = sign * u[row(k)] * v[col(k)] for every stored entry k. */
void orc_pattern_outer(int64_t n_rows, const int64_t* row_ptr, const int32_t* col,
                       double sign, const double* u, const double* v, double* gvals)
{
    for (int64_t i = 0; i < n_rows; ++i) {
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
            double t = u[i] * v[col[k]];
            gvals[k] = sign * t;
        }
    }
}

/*
 * Adjoint backward pass of x = A^{-1} b for a loss L(x) with g = dL/dx:
 *   solve A^T lambda = g by the same method as the forward solve (x0 = 0, same
 *   rtol / atol / budget, threshold relative to |g|), then dL/db = lambda and
 *   dL/dA_ij = -lambda_i x_j on the stored entries only.
 * method: 0 CG, 1 Jacobi-preconditioned CG (A^T has the same diagonal), 2 BiCGStab.
 * symmetric != 0: A^T is A (same arrays).  Otherwise A^T is formed by
 * orc_transpose.  lam and gvals (nullable) are outputs; work: 5 n doubles.
 */
static int orc_solve_method(int method, int64_t n, const int64_t* row_ptr, const int32_t* col,
                            const double* val, const double* b, double* x, double rtol, double atol,
                            int64_t max_iter, int fixed, double* work, int64_t* iters_out,
                            double* res_out, double* rhs_out)
{
    if (method == 1)
        return orc_pcg_jacobi(n, row_ptr, col, val, b, x, rtol, atol, max_iter, fixed, work, iters_out,
                              res_out, rhs_out, NULL);
    if (method == 2)
        return orc_bicgstab(n, row_ptr, col, val, b, x, rtol, atol, max_iter, fixed, work, iters_out,
                            res_out, rhs_out, NULL);
    return orc_cg(n, row_ptr, col, val, b, x, rtol, atol, max_iter, fixed, work, iters_out, res_out,
                  rhs_out, NULL);
}

int orc_solve_backward(int64_t n, const int64_t* row_ptr, const int32_t* col, const double* val,
                       int symmetric, const double* x, const double* g, double rtol, double atol,
                       int64_t max_iter, int fixed, int method, double* lam, double* gvals, double* work,
                       int64_t* iters_out, double* res_out, double* rhs_out)
{
    int state;
    if (symmetric) {
        state = orc_solve_method(method, n, row_ptr, col, val, g, lam, rtol, atol, max_iter, fixed, work,
                                 iters_out, res_out, rhs_out);
    } else {
        int64_t nnz = row_ptr[n];
        int64_t* rpt = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n + 1));
        int32_t* ct = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
        int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nnz > 0 ? nnz : 1));
        double* vt = (double*)malloc(sizeof(double) * (size_t)(nnz > 0 ? nnz : 1));
        orc_transpose(n, n, row_ptr, col, rpt, ct, perm);
        for (int64_t k = 0; k < nnz; ++k) vt[k] = val[perm[k]];
        state = orc_solve_method(method, n, rpt, ct, vt, g, lam, rtol, atol, max_iter, fixed, work,
                                 iters_out, res_out, rhs_out);
        free(rpt); free(ct); free(perm); free(vt);
    }
    if (gvals) orc_pattern_outer(n, row_ptr, col, -1.0, lam, x, gvals);
    return state;
}

/*
 * Timing mode of the CPU baseline (not a parity reference; the parity functions
 * above stay sequential).  The same steps as orc_cg run for exactly `iters`
 * iterations (the fixed-budget mode), with the SpMV rows, the vector updates and the
 * inner products split into contiguous slices over OpenMP threads: each thread sums
 * its slice as orc_dot does and the slices' sums are added in thread order, so the
 * iterates differ from orc_cg's only by that order.  Then, when adjoint != 0, the
 * backward pass of a symmetric A for g = x: the same CG on g (lam), and
 * gvals[k] = -lam[row(k)] * x[col(k)].  work: 4 n doubles (r, p, q, the adjoint's
 * right-hand side).  Returns the number of threads used.
 */
#ifdef _OPENMP
#include <omp.h>
#endif

static double dot_threads(int64_t n, const double* a, const double* b, double* part, int nt)
{
#pragma omp parallel num_threads(nt)
    {
        int t = 0, m = 1;
#ifdef _OPENMP
        t = omp_get_thread_num();
        m = omp_get_num_threads();
#endif
        int64_t lo = n * t / m, hi = n * (t + 1) / m;
        part[t] = orc_dot(hi - lo, a + lo, b + lo);
        if (t == 0)
            for (int u = m; u < nt; ++u) part[u] = 0.0;
    }
    double s = 0.0;
    for (int t = 0; t < nt; ++t) s = s + part[t];
    return s;
}

static void cg_fixed_threads(int64_t n, const int64_t* row_ptr, const int32_t* col, const double* val,
                             const double* b, double* x, int64_t iters, double* work, double* part, int nt)
{
    double* r = work;
    double* p = work + n;
    double* q = work + 2 * n;
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t i = 0; i < n; ++i) { x[i] = 0.0; r[i] = b[i]; p[i] = b[i]; }
    double rho = dot_threads(n, r, r, part, nt);
    for (int64_t k = 0; k < iters; ++k) {
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            double s = 0.0;
            for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
                double t = val[e] * p[col[e]];
                s = s + t;
            }
            q[i] = s;
        }
        double sigma = dot_threads(n, p, q, part, nt);
        if (!(sigma > 0.0)) return;
        double alpha = rho / sigma;
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            double t = alpha * p[i];
            x[i] = x[i] + t;
            double u = alpha * q[i];
            r[i] = r[i] - u;
        }
        double rho1 = dot_threads(n, r, r, part, nt);
        double beta = rho1 / rho;
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            double t = beta * p[i];
            p[i] = r[i] + t;
        }
        rho = rho1;
    }
}

/* The same BiCGStab steps as orc_bicgstab (no stop test in fixed mode; the breakdown
   guards end the run early), split over nt OpenMP threads: rows of the products and
   of the vector updates, slices of the inner products.  Timing mode only. */
static void spmv_threads(int64_t n, const int64_t* row_ptr, const int32_t* col, const double* val, const double* in,
                         double* out, int nt)
{
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            double t = val[e] * in[col[e]];
            s = s + t;
        }
        out[i] = s;
    }
}

static void bicgstab_fixed_threads(int64_t n, const int64_t* row_ptr, const int32_t* col, const double* val,
                                   const double* b, double* x, int64_t iters, double* work, double* part, int nt)
{
    double* r = work;
    double* p = work + n;
    double* v = work + 2 * n;
    double* s = work + 3 * n;
    double* t = work + 4 * n;
    const double* rh = b;
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t i = 0; i < n; ++i) { x[i] = 0.0; r[i] = b[i]; p[i] = b[i]; v[i] = 0.0; }
    double rho = dot_threads(n, rh, r, part, nt);
    double alpha = 0.0, omega = 0.0;
    for (int64_t k = 0; k < iters; ++k) {
        if (k > 0) {
            double rho1 = dot_threads(n, rh, r, part, nt);
            if (rho1 == 0.0 || omega == 0.0) return;
            double beta = (rho1 / rho) * (alpha / omega);
#pragma omp parallel for num_threads(nt) schedule(static)
            for (int64_t i = 0; i < n; ++i) {
                double tv = omega * v[i];
                double d = p[i] - tv;
                double tb = beta * d;
                p[i] = r[i] + tb;
            }
            rho = rho1;
        }
        spmv_threads(n, row_ptr, col, val, p, v, nt);
        double rv = dot_threads(n, rh, v, part, nt);
        if (!(rv == rv) || rv == 0.0) return;
        alpha = rho / rv;
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            double tv = alpha * v[i];
            s[i] = r[i] - tv;
        }
        spmv_threads(n, row_ptr, col, val, s, t, nt);
        double ts = dot_threads(n, t, s, part, nt);
        double tt = dot_threads(n, t, t, part, nt);
        if (!(tt == tt) || !(ts == ts) || tt == 0.0) return;
        omega = ts / tt;
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            double tp = alpha * p[i];
            double x1 = x[i] + tp;
            double ts_ = omega * s[i];
            x[i] = x1 + ts_;
            double tt_ = omega * t[i];
            r[i] = s[i] - tt_;
        }
    }
}

/* The CPU baseline's BiCGStab timing mode: iters fixed iterations on A, then (adjoint)
   the same on A^T (row_ptr_t, col_t, val_t: the transposed pattern and values) with
   right-hand side x (L = 0.5 |x|^2), and the gradient -lam_i x_j on A's pattern.
   work holds 6 n doubles. */
int orc_bicgstab_timing(int64_t n, const int64_t* row_ptr, const int32_t* col, const double* val,
                        const double* b, double* x, int64_t iters, int adjoint, const int64_t* row_ptr_t,
                        const int32_t* col_t, const double* val_t, double* lam, double* gvals, double* work,
                        int threads)
{
    int nt = threads > 0 ? threads : 1;
    if (nt > 1024) nt = 1024;
    double part[1024];
    bicgstab_fixed_threads(n, row_ptr, col, val, b, x, iters, work, part, nt);
    if (adjoint) {
        double* g = work + 5 * n;
        memcpy(g, x, sizeof(double) * (size_t)n);
        bicgstab_fixed_threads(n, row_ptr_t, col_t, val_t, g, lam, iters, work, part, nt);
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int64_t i = 0; i < n; ++i)
            for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
                double tg = lam[i] * x[col[e]];
                gvals[e] = -1.0 * tg;
            }
    }
    return nt;
}

int orc_cg_timing(int64_t n, const int64_t* row_ptr, const int32_t* col, const double* val, const double* b,
                  double* x, int64_t iters, int adjoint, double* lam, double* gvals, double* work, int threads)
{
    int nt = threads > 0 ? threads : 1;
    if (nt > 1024) nt = 1024;
    double part[1024];
    cg_fixed_threads(n, row_ptr, col, val, b, x, iters, work, part, nt);
    if (adjoint) {
        double* g = work + 3 * n;
        memcpy(g, x, sizeof(double) * (size_t)n);
        cg_fixed_threads(n, row_ptr, col, val, g, lam, iters, work, part, nt);
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int64_t i = 0; i < n; ++i)
            for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
                double t = lam[i] * x[col[e]];
                gvals[e] = -1.0 * t;
            }
    }
    return nt;
}
