/*
 * fp64 CPU oracle for the spectral hot path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this file's library.  The product path never does.  Nothing here is
 * shared with the HIP library: no header, no helper, no table.
 *
 * Plain, slow, obviously correct eigenvalue routines in double precision,
 * written from the textbook definitions (G. H. Golub and C. F. Van Loan,
 * "Matrix Computations", 4th ed., ch. 8; B. N. Parlett, "The Symmetric
 * Eigenvalue Problem", ch. 9 and 7):
 *
 *   oracle_jacobi_eigvalsh   cyclic-by-row Jacobi (eigenvalues only)
 *   oracle_jacobi_batched    the same over a batch (OpenMP over matrices)
 *   oracle_householder_tridiag  Householder reduction to tridiagonal form
 *   oracle_tridiag_count_below  Sturm count #{lambda < x} of a tridiagonal
 *   oracle_tridiag_eigvals   all eigenvalues by bisection on the Sturm count
 *   oracle_ldlt_count_below  #{lambda < x} of a dense symmetric matrix from the
 *                            signs of the pivots of LDL^T(A - xI) (Sylvester)
 *
 * The pages ("Random matrix theory spectral methods", section 3.2 code; the
 * Swift-SVD page, section 2) call a library eigvalsh on a covariance and then
 * flip it to descending order; every routine here returns eigenvalues in
 * descending order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- cyclic Jacobi ------------------------------------------------------ */

/* One Jacobi rotation J(p,q) chosen so that (J^T A J)_{pq} = 0 (Golub & Van
 * Loan, 2x2 symmetric Schur decomposition), applied to a full symmetric n x n
 * matrix stored row-major.  J has J_pp = J_qq = c, J_pq = s, J_qp = -s. */
static void jacobi_rotate(int64_t n, double *A, int64_t p, int64_t q)
{
    double apq = A[p * n + q];
    if (apq == 0.0) return;
    double app = A[p * n + p], aqq = A[q * n + q];
    double tau = (aqq - app) / (2.0 * apq);
    double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
    double c = 1.0 / sqrt(1.0 + t * t);
    double s = t * c;
    /* columns: A <- A J */
    for (int64_t r = 0; r < n; ++r) {
        double arp = A[r * n + p], arq = A[r * n + q];
        A[r * n + p] = c * arp - s * arq;
        A[r * n + q] = s * arp + c * arq;
    }
    /* rows: A <- J^T A */
    for (int64_t k = 0; k < n; ++k) {
        double apk = A[p * n + k], aqk = A[q * n + k];
        A[p * n + k] = c * apk - s * aqk;
        A[q * n + k] = s * apk + c * aqk;
    }
    A[p * n + q] = 0.0;
    A[q * n + p] = 0.0;
}

static int cmp_desc(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x < y) - (x > y);
}

/* Eigenvalues of the symmetric n x n matrix A (destroyed) by cyclic-by-row
 * Jacobi.  Stops when off(A) <= tol * ||A||_F, or after a sweep that changes
 * nothing, or after max_sweeps sweeps.  Returns the sweeps used (negative if
 * max_sweeps was reached without convergence).  w gets the diagonal sorted
 * descending. */
int oracle_jacobi_eigvalsh(int64_t n, double *A, double *w, double tol, int max_sweeps)
{
    double fro2 = 0.0;
    for (int64_t i = 0; i < n * n; ++i) fro2 += A[i] * A[i];
    int sweeps = 0, converged = 0;
    for (; sweeps < max_sweeps; ++sweeps) {
        double off2 = 0.0;
        for (int64_t p = 0; p < n; ++p)
            for (int64_t q = 0; q < n; ++q)
                if (p != q) off2 += A[p * n + q] * A[p * n + q];
        if (off2 <= tol * tol * fro2) { converged = 1; break; }
        for (int64_t p = 0; p < n - 1; ++p)
            for (int64_t q = p + 1; q < n; ++q)
                jacobi_rotate(n, A, p, q);
    }
    if (!converged) {
        double off2 = 0.0;
        for (int64_t p = 0; p < n; ++p)
            for (int64_t q = 0; q < n; ++q)
                if (p != q) off2 += A[p * n + q] * A[p * n + q];
        converged = off2 <= tol * tol * fro2;
    }
    for (int64_t i = 0; i < n; ++i) w[i] = A[i * n + i];
    qsort(w, (size_t)n, sizeof(double), cmp_desc);
    return converged ? sweeps : -sweeps - 1;
}

/* A: batch x n x n (read only), w: batch x n, sweeps: batch. */
void oracle_jacobi_batched(int64_t batch, int64_t n, const double *A, double *w,
                           int32_t *sweeps, double tol, int max_sweeps)
{
#pragma omp parallel
    {
        double *work = (double *)malloc((size_t)(n * n) * sizeof(double));
#pragma omp for schedule(dynamic, 16)
        for (int64_t b = 0; b < batch; ++b) {
            memcpy(work, A + b * n * n, (size_t)(n * n) * sizeof(double));
            sweeps[b] = oracle_jacobi_eigvalsh(n, work, w + b * n, tol, max_sweeps);
        }
        free(work);
    }
}

/* ---- Householder tridiagonalisation ------------------------------------ */

/* Householder vector (Golub & Van Loan, "house"): for x of length m returns v
 * with v[0] = 1 and beta so that (I - beta v v^T) x = mu e_1, mu = ||x||.
 * Returns mu. */
static double house(int64_t m, const double *x, double *v, double *beta)
{
    double sigma = 0.0;
    for (int64_t i = 1; i < m; ++i) sigma += x[i] * x[i];
    v[0] = 1.0;
    for (int64_t i = 1; i < m; ++i) v[i] = x[i];
    if (sigma == 0.0) {
        if (x[0] >= 0.0) { *beta = 0.0; return x[0]; }
        *beta = 2.0; return -x[0];
    }
    double mu = sqrt(x[0] * x[0] + sigma);
    double v0 = (x[0] <= 0.0) ? x[0] - mu : -sigma / (x[0] + mu);
    *beta = 2.0 * v0 * v0 / (sigma + v0 * v0);
    for (int64_t i = 1; i < m; ++i) v[i] /= v0;
    return mu;
}

/* Reduce the full symmetric n x n row-major A (destroyed) to tridiagonal
 * T = Q^T A Q by n-2 Householder similarity transforms (Golub & Van Loan,
 * "Householder tridiagonalization").  d[0..n-1] = diag(T), e[0..n-2] = the
 * subdiagonal. */
void oracle_householder_tridiag(int64_t n, double *A, double *d, double *e)
{
    double *x = (double *)malloc((size_t)n * sizeof(double));
    double *v = (double *)malloc((size_t)n * sizeof(double));
    double *p = (double *)malloc((size_t)n * sizeof(double));
    for (int64_t k = 0; k + 2 < n; ++k) {
        int64_t m = n - k - 1, o = k + 1;
        for (int64_t i = 0; i < m; ++i) x[i] = A[(o + i) * n + k];
        double beta;
        double mu = house(m, x, v, &beta);
        d[k] = A[k * n + k];
        e[k] = mu;
        if (beta != 0.0) {
            /* p = beta * A22 v */
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < m; ++i) {
                const double *row = A + (o + i) * n + o;
                double acc = 0.0;
                for (int64_t j = 0; j < m; ++j) acc += row[j] * v[j];
                p[i] = beta * acc;
            }
            /* w = p - (beta p^T v / 2) v, stored in p */
            double pv = 0.0;
            for (int64_t i = 0; i < m; ++i) pv += p[i] * v[i];
            double h = 0.5 * beta * pv;
            for (int64_t i = 0; i < m; ++i) p[i] -= h * v[i];
            /* A22 <- A22 - v w^T - w v^T */
#pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < m; ++i) {
                double *row = A + (o + i) * n + o;
                double vi = v[i], wi = p[i];
                for (int64_t j = 0; j < m; ++j) row[j] -= vi * p[j] + wi * v[j];
            }
        }
    }
    if (n >= 2) {
        d[n - 2] = A[(n - 2) * n + (n - 2)];
        e[n - 2] = A[(n - 1) * n + (n - 2)];
    }
    if (n >= 1) d[n - 1] = A[(n - 1) * n + (n - 1)];
    free(x); free(v); free(p);
}

/* ---- Sturm counts and bisection ---------------------------------------- */

/* Number of eigenvalues of the symmetric tridiagonal T(d, e) strictly below x:
 * the number of negative pivots q_i of the LDL^T factorisation of T - xI,
 * q_0 = d_0 - x, q_i = d_i - x - e_{i-1}^2 / q_{i-1} (Sylvester's law of
 * inertia; Parlett ch. 7).  A zero pivot is replaced by -pivmin. */
int64_t oracle_tridiag_count_below(int64_t n, const double *d, const double *e, double x,
                                   double pivmin)
{
    int64_t cnt = 0;
    double q = 1.0;
    for (int64_t i = 0; i < n; ++i) {
        double off = (i == 0) ? 0.0 : e[i - 1] * e[i - 1] / q;
        q = d[i] - x - off;
        if (fabs(q) < pivmin) q = -pivmin;
        if (q < 0.0) ++cnt;
    }
    return cnt;
}

/* smallest pivot magnitude allowed in a Sturm count: a tiny multiple of
 * max(1, max e_i^2), so a zero pivot never divides */
static double tridiag_pivmin(int64_t n, const double *e)
{
    double m = 1.0;
    for (int64_t i = 0; i + 1 < n; ++i) if (e[i] * e[i] > m) m = e[i] * e[i];
    return m * 1e-300;
}

/* All eigenvalues of T(d, e) in descending order, each by bisection on the
 * Sturm count inside the Gershgorin interval until the bracket is as narrow
 * as fp64 allows. */
void oracle_tridiag_eigvals(int64_t n, const double *d, const double *e, double *w)
{
    double lo = INFINITY, hi = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
        double r = (i > 0 ? fabs(e[i - 1]) : 0.0) + (i + 1 < n ? fabs(e[i]) : 0.0);
        if (d[i] - r < lo) lo = d[i] - r;
        if (d[i] + r > hi) hi = d[i] + r;
    }
    double span = hi - lo;
    lo -= 1e-12 * span + 1e-300;
    hi += 1e-12 * span + 1e-300;
    double pivmin = tridiag_pivmin(n, e);
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t k = 0; k < n; ++k) {
        /* the (k+1)-th largest eigenvalue is the point where the count of
         * eigenvalues below x passes n - k - 1 */
        int64_t target = n - k - 1;
        double a = lo, b = hi;
        for (int it = 0; it < 4000; ++it) {
            double mid = 0.5 * (a + b);
            if (mid <= a || mid >= b) break;
            if (oracle_tridiag_count_below(n, d, e, mid, pivmin) <= target) a = mid;
            else b = mid;
        }
        w[k] = 0.5 * (a + b);
    }
}

/* #{lambda < x} for the dense symmetric n x n A (row-major, read only) from
 * the pivots of LDL^T(A - xI) without pivoting (Sylvester's law of inertia).
 * A zero pivot is replaced by a tiny negative number. */
int64_t oracle_ldlt_count_below(int64_t n, const double *A, double x)
{
    double *M = (double *)malloc((size_t)(n * n) * sizeof(double));
    memcpy(M, A, (size_t)(n * n) * sizeof(double));
    double scale = 0.0;
    for (int64_t i = 0; i < n; ++i) scale = fmax(scale, fabs(M[i * n + i] - x));
    double pivmin = (scale > 0.0 ? scale : 1.0) * 1e-300;
    for (int64_t i = 0; i < n; ++i) M[i * n + i] -= x;
    int64_t cnt = 0;
    for (int64_t k = 0; k < n; ++k) {
        double piv = M[k * n + k];
        if (fabs(piv) < pivmin) piv = -pivmin;
        if (piv < 0.0) ++cnt;
        /* Schur complement of the trailing block: M_ij -= M_ik M_kj / piv */
#pragma omp parallel for schedule(static)
        for (int64_t i = k + 1; i < n; ++i) {
            double l = M[i * n + k] / piv;
            if (l == 0.0) continue;
            double *ri = M + i * n;
            const double *rk = M + k * n;
            for (int64_t j = k + 1; j < n; ++j) ri[j] -= l * rk[j];
        }
    }
    free(M);
    return cnt;
}

/* Eigenvalues of a dense symmetric matrix (destroyed): Householder
 * tridiagonalisation followed by bisection.  w descending. */
void oracle_eigvalsh_dense(int64_t n, double *A, double *w)
{
    double *d = (double *)malloc((size_t)n * sizeof(double));
    double *e = (double *)malloc((size_t)(n > 1 ? n - 1 : 1) * sizeof(double));
    oracle_householder_tridiag(n, A, d, e);
    oracle_tridiag_eigvals(n, d, e, w);
    free(d); free(e);
}
