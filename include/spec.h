/*
 * spec.h -- C ABI of the MI355X (gfx950) spectral hot path:
 *   covariance / Gram aggregation  ->  symmetric eigenvalue spectrum  ->  spectral descriptors.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates or frees device memory, never synchronises the device, and only
 *     enqueues work on `stream` (a hipStream_t; NULL means the default stream).
 *   - Matrices are row-major.  `ld*` arguments are leading dimensions in elements.
 *   - Symmetric matrices: only the LOWER triangle (row >= column) is read or
 *     written; the strict upper triangle is never touched.
 *   - Eigenvalues are returned in DESCENDING order.
 *   - Every argument is validated on the host before anything is enqueued.  On an
 *     error the call returns a negative spec_status and enqueues nothing.  A
 *     failed kernel launch returns SPEC_EHIP.  Faults inside a kernel surface at
 *     the caller's next synchronisation.
 *   - Alignment: every device pointer must be aligned to its element size (2 bytes
 *     for bf16, 4 for f32 and int32, 8 for f64 and the descriptor records);
 *     workspaces must be 256-byte aligned; entry points that need more say so.
 *     A violation returns SPEC_EINVAL.  Where a pointer is 16-byte aligned and
 *     its leading dimension a multiple of 16 bytes, a faster kernel is chosen
 *     (spec_cov_accumulate); otherwise a general one computes the same result.
 *   - The library keeps no data between calls and is thread-safe; calls that
 *     share output or workspace buffers on different streams race, as any
 *     stream-ordered work does.  The large eigensolvers create, on first use,
 *     one helper stream and two events per caller stream and device (kept
 *     until the process ends, at most 64 such sets) to factor panels beside
 *     the trailing update.
 *
 * Page citations name the page title and its section:
 *   [RMT]   "Random matrix theory spectral methods: EigenTrack and RMT-KD"
 *           (large-model reliability monitoring and compression, lpnh.cn)
 *   [SWIFT] Swift-SVD news article (TeleAI et al., arXiv:2604.01609)
 *   [S3]    "S3 Spectral Null-Space Swap" blog post (xxqk.cn)
 */
#ifndef SPEC_H
#define SPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPEC_OK = 0,
    SPEC_EINVAL = -1,       /* bad pointer, size, stride, or parameter value */
    SPEC_EUNSUPPORTED = -2, /* valid request the library does not implement (dtype pair, size) */
    SPEC_EWORKSPACE = -3,   /* workspace NULL or smaller than the *_workspace query returned */
    SPEC_EHIP = -4          /* a HIP runtime call (launch) failed */
} spec_status;

typedef enum { SPEC_BF16 = 0, SPEC_F32 = 1, SPEC_F64 = 2 } spec_dtype;

/* Human-readable text of a status code (static storage, never NULL). */
const char *spec_strerror(int status);

/* Library version, e.g. "0.1.0". */
const char *spec_version(void);

/* ------------------------------------------------------------------------
 * A1  Covariance aggregation (symmetric rank-k update)
 *
 *   C <- beta * C + alpha * X^T X            (lower triangle of C only)
 *
 * X is n x d (rows are samples, no centring), C is d x d.  This is the
 * second-moment matrix S = (1/n) X^T X of [RMT] section 2.1 (alpha = 1/n), the
 * window covariance (1/N) H^T H of [RMT] section 3.1, and the incremental
 * aggregation of [SWIFT] sections 2 and 7: each new block of samples is added
 * to the running matrix (beta = 1) with no recomputation.
 *
 * Supported (xt, ct) pairs and their arithmetic:
 *   (SPEC_BF16, SPEC_F32)  bf16 products on MFMA, fp32 accumulation
 *   (SPEC_F32,  SPEC_F32)  fp32 products and accumulation
 *   (SPEC_F32,  SPEC_F64)  exact fp64 products of fp32 inputs, fp64 accumulation (MFMA)
 * beta == 0 ignores the previous contents of C (NaNs included).
 * n == 0 scales C by beta.  Requires d >= 1, ldx >= d, ldc >= d.
 * Errors: SPEC_EINVAL (NULL pointer, n < 0, d < 1, ld too small, misaligned),
 *         SPEC_EUNSUPPORTED (other dtype pairs).
 * ---------------------------------------------------------------------- */
int spec_cov_accumulate(void *stream, const void *X, int xt, int64_t n, int64_t d, int64_t ldx,
                        void *C, int ct, int64_t ldc, double alpha, double beta);

/* ------------------------------------------------------------------------
 * A2  Sliding-window Gram ([RMT] section 3.1: window H = [h_{t-N+1}..h_t]^T,
 *     covariance (1/N) H^T H; its nonzero spectrum is that of the N x N Gram
 *     (1/N) H H^T, so the N x N form is computed when N << d).
 *
 * H holds `streams` independent activation sequences of T steps of d values:
 * element (s, t, k) is at H[s*ld_s + t*ld_t + k].  ht must be SPEC_BF16 or
 * SPEC_F32; products are fp32-accumulated.
 *
 * layout SPEC_GRAM_BAND: out is f32 [streams][T][N] with
 *     out[s][t][j] = <h_t, h_{t-j}>      (0 <= j < N; 0 when t - j < 0; unscaled)
 *   All windows' Grams follow from it: G_w[i][j] = scale * out[s][w*stride + max(i,j)][|i-j|].
 *   `scale` and `stride` are ignored.
 * layout SPEC_GRAM_DENSE: out is f32 [streams * W][N][N], W = (T - N) / stride + 1,
 *     out[s*W + w] = scale * H_w H_w^T, H_w = rows [w*stride, w*stride + N) of stream s
 *   (both triangles written).
 * Requires 1 <= N <= 64, N <= T, stride >= 1, ld_t >= d, ld_s >= T*ld_t.
 * ---------------------------------------------------------------------- */
enum { SPEC_GRAM_BAND = 0, SPEC_GRAM_DENSE = 1 };

int spec_gram_window(void *stream, const void *H, int ht, int64_t streams, int64_t T, int64_t d,
                     int64_t ld_t, int64_t ld_s, int N, int stride, double scale, int layout,
                     float *out);

/* ------------------------------------------------------------------------
 * A3  Batched small symmetric eigenvalues (n <= 64), one 64-lane wave per
 *     matrix: Householder reduction to tridiagonal form with the matrix in
 *     registers, then bisection on Sturm counts (fp32).  The pages call a
 *     library eigvalsh per window and flip it to descending order ([RMT]
 *     section 3.2 code).  Every eigenvalue is within a small multiple of
 *     eps_f32 * ||A|| of the exact one.
 *
 * Source of the matrices (fp32):
 *   SPEC_SRC_DENSE: matrix b is a[b*stride_a + i*lda + j]; the lower triangle is read.
 *   SPEC_SRC_BAND:  the band Gram of spec_gram_window; matrix b is window
 *                   w = b % W of stream s = b / W (W = (T - n) / stride + 1):
 *                   A[i][j] = scale * a[s*T*n + (w*stride + max(i,j))*n + |i-j|];
 *                   batch must equal streams * W.
 * w:    f32 [batch][n], eigenvalues descending.
 * info: int32 [batch] (may be NULL): the number of bisection rounds (>= 0), or -1
 *       if the matrix has a non-finite entry (its eigenvalues are then NaN).
 * The method is direct (no sweep limit to choose).
 * ---------------------------------------------------------------------- */
enum { SPEC_SRC_DENSE = 0, SPEC_SRC_BAND = 1 };

typedef struct {
    int kind;            /* SPEC_SRC_DENSE or SPEC_SRC_BAND */
    const float *a;      /* device pointer */
    int64_t lda;         /* DENSE: row stride (>= n) */
    int64_t stride_a;    /* DENSE: elements between matrices (>= n*lda) */
    int64_t streams;     /* BAND: number of streams */
    int64_t T;           /* BAND: steps per stream */
    int stride;          /* BAND: window stride (>= 1) */
    float scale;         /* BAND: 1/N for the window covariance */
} spec_batch_src;

int spec_eigvalsh_batched(void *stream, const spec_batch_src *src, int64_t batch, int n, float *w,
                          int32_t *info);

/* ------------------------------------------------------------------------
 * Eigenvalues and eigenvectors of the same batches (n <= 32): the window
 * decomposition of "Random matrix theory spectral methods", section 3.1,
 * which yields the eigenvalues {lambda_i} and the eigenvectors of each
 * window covariance (of the N x N window Gram here; an eigenvector u of the
 * d x d covariance H^T H / N is H^T v / sqrt(N lambda) for the Gram's v).
 * Parallel cyclic Jacobi with the rotations accumulated into V, one wave per
 * matrix padded to 32 x 32, in fp32: a pair rotates while
 * |a_pq| > max(2e-6 sqrt(|a_pp a_qq|), 1e-7 max|a_ij|), at most 30 sweeps.
 *
 * src, batch: as spec_eigvalsh_batched.
 * w:    f32 [batch][n], eigenvalues descending.
 * V:    f32 [batch][n][n], V[b][i][j] = component i of the unit eigenvector of
 *       w[b][j] (sign arbitrary).
 * info: int32 [batch] (may be NULL): the number of sweeps (>= 1), -2 if the
 *       30 sweeps ended with a pair still above the threshold (outputs are
 *       written, less accurate), or -1 if the matrix has a non-finite entry
 *       (every output of that matrix is NaN).
 * Requires 1 <= n <= 32 (else SPEC_EINVAL, or SPEC_EUNSUPPORTED above 32),
 * V 4-byte aligned and the conditions of spec_eigvalsh_batched.
 * ---------------------------------------------------------------------- */
int spec_eigh_batched(void *stream, const spec_batch_src *src, int64_t batch, int n, float *w, float *V,
                      int32_t *info);

/* ------------------------------------------------------------------------
 * A4  Large symmetric eigenvalues (the single eigendecomposition of the
 *     aggregated covariance in [SWIFT] sections 2 and 7; the O(d^3) step [RMT]
 *     section 6.1 names as the cost for large d).
 *
 * Two-stage reduction: blocked Householder reduction of the dense matrix to
 * band form (bandwidth 32; tall panels by TSQR with Householder reconstruction;
 * trailing updates on MFMA), bulge chasing from band to tridiagonal in one
 * persistent kernel, then all eigenvalues of the tridiagonal by multisection
 * on Sturm counts in t's precision (from a shared 4096-point grid of counts for
 * n >= 2048).  t is SPEC_F32 or SPEC_F64; the reductions run in t.
 *
 * A: n x n, lower triangle read, DESTROYED (used as the working matrix).
 * w: n values of type t, descending.
 * ws: device workspace of at least spec_eigvalsh_large_workspace(n, t) bytes
 *     (256-byte aligned); its contents on entry are ignored.
 * info: int32 [1] device (may be NULL): 0 on success, 1 if the bulge-chasing
 *       pipeline hit its bounded wait (results invalid).
 * Calls sharing one workspace must be ordered on one stream.
 * Requires 1 <= n <= 32768 (SPEC_F32) or n <= 8192 (SPEC_F64), n <= lda < 2^22
 * (offsets inside a 128-row tile of A are 32-bit); otherwise SPEC_EINVAL.
 * ---------------------------------------------------------------------- */
int spec_eigvalsh_large_workspace(int64_t n, int t, size_t *bytes);

int spec_eigvalsh_large(void *stream, void *A, int t, int64_t n, int64_t lda, void *w, void *ws,
                        size_t ws_bytes, int32_t *info);

/* ------------------------------------------------------------------------
 * Eigenvalues and the eigenvectors of the k largest ("Random matrix theory
 * spectral methods" page, section 4.1: the projection basis P = [u_1 .. u_k]
 * of the eigenvectors beyond the MP edge; section 4.2's code keeps
 * k = int(keep_ratio d) of them).  The solve of spec_eigvalsh_large, keeping
 * the reduction: each stage-1 panel's Householder vectors (in A's strictly
 * lower part below the band) and block factor T, and every bulge reflector;
 * then, in fp64 on the tridiagonal T: its unreduced blocks (a block ends where
 * |e_i| <= eps ||T||, eps of type t), each block's eigenvalues by multisection,
 * their ranks among all blocks' values, and inverse iteration on the block (one
 * eigenvalue per thread; eigenvalues of one block closer than 1e-9 ||T|| are
 * done in order by one thread and orthogonalised against each other, at
 * O(c^2 m) for a cluster of c in a block of m rows); then the
 * back-transformation through the reflectors and the panels.
 *
 * A, t, n, lda, w, info: as spec_eigvalsh_large (A destroyed; w all n
 *       eigenvalues, descending).
 * Z:    n x k of type t, row-major with row stride ldz >= k: column j is the
 *       unit eigenvector of w[j] (sign arbitrary).
 * ws:   device workspace of spec_eigh_large_workspace(n, t, k) bytes (256-byte
 *       aligned): spec_eigvalsh_large's, then the reflectors (about n^2/64 x 33
 *       values), the panels' T, and 4 n k doubles of scratch.
 * Requires 1 <= k <= n <= 8192 (else SPEC_EINVAL, or SPEC_EUNSUPPORTED above
 * 8192), (n + 128) * ldz * sizeof(t) < 2^31 (Z is addressed with 32-bit byte
 * offsets; else SPEC_EUNSUPPORTED) and the conditions of spec_eigvalsh_large.
 * ---------------------------------------------------------------------- */
int spec_eigh_large_workspace(int64_t n, int t, int64_t k, size_t *bytes);

int spec_eigh_large(void *stream, void *A, int t, int64_t n, int64_t lda, void *w, void *Z, int64_t ldz, int64_t k,
                    void *ws, size_t ws_bytes, int32_t *info);

/* ------------------------------------------------------------------------
 * Leading eigenvalues by random projection ("Random matrix theory spectral
 * methods" page, section 3.2: top-k eigenvalues from a random projection in
 * O(k d^2) rather than O(d^3)): the randomised range finder with q steps of
 * subspace iteration and Rayleigh-Ritz,
 *     Y = A Omega, Q = orth(Y);  q times: Q = orth(A Q);  w = eig(Q^T A Q),
 * orth a Householder QR.  Returns all 32 Ritz values, descending; the leading
 * k < 32 approximate the k largest eigenvalues of A (the other columns are
 * oversampling).
 *
 * A:     [n][lda] f32 device, symmetric, LOWER triangle read; not modified.
 * Omega: [n][32] f32 device (row-major, contiguous): the caller's random test
 *        matrix (e.g. standard normal entries).
 * w:     f32 [32] device, Ritz values descending.
 * ws:    device workspace of spec_eigvalsh_large_workspace(n, SPEC_F32) bytes
 *        (256-byte aligned); calls sharing one workspace must be ordered on
 *        one stream.
 * Requires t == SPEC_F32 (else SPEC_EUNSUPPORTED), 64 <= n <= 32768,
 * n <= lda < 2^22, 0 <= q <= 16; else SPEC_EINVAL.
 * ---------------------------------------------------------------------- */
int spec_eigvalsh_topk(void *stream, const void *A, int t, int64_t n, int64_t lda, const void *Omega, int q, void *w,
                       void *ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * Ritz vectors of the random projection: the signal-subspace basis
 * ("Random matrix theory spectral methods" page, section 4.1: the
 * eigenvectors whose eigenvalues lie beyond the MP edge lambda_plus span the
 * signal subspace, P = [u_1 .. u_k]).  The same range finder as
 * spec_eigvalsh_topk, then the eigenvectors U of B = Q^T A Q (32 x 32, Jacobi
 * with round-robin pair ordering, 16 disjoint rotations per step, in one
 * workgroup) and P = Q U.  Column i of P is the Ritz vector of w[i]
 * (w descending); the columns are orthonormal to f32 rounding, each with an
 * arbitrary sign.  The caller keeps the leading columns whose Ritz value
 * exceeds its lambda_plus.
 *
 * A, Omega, t, n, lda, q, ws, ws_bytes: as for spec_eigvalsh_topk.
 * w:   f32 [32] device, Ritz values descending (the same values as
 *      spec_eigvalsh_topk up to the rounding of the small eigensolver).
 * P:   f32 [n][ldp] device, row-major; columns 0..31 of each row written,
 *      the rest untouched.  Must not overlap A, Omega, w or ws.
 * info: int32 [1] device (may be NULL): 0 when the Jacobi sweeps converged;
 *      1 when Q^T A Q has a NaN or Inf entry (non-finite A or Omega): every
 *      value of w and of P's 32 columns is then NaN; 2 when the sweep limit
 *      (30) was reached first (the values and vectors are the last iterate).
 *      Every slot of w and P is written in all three cases.
 * Requires 32 <= ldp < 2^22 and the conditions of spec_eigvalsh_topk;
 * else SPEC_EINVAL (SPEC_EUNSUPPORTED for t != SPEC_F32).
 * ---------------------------------------------------------------------- */
int spec_eigvecs_topk(void *stream, const void *A, int t, int64_t n, int64_t lda, const void *Omega, int q, void *w,
                      void *P, int64_t ldp, void *ws, size_t ws_bytes, int32_t *info);

/* ------------------------------------------------------------------------
 * Projection compression of a square weight ("Random matrix theory spectral
 * methods" page, section 4.1: with the signal-subspace basis P = [u_1 .. u_k]
 * in R^{d x k}, the d x d layer weight W is compressed to W' = P^T W P in
 * R^{k x k}).  Also returns, when X != NULL, the right factor X = W P, so that
 * X P^T is W kept on the span of P (a rank-k factorisation).
 * Products in f32 (MFMA) with f32 accumulation; bf16 weights widen exactly.
 *
 * W:  [d][ldw] device, type wt = SPEC_BF16 or SPEC_F32 (else
 *     SPEC_EUNSUPPORTED), row-major, 16-byte aligned, ldw a multiple of 8
 *     (bf16) or 4 (f32); not modified.
 * P:  [d][ldp] f32 device, row-major: the k basis columns (e.g. the leading
 *     columns of spec_eigvecs_topk's output).
 * Wp: [k][ldo] f32 device, row-major: W' (columns k.. of each row untouched).
 * X:  [d][ldx] f32 device or NULL: W P (columns k.. untouched).
 * ws: device workspace of spec_project_weight_workspace(d) bytes (256-byte
 *     aligned); calls sharing one workspace must be ordered on one stream.
 * Outputs must not overlap the inputs or ws.
 * Requires 1 <= k <= min(d, 32), d <= 65536, ldw >= d, ldp, ldo >= k and
 * ldx >= k when X is given; else SPEC_EINVAL.
 * ---------------------------------------------------------------------- */
int spec_project_weight_workspace(int64_t d, size_t *bytes);

int spec_project_weight(void *stream, const void *W, int wt, int64_t d, int64_t ldw, const void *P, int64_t ldp, int k,
                        void *Wp, int64_t ldo, void *X, int64_t ldx, void *ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * A5  Spectral descriptors of `batch` spectra of r values each
 *     (w[b*ldw + i], i < r, sorted DESCENDING; type wt = SPEC_F32 or SPEC_F64).
 *
 * Negative values (round-off) are clamped to 0 first.  With S = sum(lambda),
 * p_i = lambda_i / S, all in fp64:
 *   H      = -sum p_i ln p_i  (0 ln 0 = 0)      spectral entropy     [RMT] 2.3
 *   erank  = exp(H)                             effective rank       [SWIFT] 3
 *   m1     = lambda_1 / S                        leading mass         [RMT] 2.3
 *   gk     = lambda_k / lambda_{k+1}, g1 = lambda_1 / lambda_2   (eigengap ratio) [RMT] 2.3
 *   c = p_dim / n_samples; lambda_plus = sigma2 (1 + sqrt c)^2   (MP edge) [RMT] 2.1
 *   n_above = #{lambda_i > lambda_plus}                          (BBP outliers) [RMT] 2.2
 *   mp_w1  = (1/r) sum_i |mu_(i) - Q_MP((i - 1/2)/r)|, mu ascending: the
 *            Wasserstein-1 distance to the MP law ([RMT] 2.3); if p_dim <= n_samples,
 *            mu = lambda and the MP ratio is c; else mu = (n/p) lambda, ratio n/p.
 *   sigma_i = sqrt(lambda_i) (singular values when the matrix was W^T W):
 *   top_energy = sum_{i <= floor(top_frac r)} sigma_i^2 / sum sigma_i^2,
 *   top_sigma_share = the same ratio of sigma_i               [S3] 1
 *   tail_head = sigma at rank floor(tail_frac r) + 1, tail_min = sigma_r   [S3] 1
 *   n_small = #{sigma_i < small_rel * sigma_1}                [S3] 2
 * sigma2 by sigma2_mode: SPEC_SIGMA2_GIVEN (the value given), SPEC_SIGMA2_MEDIAN
 * (median of the r clamped values, [RMT] 4.2), SPEC_SIGMA2_MEAN (S / p_dim).
 * Undefined ratios (zero denominators) are NaN and set a flag bit.
 *
 * out: device array of `batch` spec_desc records.
 * ws:  device workspace of spec_descriptors_workspace(r) bytes (the MP quantile table).
 * Requires r >= 2, ldw >= r, 1 <= k < r, n_samples >= 1, p_dim >= 1, top_frac and
 * tail_frac in [0, 1], small_rel >= 0, sigma2 > 0 when sigma2_mode is GIVEN.
 * ---------------------------------------------------------------------- */
enum { SPEC_MODE_EIG = 0, SPEC_MODE_SINGULAR = 1 };
enum { SPEC_SIGMA2_GIVEN = 0, SPEC_SIGMA2_MEDIAN = 1, SPEC_SIGMA2_MEAN = 2 };
enum {
    SPEC_FLAG_NONFINITE = 1, /* a NaN or Inf eigenvalue was seen */
    SPEC_FLAG_GK_UNDEF = 2,  /* lambda_{k+1} <= 0 */
    SPEC_FLAG_S_ZERO = 4     /* all eigenvalues are <= 0 */
};

typedef struct {
    int mode;            /* SPEC_MODE_EIG or SPEC_MODE_SINGULAR (informational) */
    int sigma2_mode;     /* SPEC_SIGMA2_* */
    double sigma2;       /* used when sigma2_mode == SPEC_SIGMA2_GIVEN */
    int64_t n_samples;   /* n */
    int64_t p_dim;       /* p */
    int64_t k;           /* eigengap index (1-based) */
    double top_frac;     /* 0.2 */
    double small_rel;    /* 1e-2 */
    double tail_frac;    /* 0.7 */
} spec_desc_params;

typedef struct {
    double S, H, erank, m1, gk, g1, sigma2, lambda_plus, mp_w1;
    double top_energy, top_sigma_share, tail_head, tail_min, sigma1;
    int64_t n_above, n_small, r_pos, flags;
} spec_desc; /* 144 bytes */

int spec_descriptors_workspace(int64_t r, size_t *bytes);

int spec_descriptors(void *stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                     const spec_desc_params *p, spec_desc *out, void *ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * S3 tail-pair screen ("S3 Spectral Null-Space Swap" page, section 3.1: swap
 * candidates (u_i, v_j) come from the tail singular vectors, i, j >= 0.9 N, must
 * satisfy |u_i^T v_j| < 0.015, and i and j must lie in the same head's index
 * range).  Exact: the t x t inner products of the tail columns of U and V, in
 * fp64 (f32 inputs widened exactly), on MFMA.
 *
 * U, V:   [n][ldu], [n][ldv] device, type dt = SPEC_F32 or SPEC_F64 (else
 *         SPEC_EUNSUPPORTED), row-major with the singular vectors as columns
 *         (U's column i is u_i); columns i0 .. i0 + t - 1 are read.
 * absdot: f64 [t][ldo] device or NULL: |u_{i0+a}^T v_{i0+b}| at [a][b].
 * keep:   uint8 [t][ldk] device: 1 where (i0 + a) / head_dim == (i0 + b) / head_dim
 *         and the product is below eps (strict), else 0.
 * count:  int64 [1] device or NULL: the number of kept pairs.
 * Requires n >= 1, i0 >= 0, 1 <= t <= 65535, i0 + t <= ldu and ldv, head_dim >= 1,
 * 0 < eps finite, ldk >= t, ldo >= t when absdot is given; else SPEC_EINVAL.
 * ---------------------------------------------------------------------- */
int spec_tail_pair_screen(void *stream, const void *U, const void *V, int dt, int64_t n, int64_t ldu, int64_t ldv,
                          int64_t i0, int64_t t, int64_t head_dim, double eps, double *absdot, int64_t ldo,
                          uint8_t *keep, int64_t ldk, int64_t *count);

/* ------------------------------------------------------------------------
 * A3 + A5 fused: the eigenvalues of each small matrix and their descriptors in
 * one pass ([RMT] section 3.2: per window, the spectrum and then its
 * descriptors).  The same eigenvalues as spec_eigvalsh_batched and the same
 * records as spec_descriptors on them (wt = SPEC_F32, r = n, ldw = n), computed
 * while the spectrum is still in registers; each record's sums are taken in a
 * different order, so fields may differ from the two-call path in the last
 * bits.
 * src, batch, info: as spec_eigvalsh_batched; w may be NULL (spectra not kept).
 * p, out, ws, ws_bytes: as spec_descriptors with r = n (ws >= spec_descriptors_workspace(n)).
 * Requires 2 <= n <= 32 (else SPEC_EINVAL, or SPEC_EUNSUPPORTED above 32) and
 * the conditions of both calls.
 * ---------------------------------------------------------------------- */
int spec_eigvalsh_batched_desc(void *stream, const spec_batch_src *src, int64_t batch, int n, float *w, int32_t *info,
                               const spec_desc_params *p, spec_desc *out, void *ws, size_t ws_bytes);

/* ------------------------------------------------------------------------
 * Sliding-window spectra by incremental updates ("Random matrix theory
 * spectral methods" page, section 3.2: update the window decomposition as the
 * window moves instead of recomputing it).  The windows of spec_eigvalsh_batched
 * with a SPEC_SRC_BAND source, with the eigenvalues carried from window to
 * window: each step drops the oldest row of the window Gram (secular equation
 * of the principal submatrix) and appends the new one (arrowhead secular
 * equation), with the eigenvectors kept in fp64 and recomputed from the roots
 * (Gu-Eisenstat weights), so they stay orthogonal to working precision.
 * A chain restarts from an empty window every `restart` windows of a stream,
 * which bounds the accumulated round-off and sets the launch's parallelism
 * (streams * ceil(W / restart) chains).
 * src:     SPEC_SRC_BAND only (else SPEC_EINVAL); batch = streams * W.
 * restart: windows per chain, >= 1.
 * w:       f32 [batch][n], eigenvalues descending (fp64 arithmetic, rounded).
 * info:    int32 [batch] (may be NULL): the largest secular iteration count of
 *          the updates that led to the window, or -1 if the window holds a step
 *          whose band row has a non-finite value within the window (its
 *          eigenvalues are then NaN; the chain restarts after that step).
 * Requires 1 <= n <= 64 and the band conditions of spec_eigvalsh_batched.
 * ---------------------------------------------------------------------- */
int spec_eigvalsh_sliding(void *stream, const spec_batch_src *src, int64_t batch, int n, int restart, float *w,
                          int32_t *info);

/* ------------------------------------------------------------------------
 * spec_descriptors_static: spec_descriptors for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same records, computed by the same kernels, with
 * the MP quantile table held in the library's own device memory (one 256 KiB
 * table per GPU, kept until the process ends) instead of a caller workspace.
 * Allocates nothing.  Every call rewrites the table of its stream's GPU before
 * reading it; calls that overlap on one GPU (different streams, or threads)
 * race on it.
 * Requires r <= 32768 (else SPEC_EUNSUPPORTED) and the conditions of
 * spec_descriptors; SPEC_EHIP if the table's address cannot be obtained.
 * ---------------------------------------------------------------------- */
int spec_descriptors_static(void *stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                            const spec_desc_params *p, spec_desc *out);

/* ------------------------------------------------------------------------
 * Post-processing of descriptor series and spectra ("Random matrix theory
 * spectral methods" page, sections 3.2 and 4.2; section 2.3 for the KL form).
 *
 * spec_desc_smooth: exponential smoothing of descriptor time series.
 *   in, out: device spec_desc records [streams][W] (window index fastest;
 *   out must not overlap in).  Each of the 14 fp64 fields (S .. sigma1) is
 *   smoothed along W: y_0 = x_0, y_t = alpha x_t + (1 - alpha) y_{t-1}.  A
 *   non-finite x_t leaves the state unchanged and sets SPEC_FLAG_HELD in that
 *   record's flags; until the first finite value the output is NaN.  Counts
 *   (n_above, n_small, r_pos) are copied.
 *   Requires 0 < alpha <= 1, streams >= 0, W >= 1; else SPEC_EINVAL.
 *
 * spec_spectrum_robust: per spectrum (w[b*ldw + i], i < r, sorted DESCENDING,
 *   negative values clamped to 0; wt = SPEC_F32 or SPEC_F64), in fp64:
 *     median         the median of the r values
 *     sigma2_winsor  sum of the spectrum winsorised at q = floor(winsor_frac r)
 *                    values per end (q <= (r-1)/2), divided by p_dim: the
 *                    trace estimate of sigma^2 with extreme eigenvalues clipped
 *     mad            median |lambda - median|;  n_mad = #{|lambda - median| >
 *                    mad_k * 1.4826 * mad} (MAD outlier count)
 *     log_mean, log_std  mean and population standard deviation of ln lambda
 *                    over the positive values (log transform)
 *     sigma2         the sigma^2 of the MP reference: sigma2_mode GIVEN, MEDIAN,
 *                    MEAN (sum / p_dim) or WINSOR (sigma2_winsor)
 *     kl_mp          sum_b p_b ln(p_b / q_b) over `bins` equal-width bins of the
 *                    MP support [lambda_-, lambda_+] of that sigma^2 and ratio c
 *                    = p/n (if p_dim > n_samples: mu = (n/p) lambda and ratio n/p,
 *                    as for mp_w1); values outside the support count in the end
 *                    bins; p_b the fraction of values in bin b, q_b its MP mass
 *   flags: SPEC_FLAG_NONFINITE (a NaN or Inf value: median, sigma2_winsor, mad,
 *   kl_mp and a sigma2 not GIVEN are NaN; the log statistics use the finite
 *   values), SPEC_FLAG_S_ZERO (no finite positive value: log statistics NaN);
 *   kl_mp is NaN when sigma2 <= 0.
 *   out: device array of `batch` spec_robust records.
 *   Requires r >= 2, ldw >= r, 1 <= bins <= 64, 0 <= winsor_frac <= 0.5,
 *   mad_k > 0, n_samples, p_dim >= 1, sigma2_mode in 0..3 and sigma2 > 0 when
 *   it is GIVEN; else SPEC_EINVAL (SPEC_EUNSUPPORTED for other wt).
 * ---------------------------------------------------------------------- */
enum { SPEC_SIGMA2_WINSOR = 3 };
enum { SPEC_FLAG_HELD = 8 }; /* spec_desc_smooth: a non-finite field was held */

typedef struct {
    int32_t sigma2_mode; /* SPEC_SIGMA2_GIVEN, _MEDIAN, _MEAN, _WINSOR */
    int32_t bins;        /* histogram bins for kl_mp (1..64) */
    double sigma2;       /* used when sigma2_mode == SPEC_SIGMA2_GIVEN */
    int64_t n_samples;   /* n */
    int64_t p_dim;       /* p */
    double winsor_frac;  /* fraction clipped at each end, e.g. 0.05 */
    double mad_k;        /* outlier cut in robust standard deviations, e.g. 3 */
} spec_robust_params;

typedef struct {
    double median, sigma2_winsor, mad, log_mean, log_std, sigma2, kl_mp;
    int64_t n_mad, flags;
} spec_robust; /* 72 bytes */

int spec_desc_smooth(void *stream, const spec_desc *in, int64_t streams, int64_t W, double alpha, spec_desc *out);

int spec_spectrum_robust(void *stream, const void *w, int wt, int64_t batch, int64_t r, int64_t ldw,
                         const spec_robust_params *p, spec_robust *out);

/* ------------------------------------------------------------------------
 * Kernel timing for measurement tools (not part of the computation).
 *
 * spec_timing_enable(mask): from now on, every launch of a kernel whose bit
 *   (1 << SPEC_KT_*) is set in `mask` is bracketed by two HIP events recorded
 *   on the stream it is launched on; earlier records are discarded.  mask = 0
 *   stops recording.  The first non-zero call creates a pool of 16384 event
 *   pairs (host-side HIP objects; no device memory), kept until the process
 *   ends; launches beyond the pool are not timed.  Returns SPEC_EHIP if the
 *   events cannot be created.
 * spec_timing_read(kernel, &total_ms, &launches): waits for the recorded end
 *   events of that kernel (the one call here that blocks the host) and returns
 *   the summed device time in milliseconds and the number of timed launches;
 *   SPEC_EWORKSPACE when some launches were not timed for lack of events.
 * Not thread-safe with respect to concurrent measurement sessions.
 * ---------------------------------------------------------------------- */
enum {
    SPEC_KT_SYRK = 0,      /* spec_cov_accumulate's kernel */
    SPEC_KT_GRAM = 1,      /* spec_gram_window's kernel */
    SPEC_KT_SMALL_EIG = 2, /* spec_eigvalsh_batched's kernel */
    SPEC_KT_DESC = 3,      /* spec_descriptors' record kernel */
    SPEC_KT_SYMM = 4,      /* spec_eigvalsh_large, stage 1: A (V T) products */
    SPEC_KT_SYR2K = 5,     /* stage 1: rank-2k trailing updates */
    SPEC_KT_PANEL = 6,     /* stage 1: panel factorisations (TSQR, reconstruction, V/W, M/Z) */
    SPEC_KT_BULGE = 7,     /* stage 2: bulge chasing */
    SPEC_KT_TRIDIAG = 8,   /* stage 3: tridiagonal eigenvalues */
    SPEC_KT_COUNT = 9
};

int spec_timing_enable(unsigned kernels);

int spec_timing_read(int kernel, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_H */
