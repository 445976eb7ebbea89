"""fp64 CPU oracle of the spectral hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
this package imports nothing from it: the two share only the seeded input
generators.

What it computes, each function citing the passage it follows:

* :func:`covariance`      C = alpha * X^T X with no centring ("Random matrix
  theory spectral methods" page, section 2.1: S = (1/n) X^T X; section 3.2 code:
  C = H^T H / N), accumulated chunk by chunk by plain matrix addition (Swift-SVD
  page, sections 2 and 7).
* :func:`window_gram`     G_w = (1/N) H_w H_w^T for each full sliding window of
  N steps (RMT page, section 3.1: the window H = [h_{t-N+1}..h_t]^T and its
  covariance (1/N) H^T H, whose nonzero spectrum equals that of G_w).
* :func:`band_gram`       <h_t, h_{t-j}> for 0 <= j < N, the only inner products
  the windows use.
* :func:`band_window_gram` the window Gram rebuilt from a band, scale *
  B[w*stride + max(i, j), |i - j|]: what the windows' eigensolvers (batched, or
  by incremental updates as RMT page, section 3.2 suggests) see as input.
* :func:`eigvalsh_small`  cyclic Jacobi (C, fp64), descending.
* :func:`eigvalsh_large`  Householder tridiagonalisation + Sturm bisection.
* :func:`eigh_vectors`    the k largest eigenpairs by LAPACK's symmetric solver
  (the eigenvectors' plain definition A u = lambda u, |u| = 1, up to sign), the
  projection basis of RMT page, section 4.1.
* :func:`mp_quantiles`    quantiles of the Marchenko-Pastur law (RMT page,
  section 2.1) by Gauss-Legendre quadrature of the density.
* :func:`descriptors`     spectral entropy, effective rank, leading mass,
  eigengap, MP edge and outlier count, W1 distance to MP (RMT page, section
  2.3), top-20 % energy share, tail level and small-sigma count (S3 page,
  sections 1 and 2).
* :func:`smooth_descriptors` exponential smoothing of descriptor time series
  (RMT page, section 3.2).
* :func:`robust_stats`    median and winsorised sigma^2 estimates, MAD outlier
  count (RMT page, section 4.2), log-eigenvalue mean and spread (section 3.2)
  and the KL form of the MP deviation over a histogram (section 2.3).
* :func:`topk_ritz`       leading eigenvalues by random projection (RMT page,
  section 3.2): range finder, subspace iteration, Rayleigh-Ritz;
  :func:`topk_ritz_vectors` also returns the Ritz vectors (the signal-subspace
  basis of RMT page, section 4.1).
* :func:`project_weight`  the compressed weight W' = P^T W P of a d x d weight
  on a d x k basis (RMT page, section 4.1) and the low-rank factor W P.
* :func:`tail_pair_screen` the S3 page's screen of swap candidates (section
  3.1): |u_i^T v_j| over the tail singular vectors, same-head pairs below eps.

All arithmetic is fp64.  bf16 inputs arrive as uint16 bit patterns and are
widened exactly.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (no fast-math, portable ISA)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, dp, ip = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)
        lib.oracle_jacobi_eigvalsh.argtypes = [i64, dp, dp, ctypes.c_double, ctypes.c_int]
        lib.oracle_jacobi_eigvalsh.restype = ctypes.c_int
        lib.oracle_jacobi_batched.argtypes = [i64, i64, dp, dp, ip, ctypes.c_double, ctypes.c_int]
        lib.oracle_jacobi_batched.restype = None
        lib.oracle_householder_tridiag.argtypes = [i64, dp, dp, dp]
        lib.oracle_householder_tridiag.restype = None
        lib.oracle_tridiag_count_below.argtypes = [i64, dp, dp, ctypes.c_double, ctypes.c_double]
        lib.oracle_tridiag_count_below.restype = i64
        lib.oracle_tridiag_eigvals.argtypes = [i64, dp, dp, dp]
        lib.oracle_tridiag_eigvals.restype = None
        lib.oracle_ldlt_count_below.argtypes = [i64, dp, ctypes.c_double]
        lib.oracle_ldlt_count_below.restype = i64
        lib.oracle_eigvalsh_dense.argtypes = [i64, dp, dp]
        lib.oracle_eigvalsh_dense.restype = None
        _lib = lib
    return _lib


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


# ---------------------------------------------------------------- inputs

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of an input given as f32 values or bf16 bit patterns."""
    if dtype == "bf16":
        b = np.ascontiguousarray(x, dtype=np.uint16)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------- aggregation

def covariance(X: np.ndarray, dtype: str, alpha: float = 1.0, C0: np.ndarray | None = None,
               beta: float = 0.0, row_block: int = 4096) -> np.ndarray:
    """C = beta * C0 + alpha * X^T X in fp64, rows of X are samples, no centring.

    The sum over rows is taken block by block, each block's X_b^T X_b added to
    the running matrix: the incremental aggregation of the Swift-SVD page
    (sections 2 and 7).  A matrix product serves as the step inside a block."""
    n, d = X.shape
    acc = np.zeros((d, d), dtype=np.float64)
    for r0 in range(0, n, row_block):
        xb = widen(X[r0:r0 + row_block], dtype)
        acc += xb.T @ xb
    C = alpha * acc
    if beta != 0.0 and C0 is not None:
        C = C + beta * np.asarray(C0, dtype=np.float64)
    return C


def band_gram(H: np.ndarray, dtype: str, N: int) -> np.ndarray:
    """B[s, t, j] = <h_t, h_{t-j}> for 0 <= j < N (0 where t - j < 0), fp64.

    H is [streams, T, d] (or [T, d])."""
    h = widen(H, dtype)
    if h.ndim == 2:
        h = h[None]
    S, T, d = h.shape
    B = np.zeros((S, T, N), dtype=np.float64)
    for j in range(min(N, T)):
        B[:, j:, j] = np.einsum("std,std->st", h[:, j:, :], h[:, :T - j, :])
    return B


def window_gram(H: np.ndarray, dtype: str, N: int, windows=None, stride: int = 1) -> np.ndarray:
    """Dense G_w = (1/N) H_w H_w^T for the full windows w (rows [w*stride, w*stride + N)).

    H is [T, d] for one stream; ``windows`` selects window indices (default all
    W = (T - N) // stride + 1 of them)."""
    h = widen(H, dtype)
    T = h.shape[0]
    W = (T - N) // stride + 1
    idx = range(W) if windows is None else windows
    out = []
    for w in idx:
        hw = h[w * stride: w * stride + N]
        out.append(hw @ hw.T / N)
    return np.array(out, dtype=np.float64)


def band_window_gram(B: np.ndarray, N: int, scale: float, stride: int = 1, windows=None) -> np.ndarray:
    """K_w[i, j] = scale * B[w*stride + max(i, j), |i - j|] for one stream's band
    B [T, N] (entry j of row t is <h_t, h_{t-j}>): the window Gram of window w
    written out from the band, fp64 ("Random matrix theory spectral methods"
    page, section 3.1; with scale = 1/N it is window_gram)."""
    B = np.asarray(B, dtype=np.float64)
    T = B.shape[0]
    W = (T - N) // stride + 1
    idx = range(W) if windows is None else windows
    i = np.arange(N)
    rows = np.maximum.outer(i, i)
    lags = np.abs(np.subtract.outer(i, i))
    return np.array([scale * B[w * stride + rows, lags] for w in idx], dtype=np.float64).reshape(-1, N, N)


# ---------------------------------------------------------------- spectra

def eigvalsh_small(A: np.ndarray, tol: float = 1e-15, max_sweeps: int = 100):
    """Eigenvalues (descending) of one n x n or a batch [b, n, n] of symmetric
    matrices by cyclic Jacobi; returns (w, sweeps)."""
    A = np.ascontiguousarray(A, dtype=np.float64)
    single = A.ndim == 2
    if single:
        A = A[None]
    b, n, _ = A.shape
    w = np.empty((b, n), dtype=np.float64)
    sw = np.empty(b, dtype=np.int32)
    _load().oracle_jacobi_batched(b, n, _dp(A), _dp(w),
                                  sw.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), tol, max_sweeps)
    return (w[0], sw[0]) if single else (w, sw)


def tridiagonalize(A: np.ndarray):
    """(d, e) of the Householder tridiagonal form of the symmetric matrix A."""
    M = np.array(A, dtype=np.float64, order="C", copy=True)
    n = M.shape[0]
    d = np.empty(n, dtype=np.float64)
    e = np.empty(max(n - 1, 1), dtype=np.float64)
    _load().oracle_householder_tridiag(n, _dp(M), _dp(d), _dp(e))
    return d, e[: n - 1]


def tridiag_eigvals(d: np.ndarray, e: np.ndarray) -> np.ndarray:
    d = np.ascontiguousarray(d, dtype=np.float64)
    e = np.ascontiguousarray(e if len(e) else np.zeros(1), dtype=np.float64)
    w = np.empty(len(d), dtype=np.float64)
    _load().oracle_tridiag_eigvals(len(d), _dp(d), _dp(e), _dp(w))
    return w


def tridiag_count_below(d: np.ndarray, e: np.ndarray, x: float) -> int:
    d = np.ascontiguousarray(d, dtype=np.float64)
    e = np.ascontiguousarray(e if len(e) else np.zeros(1), dtype=np.float64)
    pivmin = max(1.0, float(np.max(e * e)) if len(e) else 1.0) * 1e-300
    return int(_load().oracle_tridiag_count_below(len(d), _dp(d), _dp(e), float(x), pivmin))


def eigvalsh_large(A: np.ndarray) -> np.ndarray:
    """Eigenvalues (descending) of a dense symmetric matrix: Householder
    tridiagonalisation, then bisection on Sturm counts.  Only the lower
    triangle of A is read (it is mirrored first)."""
    L = np.tril(np.asarray(A, dtype=np.float64))
    M = np.ascontiguousarray(L + np.tril(L, -1).T)
    n = M.shape[0]
    w = np.empty(n, dtype=np.float64)
    _load().oracle_eigvalsh_dense(n, _dp(M), _dp(w))
    return w


def eigh_vectors(A: np.ndarray, k: int):
    """(w, U): the k largest eigenvalues of the symmetric A, descending, and
    their unit eigenvectors as U's columns (fp64, LAPACK's dsyevd as the library
    step; signs as LAPACK returns them) -- "Random matrix theory spectral
    methods" page, section 4.1 (P = [u_1 .. u_k], the eigenvectors of the
    largest eigenvalues)."""
    A = np.asarray(A, dtype=np.float64)
    w, U = np.linalg.eigh((A + A.T) / 2)
    return w[::-1][:k].copy(), U[:, ::-1][:, :k].copy()


def count_below_dense(A: np.ndarray, x: float) -> int:
    """#{lambda < x} of a dense symmetric matrix from the inertia of LDL^T(A - xI)."""
    L = np.tril(np.asarray(A, dtype=np.float64))
    M = np.ascontiguousarray(L + np.tril(L, -1).T)
    return int(_load().oracle_ldlt_count_below(M.shape[0], _dp(M), float(x)))


# ---------------------------------------------------------------- Marchenko-Pastur

def mp_edges(sigma2: float, c: float):
    """(lambda_minus, lambda_plus) = sigma^2 (1 -/+ sqrt(c))^2 (RMT page, section 2.1)."""
    return sigma2 * (1.0 - math.sqrt(c)) ** 2, sigma2 * (1.0 + math.sqrt(c)) ** 2


def mp_density(x, sigma2: float, c: float):
    """rho(x) = sqrt((l+ - x)(x - l-)) / (2 pi sigma^2 c x) on [l-, l+] (RMT page, section 2.1)."""
    lm, lp = mp_edges(sigma2, c)
    x = np.asarray(x, dtype=np.float64)
    inside = (x > lm) & (x < lp)
    r = np.zeros_like(x)
    xi = x[inside]
    r[inside] = np.sqrt((lp - xi) * (xi - lm)) / (2.0 * math.pi * sigma2 * c * xi)
    return r


_GL = {}


def _gauss_legendre(m: int):
    if m not in _GL:
        _GL[m] = np.polynomial.legendre.leggauss(m)
    return _GL[m]


def _mp_cdf_phi(phi, sigma2: float, c: float, nodes: int = 24) -> np.ndarray:
    """F at lambda(phi) = m - h cos(phi), m = (l+ + l-)/2, h = (l+ - l-)/2.

    In phi the measure rho(lambda) dlambda = h^2 sin^2(phi) / (2 pi sigma^2 c
    lambda(phi)) dphi is smooth on [0, pi] but, for c close to 1, sharply
    peaked near phi = 0 (lambda_minus -> 0); composite Gauss-Legendre on the
    panels [0, 2^-20 phi], [2^-20 phi, 2^-19 phi], ..., [phi / 2, phi]."""
    lm, lp = mp_edges(sigma2, c)
    m, h = 0.5 * (lp + lm), 0.5 * (lp - lm)
    phi = np.atleast_1d(np.asarray(phi, dtype=np.float64))
    t, wt = _gauss_legendre(nodes)
    edges = np.concatenate([[0.0], 2.0 ** np.arange(-20, 1)])  # fractions of phi
    total = np.zeros_like(phi)
    for a, b in zip(edges[:-1], edges[1:]):
        lo, hi = a * phi, b * phi
        ph = 0.5 * (hi - lo)[:, None] * (t[None, :] + 1.0) + lo[:, None]
        lam = lm + 2.0 * h * np.sin(0.5 * ph) ** 2  # = m - h cos(phi), no cancellation
        f = h * h * np.sin(ph) ** 2 / (2.0 * math.pi * sigma2 * c * lam)
        total += 0.5 * (hi - lo) * np.sum(wt[None, :] * f, axis=1)
    return total


def mp_cdf(x: float, sigma2: float, c: float, nodes: int = 24) -> float:
    """F(x) = integral of rho from lambda_minus to x, for 0 < c <= 1."""
    lm, lp = mp_edges(sigma2, c)
    if x <= lm:
        return 0.0
    if x >= lp:
        return 1.0
    m, h = 0.5 * (lp + lm), 0.5 * (lp - lm)
    phi_x = math.acos(max(-1.0, min(1.0, (m - x) / h)))
    return float(_mp_cdf_phi(phi_x, sigma2, c, nodes)[0])


_QCACHE = {}


def mp_quantiles(sigma2: float, c: float, r: int, u=None) -> np.ndarray:
    """Midpoint quantiles Q((i - 1/2)/r), i = 1..r, ascending (or Q(u) for the
    given levels), for 0 < c <= 1: each by bisection in phi on [0, pi] until
    the bracket stops shrinking, all levels side by side."""
    key = (float(sigma2), float(c), int(r)) if u is None else None
    if key is not None and key in _QCACHE:
        return _QCACHE[key].copy()
    lm, lp = mp_edges(sigma2, c)
    m, h = 0.5 * (lp + lm), 0.5 * (lp - lm)
    if u is None:
        u = (np.arange(1, r + 1, dtype=np.float64) - 0.5) / r
    u = np.atleast_1d(np.asarray(u, dtype=np.float64))
    a = np.zeros_like(u)
    b = np.full_like(u, math.pi)
    for _ in range(64):
        mid = 0.5 * (a + b)
        below = _mp_cdf_phi(mid, sigma2, c) < u
        a = np.where(below, mid, a)
        b = np.where(below, b, mid)
    q = lm + 2.0 * h * np.sin(0.25 * (a + b)) ** 2
    if key is not None:
        _QCACHE[key] = q.copy()
    return q


def mp_quantile(u: float, sigma2: float, c: float) -> float:
    return float(mp_quantiles(sigma2, c, 1, u=[u])[0])


# ---------------------------------------------------------------- descriptors

EIG, SINGULAR = 0, 1
SIGMA2_GIVEN, SIGMA2_MEDIAN, SIGMA2_MEAN = 0, 1, 2


def descriptors(w, *, mode: int = EIG, n_samples: int = 1, p_dim: int = 1, k: int = 1,
                sigma2: float = 1.0, sigma2_mode: int = SIGMA2_GIVEN, top_frac: float = 0.2,
                small_rel: float = 1e-2, tail_frac: float = 0.7, with_mp: bool = True) -> dict:
    """Spectral descriptors of one spectrum ``w`` (eigenvalues of a covariance,
    any order).  Negative round-off is clamped to zero first.

    * S = sum(lambda); p_i = lambda_i / S
    * H = -sum p_i ln p_i with 0 ln 0 = 0 (spectral entropy); erank = exp(H)
    * m1 = lambda_1 / S (leading eigenvalue mass); g_k = lambda_k / lambda_{k+1}
      (eigengap as a ratio); g1 = lambda_1 / lambda_2
      -- RMT page, section 2.3
    * c = p / n; lambda_plus = sigma^2 (1 + sqrt c)^2; n_above = #{lambda > lambda_plus}
      -- RMT page, section 2.1
    * mp_w1: W1 distance between the spectrum and the MP law, as the mean of
      |mu_(i) - Q((i - 1/2)/r)| over the ascending spectrum; for p > n the
      companion spectrum mu = (n/p) lambda with ratio n/p is used
    * sigma_i = sqrt(lambda_i): top_energy = sum_{i<=floor(f r)} sigma_i^2 / sum sigma^2,
      top_sigma_share the same with sigma_i; tail_head = sigma at rank
      floor(0.7 r) + 1, tail_min = sigma_r; n_small = #{sigma_i < small_rel sigma_1}
      -- S3 page, section 1 (the long-tail test) and section 2 (the count of
      near-zero singular values)
    """
    lam = np.sort(np.maximum(np.asarray(w, dtype=np.float64), 0.0))[::-1]
    r = lam.size
    S = float(np.sum(lam))
    out = {"S": S}
    p = lam / S if S > 0 else np.full(r, np.nan)
    nz = p > 0
    H = float(-np.sum(p[nz] * np.log(p[nz]))) if S > 0 else float("nan")
    out["H"] = H
    out["erank"] = math.exp(H) if S > 0 else float("nan")
    out["m1"] = float(lam[0] / S) if S > 0 else float("nan")
    out["gk"] = float(lam[k - 1] / lam[k]) if (k < r and lam[k] > 0) else float("nan")
    out["g1"] = float(lam[0] / lam[1]) if (r > 1 and lam[1] > 0) else float("nan")
    if sigma2_mode == SIGMA2_MEDIAN:
        s2 = float(np.median(lam))
    elif sigma2_mode == SIGMA2_MEAN:
        s2 = S / p_dim
    else:
        s2 = float(sigma2)
    out["sigma2"] = s2
    c = p_dim / n_samples
    out["lambda_plus"] = s2 * (1.0 + math.sqrt(c)) ** 2
    out["n_above"] = int(np.sum(lam > out["lambda_plus"]))
    out["r_pos"] = int(np.sum(lam > 0))
    if with_mp and s2 > 0:
        if p_dim <= n_samples:
            mu, cc = lam[::-1], c
        else:
            mu, cc = (n_samples / p_dim) * lam[::-1], n_samples / p_dim
        q = mp_quantiles(s2, cc, r)
        out["mp_w1"] = float(np.mean(np.abs(mu - q)))
    else:
        out["mp_w1"] = float("nan")
    sig = np.sqrt(lam)
    kt = int(math.floor(top_frac * r))
    e2 = float(np.sum(sig * sig))
    out["top_energy"] = float(np.sum(sig[:kt] ** 2) / e2) if e2 > 0 else float("nan")
    s1 = float(np.sum(sig))
    out["top_sigma_share"] = float(np.sum(sig[:kt]) / s1) if s1 > 0 else float("nan")
    out["tail_head"] = float(sig[min(r - 1, int(math.floor(tail_frac * r)))])
    out["tail_min"] = float(sig[-1])
    out["sigma1"] = float(sig[0])
    out["n_small"] = int(np.sum(sig < small_rel * sig[0]))
    return out


# ---------------------------------------------------------------- descriptor post-processing

SIGMA2_WINSOR = 3
#: the fp64 fields of a descriptor record, smoothed as time series
SMOOTH_FIELDS = ["S", "H", "erank", "m1", "gk", "g1", "sigma2", "lambda_plus", "mp_w1",
                 "top_energy", "top_sigma_share", "tail_head", "tail_min", "sigma1"]
FLAG_HELD = 8


def smooth_series(x, alpha: float) -> np.ndarray:
    """Exponential smoothing of one descriptor time series ("Random matrix
    theory spectral methods" page, section 3.2: the descriptor series are
    exponentially smoothed): y_0 = x_0, y_t = alpha x_t + (1 - alpha) y_{t-1}.

    Reading (the page gives no rule for gaps): a non-finite x_t leaves the state
    as it was (y_t = y_{t-1}); before the first finite value y_t is NaN."""
    y = np.empty(len(x), dtype=np.float64)
    state, have = float("nan"), False
    for t, v in enumerate(x):
        v = float(v)
        if math.isfinite(v):
            state = v if not have else alpha * v + (1.0 - alpha) * state
            have = True
        y[t] = state if have else float("nan")
    return y


def smooth_descriptors(rec: np.ndarray, alpha: float) -> np.ndarray:
    """rec: structured records [streams, W] with the fields of a descriptor
    record.  Every field in SMOOTH_FIELDS is smoothed along W (smooth_series);
    counts are copied; flags gain FLAG_HELD where a record has a non-finite
    smoothed field."""
    out = rec.copy()
    for s in range(rec.shape[0]):
        held = np.zeros(rec.shape[1], dtype=bool)
        for f in SMOOTH_FIELDS:
            out[f][s] = smooth_series(rec[f][s], alpha)
            held |= ~np.isfinite(rec[f][s].astype(np.float64))
        out["flags"][s] = rec["flags"][s] | np.where(held, FLAG_HELD, 0)
    return out


def mp_bin_masses(sigma2: float, c: float, bins: int) -> np.ndarray:
    """MP probability of each of `bins` equal-width bins of [lambda_-, lambda_+]
    (differences of mp_cdf at the bin edges)."""
    lm, lp = mp_edges(sigma2, c)
    edges = [lm + (lp - lm) * b / bins for b in range(bins + 1)]
    F = [0.0] + [mp_cdf(x, sigma2, c) for x in edges[1:-1]] + [1.0]
    return np.diff(np.asarray(F, dtype=np.float64))


def robust_stats(w, *, n_samples: int, p_dim: int, sigma2: float = 1.0, sigma2_mode: int = SIGMA2_GIVEN,
                 winsor_frac: float = 0.05, mad_k: float = 3.0, bins: int = 16) -> dict:
    """Robust and log-domain statistics of one spectrum (negative round-off
    clamped to 0):

    * median, and sigma2_winsor = (sum of the winsorised spectrum) / p: the q =
      floor(winsor_frac r) largest values set to the (q+1)-th largest and the q
      smallest to the (q+1)-th smallest (q <= (r-1)/2), the MEAN estimate of
      sigma^2 made robust to extreme eigenvalues; mad = median |lambda - median|
      and n_mad = #{|lambda - median| > mad_k * 1.4826 * mad} (outliers by the
      median absolute deviation, 1.4826 its normal-consistency factor) -- RMT
      page, section 4.2 (median rather than mean for sigma^2, winsorised
      extremes, MAD anomaly detection)
    * log_mean, log_std: mean and (population) standard deviation of ln lambda
      over the finite positive eigenvalues -- section 3.2 (log transform of the
      eigenvalues)
    * kl_mp = sum_b p_b ln(p_b / q_b): KL divergence of the spectrum's histogram
      over `bins` equal-width bins of [lambda_-, lambda_+] (values outside
      counted in the end bins) from the MP bin masses q_b -- section 2.3 (KL form
      of the MP deviation); sigma^2 by sigma2_mode (GIVEN, MEDIAN, MEAN = S/p,
      WINSOR = sigma2_winsor) and the companion form for p > n as in mp_w1.
    Undefined values are NaN (flags: 1 non-finite input -- a NaN makes every
    order statistic, sum and sigma^2 estimate NaN, an infinity enters them as a
    value; 4 no finite positive value)."""
    raw = np.asarray(w, dtype=np.float64)
    flags = 0 if np.all(np.isfinite(raw)) else 1
    lam = np.sort(np.maximum(raw, 0.0))[::-1]
    r = lam.size
    med = float(np.median(lam))
    asc = lam[::-1]
    q = min(int(math.floor(winsor_frac * r)), (r - 1) // 2)
    wz = np.clip(asc, asc[q], asc[r - 1 - q])
    s2w = float(np.sum(wz)) / p_dim
    dev = np.abs(lam - med)
    mad = float(np.median(dev))
    n_mad = int(np.sum(dev > mad_k * 1.4826 * mad))
    pos = lam[(lam > 0) & np.isfinite(lam)]
    if pos.size:
        lg = np.log(pos)
        log_mean = float(np.mean(lg))
        log_std = float(math.sqrt(np.mean((lg - log_mean) ** 2)))
    else:
        log_mean = log_std = float("nan")
        flags |= 4
    S = float(np.sum(lam))
    if sigma2_mode == SIGMA2_MEDIAN:
        s2 = med
    elif sigma2_mode == SIGMA2_MEAN:
        s2 = S / p_dim
    elif sigma2_mode == SIGMA2_WINSOR:
        s2 = s2w
    else:
        s2 = float(sigma2)
    kl = float("nan")
    if s2 > 0 and flags & 1 == 0:
        if p_dim <= n_samples:
            mu, cc = lam, p_dim / n_samples
        else:
            mu, cc = (n_samples / p_dim) * lam, n_samples / p_dim
        lm, lp = mp_edges(s2, cc)
        qb = mp_bin_masses(s2, cc, bins)
        cnt = np.zeros(bins, dtype=np.int64)
        for v in mu:
            b = int(math.floor((v - lm) / (lp - lm) * bins))
            cnt[min(max(b, 0), bins - 1)] += 1
        pb = cnt / r
        nz = pb > 0
        kl = float(np.sum(pb[nz] * np.log(pb[nz] / qb[nz])))
    return {"median": med, "sigma2_winsor": s2w, "mad": mad, "log_mean": log_mean, "log_std": log_std,
            "sigma2": s2, "kl_mp": kl, "n_mad": n_mad, "flags": flags}


# ---------------------------------------------------------------- randomised top eigenvalues

def topk_ritz(A: np.ndarray, Omega: np.ndarray, q: int) -> np.ndarray:
    """Approximate leading eigenvalues of the symmetric A (d x d) by random
    projection ("Random matrix theory spectral methods" page, section 3.2: top-k
    eigenvalues from a random projection in O(k d^2) instead of O(d^3)).

    Reading (the page names the idea only): the randomised range finder with q
    steps of subspace iteration and Rayleigh-Ritz -- Y = A Omega, Q = orth(Y),
    then q times Q = orth(A Q), and the Ritz values eig(Q^T A Q), descending.
    Omega (d x l) is the caller's random test matrix; orth is a Householder QR
    (numpy.linalg.qr, a library primitive).  All l Ritz values are returned; the
    leading k of them, k < l, approximate the leading k eigenvalues."""
    A = np.asarray(A, dtype=np.float64)
    Q, _ = np.linalg.qr(A @ np.asarray(Omega, dtype=np.float64))
    for _ in range(q):
        Q, _ = np.linalg.qr(A @ Q)
    B = Q.T @ A @ Q
    B = 0.5 * (B + B.T)
    return np.sort(np.linalg.eigvalsh(B))[::-1]


def topk_ritz_vectors(A: np.ndarray, Omega: np.ndarray, q: int):
    """Ritz values (descending) and Ritz vectors P = Q U of topk_ritz: the
    columns of P are orthonormal and span the range found by the projection;
    column i belongs to Ritz value i.  The leading columns approximate the
    leading eigenvectors; those with a Ritz value above the MP edge are the
    signal subspace (RMT page, section 4.1: the eigenvectors
    beyond lambda_plus span it, P = [u_1 .. u_k])."""
    A = np.asarray(A, dtype=np.float64)
    Q, _ = np.linalg.qr(A @ np.asarray(Omega, dtype=np.float64))
    for _ in range(q):
        Q, _ = np.linalg.qr(A @ Q)
    B = Q.T @ A @ Q
    B = 0.5 * (B + B.T)
    th, U = np.linalg.eigh(B)
    order = np.argsort(th)[::-1]
    return th[order], Q @ U[:, order]


def project_weight(W, P):
    """Projection compression of a square weight (RMT page, section 4.1: with
    the signal-subspace basis P = [u_1 .. u_k] in R^{d x k}, the d x d layer
    weight W becomes W' = P^T W P in R^{k x k}).  Returns (W', X) with the
    right factor X = W P in R^{d x k}, the factor of the rank-k map
    W P P^T (W kept on the span of P).

    W: [d, d] float (bf16 as uint16 bit patterns, widened exactly); P: [d, k].
    Both products are plain fp64 matrix products, first X = W P, then
    W' = P^T X."""
    W = np.asarray(W)
    if W.dtype == np.uint16:
        W = (W.astype(np.uint32) << 16).view(np.float32)
    W = W.astype(np.float64)
    P = np.asarray(P, dtype=np.float64)
    X = W @ P
    return P.T @ X, X


def tail_pair_screen(U, V, *, i0: int, t: int, head_dim: int, eps: float = 0.015):
    """Screen of the swap candidates of the S3 page (section 3.1): for the left
    singular vectors u_i and right singular vectors v_j of the tail, i and j in
    [i0, i0 + t) (the page takes the last 10 %, i >= 0.9 N), the inner products
    |u_i^T v_j|; a pair is kept when it lies in one head's index range (indices
    split into consecutive blocks of head_dim: i // head_dim == j // head_dim)
    and |u_i^T v_j| < eps (the page keeps |u_i^T v_j| below 0.015, from its
    orthogonality constraint |u_i^T v_j| < eps, eps ~ 1e-2).

    U, V: [N, >= i0 + t] with the singular vectors as columns (f32 widened
    exactly, or f64).  Returns (absdot [t, t] fp64, keep [t, t] bool, count)."""
    Ut = np.asarray(U)[:, i0:i0 + t].astype(np.float64)
    Vt = np.asarray(V)[:, i0:i0 + t].astype(np.float64)
    absdot = np.abs(Ut.T @ Vt)
    idx = np.arange(i0, i0 + t)
    same = (idx[:, None] // head_dim) == (idx[None, :] // head_dim)
    keep = same & (absdot < eps)
    return absdot, keep, int(np.sum(keep))
