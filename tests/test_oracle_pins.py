"""Pins of the fp64 oracle against what the mathematics and the pages fix.

Nothing here compares the oracle with itself: each test checks it against a
closed form, an invariant, a textbook special case, a library routine on the
same input, or brute force on a tiny input, chosen so that a dropped term, a
wrong sign, a wrong index or a transposed operand in the oracle fails one of
them.  No test here needs a GPU.
"""
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg

import oracle
from gen import synth


def _sym(rng, n, scale=1.0):
    a = rng.standard_normal((n, n)) * scale
    return a + a.T


# ------------------------------------------------------------- P1/P2 invariants

@pytest.mark.parametrize("n,d", [(64, 32), (50, 7), (7, 50)])
def test_trace_and_frobenius(n, d):
    rng = np.random.default_rng(n * 100 + d)
    X = rng.standard_normal((n, d)).astype(np.float32)
    alpha = 1.0 / n
    C = oracle.covariance(X, "f32", alpha)
    w = oracle.eigvalsh_large(C)
    wj, _ = oracle.eigvalsh_small(C)
    tr = alpha * float(np.sum(X.astype(np.float64) ** 2))  # alpha ||X||_F^2
    for ev in (w, wj):
        assert abs(ev.sum() - tr) <= 1e-12 * tr
        fro2 = float(np.sum(C * C))
        assert abs(np.sum(ev ** 2) - fro2) <= 1e-11 * fro2


def test_covariance_brute_force():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((9, 5)).astype(np.float32)
    C = oracle.covariance(X, "f32", 0.5, C0=np.eye(5), beta=2.0, row_block=4)
    for i in range(5):
        for j in range(5):
            s = sum(float(X[r, i]) * float(X[r, j]) for r in range(9))
            assert abs(C[i, j] - (0.5 * s + 2.0 * (i == j))) <= 1e-13


def test_bf16_widening_and_rounding():
    import torch
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(10000) * 10.0 ** rng.uniform(-5, 5, 10000)).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]  # exact ties
    bits = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    wide = oracle.widen(bits, "bf16")
    assert np.array_equal(wide, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


# ------------------------------------------------------------- P3 library eigvalsh

@pytest.mark.parametrize("n", [1, 2, 3, 17, 30, 32, 64, 200])
def test_eigensolvers_vs_lapack(n):
    rng = np.random.default_rng(n)
    A = _sym(rng, n)
    ref = np.linalg.eigvalsh(A)[::-1]
    lmax = max(1.0, np.max(np.abs(ref)))
    w_large = oracle.eigvalsh_large(A)
    assert np.max(np.abs(w_large - ref)) <= 1e-12 * lmax
    if n <= 64:
        w_small, sweeps = oracle.eigvalsh_small(A)
        assert sweeps >= 0
        assert np.max(np.abs(w_small - ref)) <= 1e-12 * lmax
        # P11: both oracle eigensolvers agree
        assert np.max(np.abs(w_small - w_large)) <= 1e-12 * lmax


def test_eigensolvers_degenerate():
    # repeated eigenvalues, rank deficiency, zero matrix, huge dynamic range
    rng = np.random.default_rng(11)
    Q, _ = np.linalg.qr(rng.standard_normal((40, 40)))
    lam = np.array([5.0] * 10 + [1e-9] * 5 + [0.0] * 10 + list(np.logspace(-6, 6, 15)))
    A = (Q * lam) @ Q.T
    A = 0.5 * (A + A.T)
    ref = np.sort(lam)[::-1]
    for w in (oracle.eigvalsh_large(A), oracle.eigvalsh_small(A)[0]):
        assert np.max(np.abs(w - ref)) <= 1e-9 * ref[0]
    Z = np.zeros((8, 8))
    assert np.all(np.abs(oracle.eigvalsh_large(Z)) <= 1e-290) and np.all(oracle.eigvalsh_small(Z)[0] == 0)


def test_tridiagonal_form_is_similar():
    rng = np.random.default_rng(4)
    A = _sym(rng, 25)
    d, e = oracle.tridiagonalize(A)
    T = np.diag(d) + np.diag(e, 1) + np.diag(e, -1)
    assert np.allclose(np.linalg.eigvalsh(T), np.linalg.eigvalsh(A), atol=1e-12)
    # Sturm count against the eigenvalues of T from LAPACK
    ev = scipy.linalg.eigvalsh_tridiagonal(d, e)
    for x in [-5.0, 0.0, 0.3, 2.0, 10.0]:
        assert oracle.tridiag_count_below(d, e, x) == int(np.sum(ev < x))


# ------------------------------------------------------------- P4 Gram duality

def test_window_gram_duality_and_band():
    H = synth.eigentrack(streams=2, T=40, d=96)
    N = 30
    G = oracle.window_gram(H[1], "bf16", N)
    assert G.shape == (40 - N + 1, N, N)
    h = oracle.widen(H[1], "bf16")
    for w in [0, 5, 10]:
        hw = h[w:w + N]
        cov = hw.T @ hw / N  # d x d covariance of the window
        ev_cov = np.linalg.eigvalsh(cov)[::-1]
        ev_g, _ = oracle.eigvalsh_small(G[w])
        assert np.max(np.abs(ev_cov[:N] - ev_g)) <= 1e-11 * ev_g[0]
        assert np.max(np.abs(ev_cov[N:])) <= 1e-11 * ev_g[0]
    # band entries by brute-force dot products, and the window Gram from the band
    B = oracle.band_gram(H, "bf16", N)
    for (s, t, j) in [(0, 0, 0), (0, 39, 29), (1, 17, 3), (1, 29, 29), (1, 5, 9)]:
        hs = oracle.widen(H[s], "bf16")
        ref = sum(hs[t, k] * hs[t - j, k] for k in range(96)) if t - j >= 0 else 0.0
        assert abs(B[s, t, j] - ref) <= 1e-12 * max(1.0, abs(ref))
    for w in [0, 7, 10]:
        for i in range(N):
            for j in range(N):
                assert abs(G[w, i, j] - B[1, w + max(i, j), abs(i - j)] / N) <= 1e-12 * G[w, 0, 0]


def test_band_window_gram_pins():
    """The window Gram rebuilt from a band: equal to window_gram straight from H
    (stride 1 and 3), entries by hand-indexed loops, and consecutive windows
    sharing their (N-1) x (N-1) block, whose spectrum interlaces both windows'
    (Cauchy), so a shifted or transposed band index fails."""
    H = synth.eigentrack(streams=1, T=60, d=40)[0]
    N = 9
    B = oracle.band_gram(H, "bf16", N)[0]
    for stride in (1, 3):
        K = oracle.band_window_gram(B, N, 1.0 / N, stride=stride)
        G = oracle.window_gram(H, "bf16", N, stride=stride)
        assert K.shape == G.shape == ((60 - N) // stride + 1, N, N)
        assert np.max(np.abs(K - G)) <= 1e-12 * np.max(np.abs(G))
    K = oracle.band_window_gram(B, N, 2.0, stride=2, windows=[4])[0]
    for i in range(N):
        for j in range(N):
            t, lag = 8 + max(i, j), abs(i - j)
            assert K[i, j] == 2.0 * B[t, lag]
    K = oracle.band_window_gram(B, N, 1.0)
    for w in range(0, K.shape[0] - 1, 7):
        assert np.array_equal(K[w, 1:, 1:], K[w + 1, :-1, :-1])
        inner = np.linalg.eigvalsh(K[w, 1:, 1:])
        for A in (K[w], K[w + 1]):
            lam = np.linalg.eigvalsh(A)
            tol = 1e-12 * lam[-1]
            assert np.all(lam[:-1] <= inner + tol) and np.all(inner <= lam[1:] + tol)


# ------------------------------------------------------------- P5 MP bulk

def test_mp_bulk_pure_noise():
    rng = np.random.default_rng(21)
    n, p = 4096, 1024
    X = rng.standard_normal((n, p)).astype(np.float32)
    C = oracle.covariance(X, "f32", 1.0 / n)
    w = oracle.eigvalsh_large(C)
    c = p / n
    lm, lp = oracle.mp_edges(1.0, c)
    sj = (math.sqrt(n - 1) + math.sqrt(p)) * (1 / math.sqrt(n - 1) + 1 / math.sqrt(p)) ** (1 / 3)
    delta = 5 * sj / n
    assert w.min() >= lm - delta and w.max() <= lp + delta
    # Kolmogorov distance to F_MP
    ws = np.sort(w)
    F = np.array([oracle.mp_cdf(x, 1.0, c) for x in ws])
    emp = np.arange(1, p + 1) / p
    assert np.max(np.abs(F - emp)) < 0.02
    # the W1 descriptor is small on pure noise and grows with a spike
    d0 = oracle.descriptors(w, n_samples=n, p_dim=p)["mp_w1"]
    assert d0 < 0.01
    X2 = X + 3.0 * rng.standard_normal((n, 1)).astype(np.float32) @ np.ones((1, p), np.float32) / math.sqrt(p)
    d1 = oracle.descriptors(oracle.eigvalsh_large(oracle.covariance(X2, "f32", 1.0 / n)),
                            n_samples=n, p_dim=p)["mp_w1"]
    assert d1 > d0


# ------------------------------------------------------------- P6 BBP outliers

def test_bbp_outliers_tiny_config():
    X = synth.tiny()
    C = oracle.covariance(X, "f32", 1.0 / 64)
    w = oracle.eigvalsh_large(C)
    D = oracle.descriptors(w, n_samples=64, p_dim=32, k=1)
    assert abs(D["lambda_plus"] - (1 + math.sqrt(0.5)) ** 2) < 1e-15
    assert D["n_above"] == 2  # the two planted spikes, both far above the edge


def test_bbp_outlier_location():
    # additive spike theta u u^T on sigma^2 = 1 noise; above sigma^2 sqrt(c) the top
    # sample eigenvalue sits near (1 + theta)(1 + c / theta) (Baik-Silverstein, Paul 2007)
    rng = np.random.default_rng(8)
    n, p = 8000, 400
    c = p / n
    thetas = np.array([3.0, 1.0])
    u, _ = np.linalg.qr(rng.standard_normal((p, 2)))
    X = rng.standard_normal((n, p)) + (rng.standard_normal((n, 2)) * np.sqrt(thetas)) @ u.T
    w = oracle.eigvalsh_large(oracle.covariance(X.astype(np.float32), "f32", 1.0 / n))
    for i, th in enumerate(thetas):
        pred = (1 + th) * (1 + c / th)
        sd = math.sqrt(2.0 / n) * (1 + th) * math.sqrt(1 - c / th ** 2)
        assert abs(w[i] - pred) < 5 * sd
    lp = oracle.mp_edges(1.0, c)[1]
    assert np.sum(w > lp) == 2


# ------------------------------------------------------------- P7 descriptors

def test_descriptors_diagonal_identity_rank1():
    lam = np.array([4.0, 3.0, 2.0, 1.0, 0.0])
    D = oracle.descriptors(lam[::-1], n_samples=10, p_dim=5, k=2)  # any input order
    p = lam / 10.0
    H = -sum(x * math.log(x) for x in p if x > 0)
    assert abs(D["S"] - 10.0) < 1e-15 and abs(D["H"] - H) < 1e-15
    assert abs(D["erank"] - math.exp(H)) < 1e-14
    assert D["m1"] == 0.4 and D["gk"] == 1.5 and abs(D["g1"] - 4 / 3) < 1e-15
    assert D["r_pos"] == 4
    n = 37
    Di = oracle.descriptors(np.ones(n), n_samples=1000, p_dim=n, k=3)
    assert abs(Di["H"] - math.log(n)) < 1e-13 and abs(Di["m1"] - 1 / n) < 1e-15 and Di["gk"] == 1.0
    Dr = oracle.descriptors(np.array([7.0] + [0.0] * 9), n_samples=100, p_dim=10, k=1)
    assert Dr["H"] == 0.0 and Dr["m1"] == 1.0 and math.isnan(Dr["gk"])
    # negative round-off is clamped before anything else
    Dn = oracle.descriptors(np.array([2.0, 1.0, -1e-17]), n_samples=100, p_dim=3)
    assert Dn["r_pos"] == 2 and Dn["tail_min"] == 0.0


def test_descriptors_sigma2_mean_from_the_data():
    # MEAN: sigma^2 = tr C / p.  For C = alpha X^T X that is alpha ||X||_F^2 / p,
    # computed here from X itself, whatever the number r of eigenvalues handed
    # over: the n nonzero eigenvalues of the Gram (r = n < p) or all p of them.
    rng = np.random.default_rng(31)
    for n, p, alpha in [(30, 200, 1.0 / 30), (500, 60, 1.0), (64, 32, 1.0 / 64)]:
        X = rng.standard_normal((n, p)) * 1.5
        fro2 = float(np.sum(X * X))
        if n < p:
            w = np.linalg.eigvalsh(alpha * (X @ X.T))  # r = n values
        else:
            w = np.linalg.eigvalsh(alpha * (X.T @ X))  # r = p values
        assert w.size != p or n >= p
        D = oracle.descriptors(w, n_samples=n, p_dim=p, k=1, sigma2_mode=oracle.SIGMA2_MEAN)
        s2 = alpha * fro2 / p
        assert abs(D["sigma2"] - s2) <= 1e-12 * s2
        lp = s2 * (1.0 + math.sqrt(p / n)) ** 2
        assert abs(D["lambda_plus"] - lp) <= 1e-12 * lp
        assert D["n_above"] == int(np.sum(w > lp))
    # a spectrum with one value far out: sigma^2 = 23 / 4, lambda_plus = 5.75 (1 + 1)^2 = 23,
    # so 20 is below the edge and only a value above 23 would count
    D = oracle.descriptors([20.0, 1.0, 1.0, 1.0], n_samples=4, p_dim=4, sigma2_mode=oracle.SIGMA2_MEAN)
    assert D["sigma2"] == 23.0 / 4 and D["lambda_plus"] == 23.0 and D["n_above"] == 0


def test_descriptors_sigma2_median_by_hand():
    # odd r: median of (5, 1, 3) is 3; c = 3 / 12 -> lambda_plus = 3 (1 + 1/2)^2 = 6.75
    D = oracle.descriptors([5.0, 1.0, 3.0], n_samples=12, p_dim=3, sigma2_mode=oracle.SIGMA2_MEDIAN)
    assert D["sigma2"] == 3.0 and D["lambda_plus"] == 6.75 and D["n_above"] == 0
    # even r: the mean of the two middle values, (6 + 2) / 2 = 4; c = 1 -> lambda_plus = 16
    D = oracle.descriptors([8.0, 0.0, 6.0, 2.0, 17.0, 1.0], n_samples=6, p_dim=6,
                           sigma2_mode=oracle.SIGMA2_MEDIAN)
    assert D["sigma2"] == (6.0 + 2.0) / 2 and D["lambda_plus"] == 16.0 and D["n_above"] == 1
    # negative round-off is clamped before the median: (-1e-9, 0, 0, 7) -> (0 + 0) / 2
    D = oracle.descriptors([-1e-9, 0.0, 0.0, 7.0], n_samples=8, p_dim=4, sigma2_mode=oracle.SIGMA2_MEDIAN)
    assert D["sigma2"] == 0.0 and math.isnan(D["mp_w1"])
    # GIVEN ignores the spectrum
    D = oracle.descriptors([5.0, 1.0, 3.0], n_samples=12, p_dim=3, sigma2=0.5)
    assert D["sigma2"] == 0.5 and D["lambda_plus"] == 0.5 * 2.25


def test_descriptors_singular_mode_counts():
    d = 4096
    sig = synth.s3_sigma(d)
    assert sig[0] == 1.0 and abs(sig[-1] - 1e-3) < 1e-15
    assert np.min(np.abs(sig - 1e-2)) > 1e-5  # no tie at the small-sigma threshold
    D = oracle.descriptors(sig ** 2, mode=oracle.SINGULAR, n_samples=d, p_dim=d)
    assert D["n_small"] == int(np.sum(sig < 1e-2)) == d - 203
    k = int(0.2 * d)
    assert abs(D["top_energy"] - np.sum(sig[:k] ** 2) / np.sum(sig ** 2)) < 1e-14
    assert abs(D["top_sigma_share"] - np.sum(sig[:k]) / np.sum(sig)) < 1e-14
    assert D["tail_head"] == sig[int(0.7 * d)] and D["tail_min"] == sig[-1]


@pytest.mark.parametrize("c", [0.01, 0.25, 0.5, 0.9, 0.99, 1.0])
def test_mp_law_moments_and_cdf(c):
    s2 = 1.7
    lm, lp = oracle.mp_edges(s2, c)
    # total mass 1 (c <= 1), mean sigma^2, second moment sigma^4 (1 + c)
    mass = scipy.integrate.quad(lambda x: oracle.mp_density([x], s2, c)[0], lm, lp, limit=200)[0]
    assert abs(mass - 1.0) < 1e-6
    assert abs(oracle.mp_cdf(lp * (1 - 1e-15), s2, c) - 1.0) < 1e-9
    r = 2000
    q = oracle.mp_quantiles(s2, c, r)
    assert np.all(np.diff(q) > 0) and q[0] > lm and q[-1] < lp
    assert abs(q.mean() - s2) < 2e-3 * s2
    assert abs(np.mean(q ** 2) - s2 ** 2 * (1 + c)) < 5e-3 * s2 ** 2
    # the quadrature CDF against adaptive quadrature of the printed density
    for u in [0.1, 0.5, 0.9]:
        x = oracle.mp_quantile(u, s2, c)
        F = scipy.integrate.quad(lambda t: oracle.mp_density([t], s2, c)[0], lm, x, limit=200)[0]
        assert abs(F - u) < 1e-7


def test_w1_zero_on_quantiles():
    r, c = 50, 0.3
    q = oracle.mp_quantiles(1.0, c, r)
    D = oracle.descriptors(q, n_samples=1000, p_dim=int(round(c * 1000)), k=1)
    assert D["mp_w1"] < 1e-12
    # companion form when p > n: eigenvalues lambda = (p/n) mu with mu ~ MP(n/p)
    n, p = 30, 4096
    qc = oracle.mp_quantiles(1.0, n / p, n)
    Dc = oracle.descriptors(qc * p / n, n_samples=n, p_dim=p)
    assert Dc["mp_w1"] < 1e-12


# ------------------------------------------------------------- P8 brute-force SVD

def test_singular_values_closed_form_2x2_and_svd():
    a, b, c_, d = 3.0, 1.0, -2.0, 0.5
    W = np.array([[a, b], [c_, d]], dtype=np.float32)
    C = oracle.covariance(W, "f32", 1.0)
    s = np.sqrt(np.maximum(oracle.eigvalsh_large(C), 0))
    # closed form: s1 s2 = |det W|, s1^2 + s2^2 = ||W||_F^2
    assert abs(s[0] * s[1] - abs(a * d - b * c_)) < 1e-13
    assert abs(s[0] ** 2 + s[1] ** 2 - (a * a + b * b + c_ * c_ + d * d)) < 1e-13
    rng = np.random.default_rng(9)
    for m in (5, 33, 64):
        W = rng.standard_normal((m + 3, m)).astype(np.float32)
        s = np.sqrt(np.maximum(oracle.eigvalsh_small(oracle.covariance(W, "f32", 1.0))[0], 0))
        ref = np.linalg.svd(W.astype(np.float64), compute_uv=False)
        assert np.max(np.abs(s - ref)) < 1e-12 * ref[0]


# ------------------------------------------------------------- P9 Weyl on the S3 layer

def test_s3_weyl_bound_reduced():
    d = 256
    W64 = synth.s3_layer_f64(0, d)
    W32 = W64.astype(np.float32)
    planted = synth.s3_sigma(d)
    s = np.sqrt(np.maximum(oracle.eigvalsh_large(oracle.covariance(W32, "f32", 1.0)), 0))
    bound = np.linalg.norm(W32.astype(np.float64) - W64, 2)
    # Weyl: |sigma_i(W32) - sigma_i(W64)| <= ||W32 - W64||_2; the Gram route adds
    # fp64 rounding of order eps * sigma_1^2 / sigma_i on the smallest values
    err = np.abs(s - planted)
    assert np.all(err <= bound + 1e-12 / planted)


# ------------------------------------------------------------- P10 inertia counts

def test_eigh_vectors_pins():
    """The oracle's eigenpairs: A u = lambda u and U^T U = I to rounding, its
    eigenvalues equal to the Householder + bisection ones, and the 2 x 2
    rotation in closed form (tan 2 theta = 2b / (a - c))."""
    rng = np.random.default_rng(17)
    A = _sym(rng, 120)
    w, U = oracle.eigh_vectors(A, 120)
    assert np.max(np.abs(A @ U - U * w)) <= 1e-12 * np.max(np.abs(w))
    assert np.max(np.abs(U.T @ U - np.eye(120))) <= 1e-13
    assert np.max(np.abs(w - oracle.eigvalsh_large(A))) <= 1e-12 * np.max(np.abs(w))
    w5, U5 = oracle.eigh_vectors(A, 5)
    assert np.array_equal(w5, w[:5]) and np.allclose(np.abs(U5), np.abs(U[:, :5]))
    a, b, c = 3.0, 1.5, -1.0
    th = 0.5 * math.atan2(2 * b, a - c)
    w2, U2 = oracle.eigh_vectors(np.array([[a, b], [b, c]]), 2)
    u = np.array([math.cos(th), math.sin(th)])
    assert abs(abs(U2[:, 0] @ u) - 1.0) <= 1e-14
    assert abs(w2[0] - ((a + c) / 2 + math.hypot((a - c) / 2, b))) <= 1e-14


def test_inertia_counts_match_spectrum():
    X = synth.tiny()
    C = oracle.covariance(X, "f32", 1.0 / 64)
    w = oracle.eigvalsh_large(C)
    lp = oracle.mp_edges(1.0, 0.5)[1]
    assert C.shape[0] - oracle.count_below_dense(C, lp) == int(np.sum(w > lp)) == 2
    rng = np.random.default_rng(2)
    A = _sym(rng, 120)
    ev = np.linalg.eigvalsh(A)
    for x in [-10.0, -1.0, 0.0, 2.5, 30.0]:
        assert oracle.count_below_dense(A, x) == int(np.sum(ev < x))


def test_jacobi_reports_non_convergence():
    rng = np.random.default_rng(1)
    A = _sym(rng, 30)
    w, sweeps = oracle.eigvalsh_small(A, max_sweeps=1)
    assert sweeps < 0


# ------------------------------------------------------------- descriptor post-processing

def test_smooth_closed_forms():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(40)
    assert np.array_equal(oracle.smooth_series(x, 1.0), x)  # alpha = 1: no smoothing
    assert np.allclose(oracle.smooth_series(np.full(30, 2.5), 0.3), 2.5, rtol=0, atol=1e-15)
    # step response from 0: y_t = 1 - (1 - a)^t
    a = 0.25
    y = oracle.smooth_series(np.r_[0.0, np.ones(20)], a)
    assert np.allclose(y[1:], 1.0 - (1.0 - a) ** np.arange(1, 21), rtol=0, atol=1e-15)
    # impulse after a zero start: y_t = a (1 - a)^(t - 1)
    y = oracle.smooth_series(np.r_[0.0, 1.0, np.zeros(10)], a)
    assert np.allclose(y[1:], a * (1.0 - a) ** np.arange(11), rtol=0, atol=1e-15)
    # linear in the series
    z = rng.standard_normal(40)
    assert np.allclose(oracle.smooth_series(2 * x - 3 * z, a),
                       2 * oracle.smooth_series(x, a) - 3 * oracle.smooth_series(z, a), atol=1e-13)
    # gaps: a non-finite value holds the state; NaN until the first finite value
    y = oracle.smooth_series([np.nan, 4.0, np.inf, 8.0], 0.5)
    assert np.isnan(y[0]) and y[1] == 4.0 and y[2] == 4.0 and y[3] == 6.0


def test_robust_stats_by_hand():
    # lambda = 9, 4, 3, 2, 1: median 3; |lambda - 3| = 6, 1, 0, 1, 2 -> MAD 1; with
    # k = 3 the cut is 4.4478, so one outlier; winsorising one value at each end
    # gives 4, 4, 3, 2, 2 (sum 15); ln: 0, ln 2, ln 3, ln 4, ln 9
    r = oracle.robust_stats([9, 4, 3, 2, 1], n_samples=10, p_dim=5, winsor_frac=0.2, mad_k=3.0)
    assert r["median"] == 3.0 and r["mad"] == 1.0 and r["n_mad"] == 1
    assert r["sigma2_winsor"] == 15.0 / 5
    lg = np.log([9.0, 4.0, 3.0, 2.0, 1.0])
    assert abs(r["log_mean"] - math.log(216.0) / 5) <= 1e-15
    assert abs(r["log_std"] - math.sqrt(np.mean((lg - lg.mean()) ** 2))) <= 1e-15
    # even count: the median is the mean of the two middle values
    r = oracle.robust_stats([10, 6, 2, 0], n_samples=8, p_dim=4)
    assert r["median"] == 4.0 and r["mad"] == 3.0  # deviations 6, 2, 2, 4, sorted 2, 2, 4, 6
    # no winsorising: the MEAN estimate S / p
    lam = np.random.default_rng(2).uniform(0, 3, 101)
    r = oracle.robust_stats(lam, n_samples=400, p_dim=101, winsor_frac=0.0)
    assert abs(r["sigma2_winsor"] - lam.sum() / 101) <= 1e-14 * lam.sum()
    # all zero: no positive value, no MP reference
    r = oracle.robust_stats(np.zeros(6), n_samples=10, p_dim=6, sigma2_mode=oracle.SIGMA2_MEDIAN)
    assert r["flags"] == 4 and math.isnan(r["log_mean"]) and math.isnan(r["kl_mp"])
    # a NaN value: flag 1, every order statistic and sigma^2 estimate NaN, while
    # the log statistics keep to the finite positive values (the reading for a case
    # the pages leave open), here ln 8, ln 2 and ln 1
    r = oracle.robust_stats([np.nan, 8.0, 2.0, 1.0, 0.0], n_samples=10, p_dim=5)
    assert r["flags"] & 1 and math.isnan(r["median"]) and math.isnan(r["sigma2_winsor"])
    assert abs(r["log_mean"] - math.log(16.0) / 3) <= 1e-15
    lg = np.log([8.0, 2.0, 1.0])
    assert abs(r["log_std"] - math.sqrt(np.mean((lg - lg.mean()) ** 2))) <= 1e-15


def test_mad_normal_consistency():
    # 1.4826 MAD estimates the standard deviation of a normal sample
    x = 12.0 + 2.0 * np.random.default_rng(4).standard_normal(200001)
    assert x.min() > 0  # the clamp to zero is a no-op
    r = oracle.robust_stats(x, n_samples=10 ** 6, p_dim=x.size)
    assert abs(1.4826 * r["mad"] - 2.0) < 0.02
    # and about 0.27 % of a normal sample lies beyond 3 of them
    assert abs(r["n_mad"] / x.size - 0.0027) < 0.0006


@pytest.mark.parametrize("c", [0.1, 0.5, 1.0])
def test_mp_bin_masses_by_quadrature(c):
    lm, lp = oracle.mp_edges(1.7, c)
    q = oracle.mp_bin_masses(1.7, c, 12)
    assert abs(q.sum() - 1.0) <= 1e-12
    edges = np.linspace(lm, lp, 13)
    for b in range(12):
        ref, _ = scipy.integrate.quad(lambda x: float(oracle.mp_density(np.array([x]), 1.7, c)[0]),
                                      edges[b], edges[b + 1], limit=200)
        assert abs(q[b] - ref) <= 1e-7, (b, q[b], ref)


def test_kl_pins():
    s2, n, p, B = 1.0, 1000, 250, 10  # c = 0.25
    lm, lp = oracle.mp_edges(s2, p / n)
    q = oracle.mp_bin_masses(s2, p / n, B)
    # every value in one bin: KL = -ln q_b
    for b in (0, 4, 9):
        v = lm + (lp - lm) * (b + 0.5) / B
        r = oracle.robust_stats(np.full(p, v), n_samples=n, p_dim=p, bins=B)
        assert abs(r["kl_mp"] + math.log(q[b])) <= 1e-12
    # values outside the support count in the end bins
    r = oracle.robust_stats([2 * lp, 0.5 * lm], n_samples=n, p_dim=p, bins=B)
    assert abs(r["kl_mp"] - (0.5 * math.log(0.5 / q[-1]) + 0.5 * math.log(0.5 / q[0]))) <= 1e-12
    # the MP quantiles themselves: the histogram matches the bin masses to 1/r
    rr = 20000
    mu = oracle.mp_quantiles(s2, 0.5, rr)
    r = oracle.robust_stats(mu, n_samples=2 * rr, p_dim=rr, bins=B)
    assert 0.0 <= r["kl_mp"] < 1e-6
    # non-negative on arbitrary spectra; the companion form for p > n scales by n / p
    rng = np.random.default_rng(9)
    for _ in range(5):
        lam = rng.uniform(0, 4, 64)
        assert oracle.robust_stats(lam, n_samples=100, p_dim=64, bins=8)["kl_mp"] >= 0.0
    lam = rng.uniform(0, 40, 30)
    a = oracle.robust_stats(lam, n_samples=30, p_dim=300, bins=8)["kl_mp"]
    b = oracle.robust_stats(lam * 0.1, n_samples=300, p_dim=30, bins=8)["kl_mp"]
    assert abs(a - b) <= 1e-12


def test_kl_sigma2_modes_by_hand():
    # lambda = 9, 3, 1, 1, 1 with p = 5, n = 20 (c = 0.25) and 10 bins: the MP support
    # is [0.25, 2.25] sigma^2 and a value v falls in bin floor((v / sigma^2 - 0.25) / 0.2),
    # clamped to [0, 9].  By hand, per sigma^2 mode:
    #   MEDIAN  sigma^2 = 1:                       1 -> 3.75 (bin 3); 3, 9 -> bin 9
    #   MEAN    sigma^2 = 15 / 5 = 3:              1 -> 0.42 (bin 0); 3 -> 3.75 (bin 3); 9 -> bin 9
    #   WINSOR  (q = 1: 1,1,1,3,3) sigma^2 = 1.8:  1 -> 1.53 (bin 1); 3 -> 7.08 (bin 7); 9 -> bin 9
    #   GIVEN   sigma^2 = 0.5:                     1 -> 8.75 (bin 8); 3, 9 -> bin 9
    # The MP bin masses depend on c only (sigma^2 scales the support), pinned by
    # quadrature in test_mp_bin_masses_by_quadrature.
    lam = [9.0, 3.0, 1.0, 1.0, 1.0]
    q = oracle.mp_bin_masses(1.0, 0.25, 10)
    assert np.allclose(oracle.mp_bin_masses(3.7, 0.25, 10), q, rtol=0, atol=1e-13)
    cases = [(oracle.SIGMA2_MEDIAN, 1.0, {3: 0.6, 9: 0.4}),
             (oracle.SIGMA2_MEAN, 3.0, {0: 0.6, 3: 0.2, 9: 0.2}),
             (oracle.SIGMA2_WINSOR, 1.8, {1: 0.6, 7: 0.2, 9: 0.2}),
             (oracle.SIGMA2_GIVEN, 0.5, {8: 0.6, 9: 0.4})]
    for mode, s2, bins in cases:
        r = oracle.robust_stats(lam, n_samples=20, p_dim=5, sigma2=0.5, sigma2_mode=mode,
                                winsor_frac=0.2, bins=10)
        assert abs(r["sigma2"] - s2) <= 1e-15 * s2, mode
        kl = sum(pb * math.log(pb / q[b]) for b, pb in bins.items())
        assert abs(r["kl_mp"] - kl) <= 1e-12 * abs(kl), (mode, r["kl_mp"], kl)


# ------------------------------------------------------------- randomised top eigenvalues

def _spd_with_spectrum(rng, lam):
    d = lam.size
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    return (Q * lam) @ Q.T


def test_topk_exact_on_low_rank():
    # rank 20 < 32 columns: the range finder captures the whole range, so the
    # Ritz values are the 20 nonzero eigenvalues followed by zeros
    rng = np.random.default_rng(21)
    lam = np.r_[np.linspace(10.0, 1.0, 20), np.zeros(280)]
    A = _spd_with_spectrum(rng, lam)
    r = oracle.topk_ritz(A, rng.standard_normal((300, 32)), q=0)
    assert np.max(np.abs(r[:20] - lam[:20])) <= 1e-11 * 10
    assert np.max(np.abs(r[20:])) <= 1e-11 * 10


def test_topk_interlacing_and_convergence():
    rng = np.random.default_rng(22)
    d = 400
    lam = 0.7 ** np.arange(d) * 5.0 + 1e-3  # fast decay
    A = _spd_with_spectrum(rng, lam)
    Om = rng.standard_normal((d, 32))
    ref = np.sort(np.linalg.eigvalsh(A))[::-1]
    prev = None
    for q in range(4):
        r = oracle.topk_ritz(A, Om, q)
        # Cauchy interlacing: each Ritz value is at most the eigenvalue of that rank
        assert np.all(r <= ref[:32] + 1e-12)
        err = np.max(np.abs(r[:10] - ref[:10]) / ref[:10])
        if prev is not None:
            assert err <= prev + 1e-15  # more iterations never hurt here
        prev = err
    assert prev <= 1e-10


def test_topk_depends_on_the_span_only():
    # Omega R spans the same space for an invertible R: the same Ritz values
    rng = np.random.default_rng(23)
    d = 200
    A = _spd_with_spectrum(rng, rng.uniform(0, 3, d))
    Om = rng.standard_normal((d, 32))
    R = rng.standard_normal((32, 32)) + 8 * np.eye(32)
    a = oracle.topk_ritz(A, Om, 1)
    b = oracle.topk_ritz(A, Om @ R, 1)
    assert np.max(np.abs(a - b)) <= 1e-9 * np.max(np.abs(a))


def test_topk_vectors_pins():
    rng = np.random.default_rng(31)
    d = 300
    lam = np.r_[np.linspace(12.0, 3.0, 10), rng.uniform(0.0, 0.5, d - 10)]
    A = _spd_with_spectrum(rng, lam)
    Om = rng.standard_normal((d, 32))
    th, P = oracle.topk_ritz_vectors(A, Om, 3)
    assert np.allclose(th, oracle.topk_ritz(A, Om, 3), rtol=0, atol=1e-12 * th[0])
    assert np.max(np.abs(P.T @ P - np.eye(32))) <= 1e-12           # orthonormal
    R = P.T @ A @ P
    assert np.max(np.abs(R - np.diag(th))) <= 1e-11 * th[0]        # Rayleigh-Ritz: P^T A P diagonal
    # the leading Ritz vectors approach the leading eigenvectors: the rest of
    # the spectrum is below 0.5, so each iteration shrinks the angle by <= 1/6
    w, V = np.linalg.eigh(A)
    V = V[:, ::-1]
    _, P6 = oracle.topk_ritz_vectors(A, Om, 6)
    for i in range(10):
        assert abs(abs(P6[:, i] @ V[:, i]) - 1.0) <= 1e-10, i


def test_project_weight_pins():
    rng = np.random.default_rng(41)
    d, k = 40, 7
    W = rng.standard_normal((d, d))
    # the first k unit vectors: W' is the leading k x k block, X the first k columns
    E = np.eye(d)[:, :k]
    Wp, X = oracle.project_weight(W, E)
    assert np.array_equal(Wp, W[:k, :k]) and np.array_equal(X, W[:, :k])
    # brute force on a tiny case: W'_ab = sum_ij P_ia W_ij P_jb
    P = rng.standard_normal((d, k))
    Wp, X = oracle.project_weight(W, P)
    bf = np.zeros((k, k))
    for a in range(k):
        for b in range(k):
            bf[a, b] = sum(P[i, a] * W[i, j] * P[j, b] for i in range(d) for j in range(d))
    assert np.max(np.abs(Wp - bf)) <= 1e-11 * np.max(np.abs(bf))
    # a non-symmetric W keeps its orientation: (P^T W P)^T = P^T W^T P
    Wt, _ = oracle.project_weight(W.T.copy(), P)
    assert np.allclose(Wt, Wp.T, rtol=0, atol=1e-12 * np.max(np.abs(Wp)))
    # symmetric W = Q diag(s) Q^T on its own leading eigenvectors: W' = diag(s_1..s_k)
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    s = np.sort(rng.uniform(0.1, 5.0, d))[::-1]
    Wp, _ = oracle.project_weight((Q * s) @ Q.T, Q[:, :k])
    assert np.max(np.abs(Wp - np.diag(s[:k]))) <= 1e-12 * s[0]
    # Eckart-Young: with the k leading right singular vectors, ||W P||_F^2 is the
    # sum of the k largest sigma^2 and ||W - W P P^T||_F^2 the sum of the rest,
    # the least error of any rank-k approximation
    U, sig, Vt = np.linalg.svd(W)
    _, X = oracle.project_weight(W, Vt[:k].T)
    assert abs(np.sum(X ** 2) - np.sum(sig[:k] ** 2)) <= 1e-11 * np.sum(sig ** 2)
    assert abs(np.sum((W - X @ Vt[:k]) ** 2) - np.sum(sig[k:] ** 2)) <= 1e-11 * np.sum(sig ** 2)
    # bf16 bit patterns are widened exactly
    Wb = (rng.standard_normal((d, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    Wf = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(oracle.project_weight(Wb, P)[0], oracle.project_weight(Wf, P)[0])


# ------------------------------------------------------------- P3 at the full sizes

def test_swiftsvd_golden_vs_lapack():
    """The stored oracle spectrum of the 4096 Swift-SVD covariance (the values the
    GPU parity test compares with) against LAPACK's eigvalsh of the same fp64
    matrix, rebuilt here chunk by chunk with the oracle's covariance."""
    import json
    import os
    z = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "swiftsvd.npz"))
    d = 4096
    acc = np.zeros((d, d))
    hashes = []
    for k in range(32):
        X = synth.swiftsvd_chunk(k)
        hashes.append(synth.sha256(X))
        acc = oracle.covariance(X, "bf16", 1.0, C0=acc, beta=1.0)
    assert ",".join(hashes) == str(z["sha256"])
    assert abs(np.trace(acc) - float(z["trace"])) <= 1e-13 * float(z["trace"])
    ref = np.linalg.eigvalsh(acc)[::-1]
    eig = z["eig"]
    assert np.max(np.abs(eig - ref)) <= 1e-12 * ref[0]
    assert json.loads(str(z["desc_json"]))["S"] == pytest.approx(float(np.sum(ref)), rel=1e-12)


@pytest.mark.skipif(not os.environ.get("SPEC_HEAVY_PINS"),
                    reason="minutes of CPU and ~6 GB of memory; set SPEC_HEAVY_PINS=1 to run")
def test_ffn_golden_vs_lapack():
    """The stored oracle spectrum of the 14336 FFN covariance against LAPACK's
    eigvalsh of the same fp64 matrix (C = X^T X / 65536 of the regenerated input)."""
    z = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ffn.npz"))
    X = synth.ffn()
    assert synth.sha256(X) == str(z["sha256"])
    C = oracle.covariance(X, "bf16", 1.0 / 65536)
    del X
    ref = np.linalg.eigvalsh(C)[::-1]
    assert np.max(np.abs(z["eig"] - ref)) <= 1e-12 * ref[0]
    assert int(z["n_above_inertia"]) == int(np.sum(ref > oracle.mp_edges(1.0, 14336 / 65536)[1]))



# ------------------------------------------------------------- S3 tail-pair screen

def test_tail_pair_screen_pins():
    # U = V = I: u_i^T v_j is the Kronecker delta, so every same-head pair but
    # i = j is kept; the head blocks of the tail [3687, 4096) with head_dim 128
    # have 25, 128, 128 and 128 indices
    N = 4096
    eye = np.eye(N, dtype=np.float32)
    absdot, keep, count = oracle.tail_pair_screen(eye, eye, i0=3687, t=409, head_dim=128)
    assert np.array_equal(absdot, np.eye(409))
    assert count == sum(b * b - b for b in (25, 128, 128, 128))
    assert not keep[0, 30]  # index 3687 (head 28) and 3717 (head 29)
    # brute force on a tiny case
    rng = np.random.default_rng(3)
    U = rng.standard_normal((12, 10)).astype(np.float32)
    V = rng.standard_normal((12, 10)).astype(np.float32)
    absdot, keep, count = oracle.tail_pair_screen(U, V, i0=4, t=6, head_dim=3, eps=1.5)
    for a in range(6):
        for b in range(6):
            i, j = 4 + a, 4 + b
            dot = sum(float(U[k, i]) * float(V[k, j]) for k in range(12))
            assert abs(absdot[a, b] - abs(dot)) <= 1e-12 * (1 + abs(dot))
            assert keep[a, b] == ((i // 3 == j // 3) and abs(dot) < 1.5)
    assert count == int(keep.sum())
    # a planted pair: V = U R with R a rotation by theta in the plane of columns
    # (p, q) gives u_p^T v_q = -sin(theta) and u_q^T v_q = cos(theta); strict
    # threshold on both sides of eps
    Q, _ = np.linalg.qr(rng.standard_normal((64, 64)))
    for theta, kept in [(0.0149, True), (0.0151, False)]:
        R = np.eye(64)
        p, q = 60, 62
        R[p, p] = R[q, q] = np.cos(theta)
        R[p, q], R[q, p] = -np.sin(theta), np.sin(theta)
        absdot, keep, _ = oracle.tail_pair_screen(Q, Q @ R, i0=58, t=6, head_dim=8)
        assert abs(absdot[p - 58, q - 58] - np.sin(theta)) <= 1e-14
        assert keep[p - 58, q - 58] == kept
    # Haar-orthogonal U, V of the S3 workload: u_i^T v_j is about N(0, 1/N), so
    # the kept fraction of same-head pairs is close to P(|Z| < 0.015 sqrt(N))
    U, _ = np.linalg.qr(rng.standard_normal((1024, 1024)))
    V, _ = np.linalg.qr(rng.standard_normal((1024, 1024)))
    absdot, keep, count = oracle.tail_pair_screen(U, V, i0=922, t=102, head_dim=1024)
    import scipy.stats
    frac = count / 102 ** 2
    assert abs(frac - (2 * scipy.stats.norm.cdf(0.015 * 32) - 1)) < 0.03
