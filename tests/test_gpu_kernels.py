"""GPU parity of each hot-path kernel against the fp64 oracle on seeded inputs.

Every call goes through the C ABI (libspec.so via the ctypes binding).  Sizes
span several tiles and a ragged tail; tolerances are derived from the
arithmetic (worst-case rounding bounds) or taken from the spec contract
(eigenvalues within 1e-4 lambda_max, descriptors within 1e-4 relative, counts
exact).
"""
import math

import numpy as np
import pytest

import oracle
from gpu_util import (DESC_FLOAT_FIELDS, DESC_INT_FIELDS, EPS32, EPS64, dev, dev_bf16, print_case,
                      syrk_bound)
from gen import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spec():
    import torch
    import weights_bf16_fp32_amd as spec
    assert torch.cuda.is_available()
    spec.lib()
    return spec


def _torch():
    import torch
    return torch


# ----------------------------------------------------------------- A1 SYRK

@pytest.mark.parametrize("n,d", [(1, 8), (64, 32), (130, 136), (257, 256), (1000, 520), (50, 37), (3, 300)])
def test_syrk_bf16(spec, n, d):
    torch = _torch()
    print_case("syrk_bf16", n=n, d=d)
    rng = np.random.default_rng(n * 7 + d)
    bits = synth.f32_to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32) * 3)
    X = dev_bf16(bits)
    C = torch.full((d, d), float("nan"), dtype=torch.float32, device="cuda")
    alpha = 1.0 / max(n, 1)
    spec.cov_accumulate(X, C, alpha=alpha, beta=0.0)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy().astype(np.float64)
    ref = oracle.covariance(bits, "bf16", alpha)
    bound = syrk_bound(np.abs(oracle.widen(bits, "bf16")), alpha, EPS32)
    L = np.tril_indices(d)
    assert np.all(np.abs(Cg[L] - ref[L]) <= bound[L])
    U = np.triu_indices(d, 1)
    assert np.all(np.isnan(Cg[U]))  # the strict upper triangle is never written


@pytest.mark.parametrize("ldx", [(1 << 24) - 8, 1 << 24, (1 << 24) + 64])
def test_syrk_bf16_huge_row_stride(spec, ldx):
    """Row strides at and beyond what the MFMA kernel's 32-bit buffer offsets
    reach (64 samples x ldx x 2 bytes): the larger ones take the general kernel;
    every one gives the oracle's covariance."""
    torch = _torch()
    n, d = 70, 64
    print_case("syrk_bf16_huge_ldx", n=n, d=d, ldx=ldx)
    rng = np.random.default_rng(ldx % 1000)
    bits = synth.f32_to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32))
    flat = torch.zeros(((n - 1) * ldx + d,), dtype=torch.bfloat16, device="cuda")
    X = torch.as_strided(flat, (n, d), (ldx, 1))
    X.copy_(dev_bf16(bits))
    C = torch.full((d, d), float("nan"), dtype=torch.float32, device="cuda")
    spec.cov_accumulate(X, C, alpha=1.0 / n, beta=0.0)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy().astype(np.float64)
    ref = oracle.covariance(bits, "bf16", 1.0 / n)
    bound = syrk_bound(np.abs(oracle.widen(bits, "bf16")), 1.0 / n, EPS32)
    L = np.tril_indices(d)
    assert np.all(np.abs(Cg[L] - ref[L]) <= bound[L])
    del flat, X


@pytest.mark.parametrize("n,d,beta", [(300, 5888, 0.0), (97, 6000, 0.0), (64, 6000, 1.0),
                                      (300, 4096, 0.0), (97, 4000, 0.0), (64, 5632, 1.0), (12288, 4096, 1.0)])
def test_syrk_bf16_large_d(spec, n, d, beta):
    """d large enough for the 256 x 256 tile kernel (at least 128 tiles): a
    ragged d (6000 = 23 full tiles + 112, 4000 = 15 + 160), fewer tiles than
    CUs (d = 4096: 136 tiles; 5632: 253), 12288 samples at d = 4096 so that
    every tile is split three ways along the samples (C scaled by beta first,
    the partial products added atomically), a sample count that is not a
    multiple of the 32-sample step, and beta = 1 on a random old C; every
    lower-triangle entry against the oracle within the (n + 2) u bound, the
    strict upper triangle untouched."""
    torch = _torch()
    print_case("syrk_bf16_large_d", n=n, d=d, beta=beta)
    rng = np.random.default_rng(n + d)
    bits = synth.f32_to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32) * 2)
    X = dev_bf16(bits)
    C0 = rng.standard_normal((d, d)).astype(np.float32) if beta else None
    C = torch.from_numpy(C0).cuda() if beta else torch.full((d, d), float("nan"), dtype=torch.float32, device="cuda")
    if beta:
        up = torch.triu(torch.ones((d, d), dtype=torch.bool, device="cuda"), 1)
        C[up] = float("nan")
    alpha = 1.0 / n
    spec.cov_accumulate(X, C, alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy().astype(np.float64)
    del C
    ref = oracle.covariance(bits, "bf16", alpha, C0=C0, beta=beta)
    bound = syrk_bound(np.abs(oracle.widen(bits, "bf16")), alpha, EPS32,
                       C0abs=np.abs(C0.astype(np.float64)) if beta else None, beta=beta)
    L = np.tril_indices(d)
    assert np.all(np.abs(Cg[L] - ref[L]) <= bound[L])
    U = np.triu_indices(d, 1)
    assert np.all(np.isnan(Cg[U]))


def test_syrk_bf16_accumulate(spec):
    torch = _torch()
    print_case("syrk_bf16_accumulate")
    d = 264
    chunks = [synth.f32_to_bf16_bits(np.random.default_rng(k).standard_t(4, (300 + 17 * k, d)).astype(np.float32))
              for k in range(3)]
    C = torch.empty((d, d), dtype=torch.float32, device="cuda")
    ref = np.zeros((d, d))
    absacc = np.zeros((d, d))
    for k, b in enumerate(chunks):
        spec.cov_accumulate(dev_bf16(b), C, alpha=1.0, beta=0.0 if k == 0 else 1.0)
        ref = oracle.covariance(b, "bf16", 1.0, C0=ref, beta=1.0)
        absacc += syrk_bound(np.abs(oracle.widen(b, "bf16")), 1.0, EPS32) + (EPS32 * 2) * np.abs(ref)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy().astype(np.float64)
    L = np.tril_indices(d)
    assert np.all(np.abs(Cg[L] - ref[L]) <= absacc[L])


def test_syrk_empty_rows_scales(spec):
    torch = _torch()
    d = 40
    C = torch.ones((d, d), dtype=torch.float32, device="cuda") * 3.0
    X = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    spec.cov_accumulate(X, C, alpha=1.0, beta=0.5)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy()
    assert np.all(np.tril(Cg) == np.tril(np.full((d, d), 1.5, np.float32)))
    assert np.all(np.triu(Cg, 1) == np.triu(np.full((d, d), 3.0, np.float32), 1))


def test_syrk_f32_tiny_config(spec):
    torch = _torch()
    X = synth.tiny()
    C = torch.zeros((32, 32), dtype=torch.float32, device="cuda")
    spec.cov_accumulate(dev(X), C, alpha=1.0 / 64, beta=0.0)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy().astype(np.float64)
    ref = oracle.covariance(X, "f32", 1.0 / 64)
    bound = syrk_bound(np.abs(X.astype(np.float64)), 1.0 / 64, EPS32)
    L = np.tril_indices(32)
    assert np.all(np.abs(Cg[L] - ref[L]) <= bound[L])


@pytest.mark.parametrize("n,d", [(100, 128), (37, 260), (33, 30), (5, 4)])
def test_syrk_f32_to_f64(spec, n, d):
    torch = _torch()
    print_case("syrk_f64", n=n, d=d)
    rng = np.random.default_rng(n + d)
    X = (rng.standard_normal((n, d)) * 10.0 ** rng.uniform(-3, 3, (n, d))).astype(np.float32)
    C = torch.zeros((d, d), dtype=torch.float64, device="cuda")
    spec.cov_accumulate(dev(X), C, alpha=1.0, beta=0.0)
    torch.cuda.synchronize()
    Cg = C.cpu().numpy()
    ref = oracle.covariance(X, "f32", 1.0)
    bound = syrk_bound(np.abs(X.astype(np.float64)), 1.0, EPS64)
    L = np.tril_indices(d)
    assert np.all(np.abs(Cg[L] - ref[L]) <= bound[L])


# ----------------------------------------------------------------- A2 window Gram

@pytest.mark.parametrize("S,T,d,N", [(3, 200, 256, 30), (2, 130, 136, 30), (1, 40, 64, 1),
                                     (2, 100, 128, 40), (1, 64, 64, 64), (2, 77, 40, 30)])
def test_gram_band_bf16(spec, S, T, d, N):
    torch = _torch()
    print_case("gram_band", S=S, T=T, d=d, N=N)
    H = synth.eigentrack(streams=S, T=T, d=d)
    out = spec.gram_window(dev_bf16(H), N=N)
    torch.cuda.synchronize()
    Bg = out.cpu().numpy().astype(np.float64)
    ref = oracle.band_gram(H, "bf16", N)
    h = np.abs(oracle.widen(H, "bf16"))
    for s in range(S):
        for j in range(N):
            bound = (d + 2) * EPS32 * np.concatenate(
                [np.zeros(j), np.einsum("td,td->t", h[s, j:], h[s, :T - j])]) + 1e-30
            assert np.all(np.abs(Bg[s, :, j] - ref[s, :, j]) <= bound), (s, j)


def test_gram_band_f32_and_dense(spec):
    torch = _torch()
    rng = np.random.default_rng(4)
    S, T, d, N = 2, 50, 33, 30
    Hf = rng.standard_normal((S, T, d)).astype(np.float32)
    out = spec.gram_window(dev(Hf), N=N)
    dense = spec.gram_window(dev(Hf), N=N, stride=3, scale=1.0 / N, layout=spec.GRAM_DENSE)
    torch.cuda.synchronize()
    ref = oracle.band_gram(Hf, "f32", N)
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= (d + 2) * EPS32 * d * 20
    W = (T - N) // 3 + 1
    Dg = dense.cpu().numpy().reshape(S, W, N, N)
    for s in range(S):
        G = oracle.window_gram(Hf[s], "f32", N, stride=3)
        assert np.max(np.abs(Dg[s] - G)) <= (d + 2) * EPS32 * np.max(np.abs(G)) * 4


# ----------------------------------------------------------------- A3 batched small eigenvalues

def _rand_sym_batch(rng, batch, n):
    A = rng.standard_normal((batch, n, n))
    return ((A + A.transpose(0, 2, 1)) * 0.5).astype(np.float32)


@pytest.mark.parametrize("n", [1, 2, 5, 30, 31, 32, 33, 64])
def test_batched_eig_dense(spec, n):
    torch = _torch()
    print_case("batched_eig_dense", n=n)
    rng = np.random.default_rng(100 + n)
    batch = 17
    A = _rand_sym_batch(rng, batch, n)
    A[0] = 0.0
    A[1] = np.eye(n, dtype=np.float32)
    if n > 2:
        Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
        lam = np.repeat([3.0, -1.0, 0.5], (n + 2) // 3)[:n]
        A[2] = ((Q * lam) @ Q.T).astype(np.float32)
    # garbage in the strict upper triangle must be ignored
    Au = A.copy()
    iu = np.triu_indices(n, 1)
    Au[:, iu[0], iu[1]] = 1e30
    w, info = spec.eigvalsh_batched_dense(dev(Au))
    torch.cuda.synchronize()
    wg = w.cpu().numpy().astype(np.float64)
    ref, _ = oracle.eigvalsh_small(A.astype(np.float64))
    for b in range(batch):
        lmax = max(np.max(np.abs(ref[b])), 1e-30)
        assert np.max(np.abs(wg[b] - ref[b])) <= 1e-5 * lmax, b
    assert np.all(np.diff(wg, axis=1) <= 0)
    assert np.all(info.cpu().numpy() >= 0)


@pytest.mark.parametrize("n", [30, 40])
def test_batched_eig_flags_non_finite(spec, n):
    """A matrix with a NaN or inf entry gets info -1 and NaN eigenvalues; the
    other matrices of the batch are unaffected."""
    torch = _torch()
    print_case("batched_eig_non_finite", n=n)
    rng = np.random.default_rng(5 + n)
    A = _rand_sym_batch(rng, 4, n)
    A[1, 3, 2] = np.nan
    A[2, n - 1, 0] = np.inf
    w, info = spec.eigvalsh_batched_dense(dev(A))
    torch.cuda.synchronize()
    inf_ = info.cpu().numpy()
    wg = w.cpu().numpy().astype(np.float64)
    assert inf_[1] == -1 and inf_[2] == -1 and inf_[0] >= 0 and inf_[3] >= 0
    assert np.all(np.isnan(wg[1])) and np.all(np.isnan(wg[2]))
    ref, _ = oracle.eigvalsh_small(A[[0, 3]].astype(np.float64))
    assert np.max(np.abs(wg[[0, 3]] - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_batched_eig_clustered_and_graded(spec):
    """Clustered eigenvalues (a 10-fold one and pairs 1e-6 apart) and a graded
    spectrum over 8 decades, n = 30: every eigenvalue within 1e-5 lambda_max
    and the output non-increasing."""
    torch = _torch()
    n = 30
    rng = np.random.default_rng(77)
    lam = np.concatenate([np.full(10, 2.0), 1.0 + 1e-6 * np.arange(10), 10.0 ** -np.arange(10)])
    A = np.empty((3, n, n), dtype=np.float32)
    for b in range(3):
        Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
        A[b] = ((Q * (lam if b < 2 else 10.0 ** -np.linspace(0, 8, n))) @ Q.T).astype(np.float32)
    w, info = spec.eigvalsh_batched_dense(dev(A))
    torch.cuda.synchronize()
    wg = w.cpu().numpy().astype(np.float64)
    ref, _ = oracle.eigvalsh_small(A.astype(np.float64))
    for b in range(3):
        assert np.max(np.abs(wg[b] - ref[b])) <= 1e-5 * np.max(np.abs(ref[b])), b
    assert np.all(np.diff(wg, axis=1) <= 0)


def test_batched_eig_band_windows(spec):
    torch = _torch()
    S, T, d, N = 3, 90, 512, 30
    print_case("batched_eig_band", S=S, T=T, d=d, N=N)
    H = synth.eigentrack(streams=S, T=T, d=d)
    band = spec.gram_window(dev_bf16(H), N=N)
    w, info = spec.eigvalsh_batched_band(band, n=N, scale=1.0 / N)
    torch.cuda.synchronize()
    W = T - N + 1
    wg = w.cpu().numpy().astype(np.float64).reshape(S, W, N)
    bandg = band.cpu().numpy().astype(np.float64)
    for s in range(S):
        # the same fp32 band values, assembled and solved in fp64 by the oracle
        G = np.empty((W, N, N))
        for win in range(W):
            for i in range(N):
                for j in range(N):
                    G[win, i, j] = np.float32(np.float32(1.0 / N) * np.float32(bandg[s, win + max(i, j), abs(i - j)]))
        ref, _ = oracle.eigvalsh_small(G)
        assert np.max(np.abs(wg[s] - ref)) <= 1e-5 * np.max(ref)
        # and against the oracle's own window Grams from H (spec bound)
        ref2, _ = oracle.eigvalsh_small(oracle.window_gram(H[s], "bf16", N))
        assert np.max(np.abs(wg[s] - ref2)) <= 1e-4 * np.max(ref2)
    assert np.all(info.cpu().numpy() >= 0)


# ----------------------------------------------------------------- A5 descriptors

def _cmp_desc(g, o, rel=1e-4, fields=None):
    for f in (fields or DESC_FLOAT_FIELDS):
        a, b = float(g[f]), float(o[f])
        if math.isnan(b):
            assert math.isnan(a), f
        else:
            assert abs(a - b) <= rel * max(abs(b), 1e-300), (f, a, b)
    for f in DESC_INT_FIELDS:
        assert int(g[f]) == int(o[f]), (f, g[f], o[f])


@pytest.mark.parametrize("mode", ["eig", "companion", "singular", "median", "mean"])
def test_descriptors_on_oracle_spectra(spec, mode):
    torch = _torch()
    rng = np.random.default_rng(9)
    if mode == "companion":
        n, p, r = 30, 4096, 30
        spectra = [np.sort(p / n * oracle.mp_quantiles(1.0, n / p, r) * rng.uniform(0.9, 1.1, r))[::-1]
                   for _ in range(5)]
    elif mode == "singular":
        n = p = r = 512
        spectra = [synth.s3_sigma(512) ** 2]
    else:
        n, p, r = 200, 50, 50
        spectra = [np.sort(rng.gamma(2.0, 0.5, r))[::-1] for _ in range(4)]
        spectra.append(np.concatenate([[9.0, 5.0], np.zeros(r - 2)]))
    sm = {"median": 1, "mean": 2}.get(mode, 0)
    kw = dict(n_samples=n, p_dim=p, k=3, sigma2=1.3, sigma2_mode=sm, top_frac=0.2, small_rel=1e-2,
              tail_frac=0.7)
    Wt = np.array(spectra)
    got = spec.descriptors(dev(Wt), **kw)
    got32 = spec.descriptors(dev(Wt.astype(np.float32)), **kw)
    for b in range(len(spectra)):
        ref = oracle.descriptors(Wt[b], **kw)
        _cmp_desc(got[b], ref, rel=1e-10)
        ref32 = oracle.descriptors(Wt[b].astype(np.float32).astype(np.float64), **kw)
        _cmp_desc(got32[b], ref32, rel=1e-10)


def test_descriptors_flags(spec):
    W = np.array([[3.0, 2.0, 0.0, 0.0], [np.nan, 1.0, 0.5, 0.1], [0.0, 0.0, 0.0, -1e-9]])
    got = spec.descriptors(dev(W), n_samples=10, p_dim=4, k=2)
    assert got[0]["flags"] & spec.FLAG_GK_UNDEF and math.isnan(got[0]["gk"])
    assert got[1]["flags"] & spec.FLAG_NONFINITE
    assert got[2]["flags"] & spec.FLAG_S_ZERO and math.isnan(got[2]["H"])


# ----------------------------------------------------------------- tiny config end to end

def test_tiny_config_end_to_end(spec):
    torch = _torch()
    print_case("tiny_end_to_end")
    X = synth.tiny()
    C = torch.zeros((32, 32), dtype=torch.float32, device="cuda")
    spec.cov_accumulate(dev(X), C, alpha=1.0 / 64, beta=0.0)
    w, info = spec.eigvalsh_batched_dense(C)
    got = spec.descriptors(w, n_samples=64, p_dim=32, k=1)[0]
    wg = w.cpu().numpy()[0].astype(np.float64)
    Cref = oracle.covariance(X, "f32", 1.0 / 64)
    wref, _ = oracle.eigvalsh_small(Cref)
    err = np.max(np.abs(wg - wref))
    assert err <= 1e-4 * wref[0]
    ref = oracle.descriptors(wref, n_samples=64, p_dim=32, k=1)
    margin = np.min(np.abs(wref - ref["lambda_plus"]))
    assert margin > 4 * err  # the exact count is well posed
    _cmp_desc(got, ref, rel=1e-4)
    assert ref["n_above"] == 2
