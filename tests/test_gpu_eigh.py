"""GPU parity of the eigenvector path (spec_eigh_large) against the fp64 oracle.

Each returned column z_j is checked three ways against the oracle's
eigendecomposition of the same input:
  * residual  max_j |A z_j - w_j z_j|_2 <= tol_r ||A||;
  * orthogonality  max |Z^T Z - I| <= tol_o;
  * direction, by the Davis-Kahan sin-theta bound: with rho = z^T A z and
    r = A z - rho z, the angle from z to the true eigenvector is at most
    |r|_2 / delta_j (delta_j the distance from rho to the other eigenvalues),
    and likewise for the oracle's u_j with its own residual; the test asks the
    angle between z_j and u_j for at most twice the sum (plus 1e-13), for
    every column whose delta_j is positive.
Eigenvalues: the large-solver bounds (1e-4 lambda_max for f32 inputs, 1e-10
for f64).  Tolerances: f64 residual 1e-11 ||A||, orthogonality 1e-10 (the
reduction and the back-transformation run in fp64, the inverse iteration in
fp64 with clusters below 1e-9 ||T|| orthogonalised); f32 residual 5e-5 ||A||
and orthogonality 5e-5 (fp32 reductions over n <= 4096 rows: a few sqrt(n)
eps_32).  Sizes span the direct and CholeskyQR panel paths, ragged last
panels, and the degenerate inputs: n < 3, k = 1 and k = n, repeated
eigenvalues, rank-deficient covariances, the zero and scaled identity
matrices (whose tridiagonals split into 1 x 1 blocks).
"""
import numpy as np
import pytest

import oracle
from gpu_util import dev, print_case

pytestmark = pytest.mark.gpu

TOL = {np.float32: (5e-5, 5e-5, 1e-4), np.float64: (1e-11, 1e-10, 1e-10)}


@pytest.fixture(scope="module")
def spec():
    import weights_bf16_fp32_amd as spec
    spec.lib()
    return spec


def _sym(rng, n):
    G = rng.standard_normal((n, n))
    return (G + G.T) / 2


def _planted(rng, vals):
    n = len(vals)
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    A = (Q * np.asarray(vals, dtype=np.float64)) @ Q.T
    return (A + A.T) / 2


def _run(spec, A, dtype, k):
    import torch
    Ad = dev(A.astype(dtype))
    info = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    w, Z = spec.eigh_large(Ad, k, info=info)
    torch.cuda.synchronize()
    return (w.cpu().numpy().astype(np.float64), Z.cpu().numpy().astype(np.float64),
            int(info.cpu().numpy()[0]))


def _check(spec, A, dtype, k, name, cols=None):
    """Run, then check eigenvalues, residual, orthogonality and directions;
    cols restricts the per-column checks to a sample (large n)."""
    n = A.shape[0]
    A = A.astype(dtype).astype(np.float64)  # the matrix the solver sees
    w, Z, info = _run(spec, A, dtype, k)
    wr, Ur = oracle.eigh_vectors(A, n)
    tol_r, tol_o, tol_w = TOL[dtype]
    normA = max(np.max(np.abs(wr)), 1e-300)
    assert info == 0
    assert Z.shape == (n, k) and np.all(np.isfinite(Z))
    assert np.max(np.abs(w - wr)) <= tol_w * normA
    J = np.arange(k) if cols is None else np.asarray(cols)
    Zs = Z[:, J]
    zn = np.linalg.norm(Zs, axis=0)
    R = A @ Zs - Zs * w[J]
    res = np.max(np.linalg.norm(R, axis=0)) / normA
    G = Zs.T @ Zs
    orth = np.max(np.abs(G - np.eye(len(J))))
    # Davis-Kahan on the normalised columns: sin(theta) to the true u_j is at
    # most |r|/delta for z and for the oracle's u_j alike, so the angle between
    # them at most the sum; sin(theta) measured as |z - (u^T z) u| (accurate
    # to rounding, unlike sqrt(1 - (u^T z)^2))
    Zu = Zs / np.maximum(zn, 1e-300)
    rho = np.einsum("ij,ij->j", Zu, A @ Zu)
    r = np.linalg.norm(A @ Zu - Zu * rho, axis=0)
    Uj = Ur[:, J]
    ru = np.linalg.norm(A @ Uj - Uj * wr[J], axis=0)
    cu = np.einsum("ij,ij->j", Uj, Zu)
    sin_t = np.linalg.norm(Zu - Uj * cu, axis=0)
    worst_dk = 0.0
    for t, j in enumerate(J):
        others = np.delete(wr, j)
        delta = np.min(np.abs(others - rho[t])) if others.size else np.inf
        if delta > 0:
            bound = 2.0 * (r[t] + ru[t]) / delta + 1e-13
            worst_dk = max(worst_dk, sin_t[t] / bound)
    print(f"[eigh] {name}: n={n} k={k} residual {res:.2e} orth {orth:.2e} "
          f"max |dw|/|A| {np.max(np.abs(w - wr)) / normA:.2e} sin-theta/bound {worst_dk:.2f}", flush=True)
    assert res <= tol_r
    assert orth <= tol_o
    assert worst_dk <= 1.0
    return w, Z


@pytest.mark.parametrize("n", [1, 2, 3, 20, 33, 100, 257, 600, 1000])
def test_eigh_f64_random(spec, n):
    print_case("eigh_f64_random", n=n)
    rng = np.random.default_rng(3000 + n)
    _check(spec, _sym(rng, n), np.float64, n, "f64 random")


@pytest.mark.parametrize("n", [2, 20, 100, 600, 1000, 1100])
def test_eigh_f32_random(spec, n):
    print_case("eigh_f32_random", n=n)
    rng = np.random.default_rng(4000 + n)
    _check(spec, _sym(rng, n), np.float32, n, "f32 random")


@pytest.mark.parametrize("dtype,k", [(np.float64, 1), (np.float64, 37), (np.float32, 1), (np.float32, 250)])
def test_eigh_partial_k(spec, dtype, k):
    """The k largest only: the columns belong to w[0 .. k-1], in order."""
    print_case("eigh_partial", dtype=dtype.__name__, k=k)
    rng = np.random.default_rng(5000 + k)
    _check(spec, _sym(rng, 700), dtype, k, f"partial k={k}")


def test_eigh_covariance(spec):
    """An activation covariance (positive semi-definite, decaying spectrum)."""
    print_case("eigh_covariance")
    rng = np.random.default_rng(61)
    X = rng.standard_normal((2000, 512)) * (1.0 / np.sqrt(1.0 + np.arange(512)))
    C = X.T @ X / 2000
    _check(spec, C, np.float32, 410, "f32 covariance")
    _check(spec, C, np.float64, 512, "f64 covariance")


def test_eigh_repeated_eigenvalues(spec):
    """Multiplicities 8 and 5 and a pair: the cluster path (orthogonalised
    within the cluster)."""
    print_case("eigh_repeated")
    rng = np.random.default_rng(71)
    n = 300
    vals = np.concatenate([np.full(8, 3.0), np.full(5, -1.0), [0.5, 0.5], rng.uniform(-2, 2, n - 15)])
    A = _planted(rng, vals)
    _check(spec, A, np.float64, n, "f64 repeated")
    _check(spec, A, np.float32, n, "f32 repeated")


def test_eigh_rank_deficient(spec):
    """Rank 100 covariances of 512 dimensions: 412 eigenvalues at zero."""
    print_case("eigh_rank_deficient")
    rng = np.random.default_rng(81)
    X = rng.standard_normal((100, 512))
    C = X.T @ X / 100
    _check(spec, C, np.float64, 512, "f64 rank 100")
    _check(spec, C, np.float32, 512, "f32 rank 100")


def test_eigh_zero_and_identity(spec):
    print_case("eigh_zero_identity")
    for n, c in [(200, 0.0), (150, 3.0)]:
        for dtype in (np.float32, np.float64):
            _check(spec, c * np.eye(n), dtype, n, f"{c} I")


def test_eigh_values_match_eigenvalue_solver(spec):
    """Keeping the reduction changes nothing the eigenvalues depend on: the
    same input through spec_eigvalsh_large gives the same w."""
    import torch
    print_case("eigh_vs_eigvalsh")
    rng = np.random.default_rng(91)
    for dtype, n in [(np.float32, 1500), (np.float64, 700)]:
        A = _sym(rng, n).astype(dtype)
        w1, _ = spec.eigh_large(dev(A), 16)
        w2 = spec.eigvalsh_large(dev(A))
        torch.cuda.synchronize()
        d = np.max(np.abs(w1.cpu().numpy().astype(np.float64) - w2.cpu().numpy()))
        print(f"[eigh] {dtype.__name__} n={n}: max |w_eigh - w_eigvalsh| = {d:.3g}", flush=True)
        assert d == 0.0


def test_eigh_swift_svd_shape(spec):
    """The Swift-SVD keep set at d = 4096 (keep ratio 0.8: k = 3276) on a
    covariance of that size, f32; residual and directions on a sample of 192
    columns spread over the kept range, orthogonality of the same sample."""
    print_case("eigh_4096")
    rng = np.random.default_rng(101)
    d = 4096
    X = rng.standard_normal((6144, d)).astype(np.float32) * (1.0 / np.sqrt(1.0 + np.arange(d) / 64)).astype(np.float32)
    C = (X.T.astype(np.float64) @ X.astype(np.float64)) / 6144
    cols = np.unique(np.linspace(0, 3275, 192).astype(int))
    _check(spec, C, np.float32, 3276, "f32 d=4096 k=3276", cols=cols)


def test_eigh_max_size(spec):
    """n = 8192, the vector path's limit (f32, k = 512): all eigenvalues against
    LAPACK's fp64 eigvalsh of the same matrix; residual and orthogonality on
    128 sampled columns (the full oracle decomposition would take minutes)."""
    import torch
    print_case("eigh_8192")
    rng = np.random.default_rng(111)
    d, k = 8192, 512
    X = rng.standard_normal((2048, d)).astype(np.float32) * (1.0 / np.sqrt(1.0 + np.arange(d) / 128)).astype(np.float32)
    A = ((X.T.astype(np.float64) @ X.astype(np.float64)) / 2048).astype(np.float32)
    w, Z, info = _run(spec, A.astype(np.float64), np.float32, k)
    A64 = A.astype(np.float64)
    wr = np.linalg.eigvalsh(A64)[::-1]
    normA = np.max(np.abs(wr))
    cols = np.unique(np.linspace(0, k - 1, 128).astype(int))
    Zs = Z[:, cols]
    res = np.max(np.linalg.norm(A64 @ Zs - Zs * w[cols], axis=0)) / normA
    orth = np.max(np.abs(Zs.T @ Zs - np.eye(len(cols))))
    werr = np.max(np.abs(w - wr)) / normA
    print(f"[eigh] f32 n=8192 k=512: residual {res:.2e} orth {orth:.2e} max |dw|/|A| {werr:.2e}", flush=True)
    assert info == 0 and np.all(np.isfinite(Z))
    assert werr <= 1e-4 and res <= 5e-5 and orth <= 5e-5
