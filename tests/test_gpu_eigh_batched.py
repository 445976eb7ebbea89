"""GPU parity of the batched eigenpairs (spec_eigh_batched, parallel Jacobi
with accumulated rotations) against the fp64 oracle.

Per matrix, against the oracle's eigendecomposition of the same fp32 input:
eigenvalues within 5e-6 ||A|| (n eps_32 of rounding over the rotations); residual
max_j |A v_j - w_j v_j|_2 <= 3e-5 ||A|| (the stopping threshold leaves
off-diagonal entries up to 2e-6 sqrt(|a_pp a_qq|), sqrt(n) of them per
column); orthogonality max |V^T V - I| <= 3e-5 (fp32 rotations); the
Davis-Kahan angle to the oracle's vector at most twice the bound from both
residuals (plus 1e-6, the fp32 rounding of the output), for every column
whose eigenvalue is separated.  Cases: random symmetric matrices of order 1
to 32, EigenTrack windows from the GPU band Gram (and the direct eigenvalue
solver's values on the same windows), rank-deficient windows (repeated
steps), planted repeated eigenvalues, the zero and identity matrices, and a
matrix with a NaN entry.
"""
import numpy as np
import pytest

import oracle
from gpu_util import dev, dev_bf16, print_case
from gen import synth

pytestmark = pytest.mark.gpu

TOL_W, TOL_R, TOL_O = 5e-6, 3e-5, 3e-5


@pytest.fixture(scope="module")
def spec():
    import weights_bf16_fp32_amd as spec
    spec.lib()
    return spec


def _check_one(A, w, V, name):
    """A fp64 (the solver's fp32 input), w [n], V [n, n] from the GPU."""
    n = A.shape[0]
    wr, Ur = oracle.eigh_vectors(A, n)
    normA = max(np.max(np.abs(wr)), 1e-300)
    werr = np.max(np.abs(w - wr)) / normA
    res = np.max(np.linalg.norm(A @ V - V * w, axis=0)) / normA
    orth = np.max(np.abs(V.T @ V - np.eye(n)))
    Vu = V / np.maximum(np.linalg.norm(V, axis=0), 1e-300)
    rho = np.einsum("ij,ij->j", Vu, A @ Vu)
    r = np.linalg.norm(A @ Vu - Vu * rho, axis=0)
    ru = np.linalg.norm(A @ Ur - Ur * wr, axis=0)
    cu = np.einsum("ij,ij->j", Ur, Vu)
    sin_t = np.linalg.norm(Vu - Ur * cu, axis=0)
    worst = 0.0
    for j in range(n):
        others = np.delete(wr, j)
        delta = np.min(np.abs(others - rho[j])) if others.size else np.inf
        if delta > 1e-4 * normA:
            worst = max(worst, sin_t[j] / (2.0 * (r[j] + ru[j]) / delta + 1e-6))
    return werr, res, orth, worst


def _check_batch(As, w, V, info, name):
    worst = np.zeros(4)
    for b in range(As.shape[0]):
        worst = np.maximum(worst, _check_one(As[b], w[b], V[b], name))
    print(f"[eigh_batched] {name}: {As.shape[0]} x {As.shape[1]}: max |dw|/|A| {worst[0]:.2e} residual "
          f"{worst[1]:.2e} orth {worst[2]:.2e} sin-theta/bound {worst[3]:.2f}, sweeps <= {info.max()}", flush=True)
    assert np.all(info >= 1) and np.all(info <= 30)
    assert worst[0] <= TOL_W and worst[1] <= TOL_R and worst[2] <= TOL_O and worst[3] <= 1.0


def _run_dense(spec, As):
    import torch
    w, V, info = spec.eigh_batched_dense(dev(As.astype(np.float32)))
    torch.cuda.synchronize()
    return w.cpu().numpy().astype(np.float64), V.cpu().numpy().astype(np.float64), info.cpu().numpy()


@pytest.mark.parametrize("n", [1, 2, 3, 7, 16, 30, 31, 32])
def test_eigh_batched_random(spec, n):
    print_case("eigh_batched_random", n=n)
    rng = np.random.default_rng(700 + n)
    G = rng.standard_normal((64, n, n))
    As = ((G + G.transpose(0, 2, 1)) / 2).astype(np.float32)
    w, V, info = _run_dense(spec, As)
    _check_batch(As.astype(np.float64), w, V, info, f"random n={n}")


def test_eigh_batched_eigentrack_windows(spec):
    """Windows of N = 30 steps from the GPU band Gram of bf16 activations; the
    oracle's window Grams come from H directly; the eigenvalues also match
    the direct batched solver on the same band."""
    import torch
    print_case("eigh_batched_eigentrack")
    S, T, d, N = 3, 120, 512, 30
    H = synth.eigentrack(streams=S, T=T, d=d)
    band = spec.gram_window(dev_bf16(H), N=N)
    w, V, info = spec.eigh_batched_band(band, n=N, scale=1.0 / N)
    wd, _ = spec.eigvalsh_batched_band(band, n=N, scale=1.0 / N)
    torch.cuda.synchronize()
    w, V, info, wd = (w.cpu().numpy().astype(np.float64), V.cpu().numpy().astype(np.float64), info.cpu().numpy(),
                      wd.cpu().numpy().astype(np.float64))
    W = T - N + 1
    # the solver's own input: the f32 band the GPU wrote, as fp64 windows
    b32 = band.cpu().numpy().astype(np.float64)
    As = np.concatenate([oracle.band_window_gram(b32[s], N, 1.0 / N) for s in range(S)])
    _check_batch(As, w, V, info, "eigentrack windows")
    ref = np.concatenate([oracle.eigvalsh_small(oracle.window_gram(H[s], "bf16", N))[0] for s in range(S)])
    assert np.max(np.abs(w - ref) / ref[:, :1]) <= 1e-4
    assert np.max(np.abs(w - wd) / wd[:, :1]) <= 1e-5
    assert w.shape == (S * W, N)


def test_eigh_batched_degenerate(spec):
    """Rank-deficient windows (each step repeated three times: rank 10 of 30),
    planted repeated eigenvalues, zero and identity matrices."""
    print_case("eigh_batched_degenerate")
    rng = np.random.default_rng(801)
    rep = np.repeat(rng.standard_normal((4, 10, 64)), 3, axis=1)  # 4 windows of 30 steps
    low = np.einsum("bid,bjd->bij", rep, rep) / 30
    Q, _ = np.linalg.qr(rng.standard_normal((4, 24, 24)))
    vals = np.concatenate([np.full(6, 2.0), np.full(4, -1.0), rng.uniform(-3, 3, 14)])
    planted = np.einsum("bij,j,bkj->bik", Q, vals, Q)
    for As, name in [(low, "rank 10 of 30"), (planted, "repeated eigenvalues"),
                     (np.zeros((3, 30, 30)), "zero"), (np.stack([np.eye(32) * 2.5] * 2), "identity")]:
        As = ((As + As.transpose(0, 2, 1)) / 2).astype(np.float32)
        w, V, info = _run_dense(spec, As)
        _check_batch(As.astype(np.float64), w, V, info, name)


def test_eigh_batched_non_finite(spec):
    print_case("eigh_batched_non_finite")
    rng = np.random.default_rng(901)
    G = rng.standard_normal((3, 20, 20))
    As = ((G + G.transpose(0, 2, 1)) / 2).astype(np.float32)
    As[1, 7, 3] = np.nan
    w, V, info = _run_dense(spec, As)
    assert info[1] == -1 and np.all(np.isnan(w[1])) and np.all(np.isnan(V[1]))
    assert info[0] >= 1 and info[2] >= 1
    _check_batch(As[[0, 2]].astype(np.float64), w[[0, 2]], V[[0, 2]], info[[0, 2]], "finite neighbours")
