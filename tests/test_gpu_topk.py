"""Parity of the randomised leading eigenvalues (random projection, subspace
iteration, Rayleigh-Ritz) with the fp64 oracle on the same f32 matrix and the
same seeded test matrix, through the C ABI.

Bound: every Ritz value within 1e-4 * lambda_max (the eigenvalue tolerance of
the large solver); the Ritz values of an exactly low-rank matrix are its
eigenvalues, and no Ritz value exceeds the eigenvalue of its rank (interlacing).
"""
import numpy as np
import pytest

import oracle
from gpu_util import dev, print_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spec():
    import weights_bf16_fp32_amd as spec
    spec.lib()
    return spec


def _cov(rng, n_rows, d, spikes):
    X = rng.standard_normal((n_rows, d))
    U, _ = np.linalg.qr(rng.standard_normal((d, len(spikes))))
    X += (rng.standard_normal((n_rows, len(spikes))) * np.sqrt(spikes)) @ U.T
    return ((X.T @ X) / n_rows).astype(np.float32)


@pytest.mark.parametrize("d,q", [(300, 0), (1000, 1), (1000, 3), (4096, 2)])
def test_topk_parity(spec, d, q):
    import torch
    print_case("topk", d=d, q=q)
    rng = np.random.default_rng(d + q)
    A = _cov(rng, 2 * d if d < 4096 else 4096, d, spikes=np.geomspace(50, 2, 12))
    Om = rng.standard_normal((d, 32)).astype(np.float32)
    Ad = dev(A)
    Au = Ad.clone()
    iu = np.triu_indices(d, 1)
    Au[iu[0], iu[1]] = 1e30  # the upper triangle is never read
    w = spec.eigvalsh_topk(Au, dev(Om), q=q)
    torch.cuda.synchronize()
    wg = w.cpu().numpy().astype(np.float64)
    ref = oracle.topk_ritz(A.astype(np.float64), Om, q)
    lmax = ref[0]
    err = np.max(np.abs(wg - ref))
    print(f"[topk] d={d} q={q} max |dtheta| {err:.3g} lambda_max {lmax:.4g}", flush=True)
    assert err <= 1e-4 * lmax
    assert np.all(np.diff(wg) <= 0)
    # A was only read
    assert torch.equal(Au[iu[1], iu[0]], Ad[iu[1], iu[0]])


def test_topk_low_rank_exact(spec):
    import torch
    print_case("topk_low_rank")
    rng = np.random.default_rng(3)
    d = 512
    lam = np.r_[np.linspace(9.0, 1.0, 20), np.zeros(d - 20)]
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    A = ((Q * lam) @ Q.T).astype(np.float32)
    Om = rng.standard_normal((d, 32)).astype(np.float32)
    w = spec.eigvalsh_topk(dev(A), dev(Om), q=1)
    torch.cuda.synchronize()
    wg = w.cpu().numpy().astype(np.float64)
    ev = np.sort(np.linalg.eigvalsh(A.astype(np.float64)))[::-1]
    assert np.max(np.abs(wg[:20] - ev[:20])) <= 1e-4 * ev[0]
    assert np.max(np.abs(wg[20:])) <= 1e-4 * ev[0]
    assert np.all(wg <= ev[:32] + 1e-4 * ev[0])


@pytest.mark.parametrize("d,q", [(300, 0), (1000, 3), (4096, 2)])
def test_eigvecs_parity(spec, d, q):
    """Ritz vectors: values as above; P^T P = I and the Rayleigh quotients
    p_i^T A p_i = theta_i to 1e-4 (f32 rounding of Q and P); columns whose Ritz
    value is separated from the others by gap_i >= 1e-2 lambda_max match the
    oracle's up to sign, within 1e-4 lambda_max / gap_i + 1e-4 (the
    perturbation bound of an eigenvector over its gap)."""
    import torch
    print_case("eigvecs_topk", d=d, q=q)
    rng = np.random.default_rng(10 * d + q)
    A = _cov(rng, 2 * d if d < 4096 else 4096, d, spikes=np.geomspace(50, 2, 12))
    Om = rng.standard_normal((d, 32)).astype(np.float32)
    Ad = dev(A)
    Au = Ad.clone()
    iu = np.triu_indices(d, 1)
    Au[iu[0], iu[1]] = 1e30  # the upper triangle is never read
    ldp = 40
    Pbuf = torch.full((d, ldp), 7.0, dtype=torch.float32, device=Ad.device)
    w, P = spec.eigvecs_topk(Au, dev(Om), q=q, P=Pbuf)
    torch.cuda.synchronize()
    wg = w.cpu().numpy().astype(np.float64)
    Pb = P.cpu().numpy().astype(np.float64)
    assert np.all(Pb[:, 32:] == 7.0)  # columns past 32 untouched
    Pg = Pb[:, :32]
    tr, Pr = oracle.topk_ritz_vectors(A.astype(np.float64), Om, q)
    lmax = tr[0]
    err = np.max(np.abs(wg - tr))
    orth = np.max(np.abs(Pg.T @ Pg - np.eye(32)))
    A64 = A.astype(np.float64)
    rq = np.einsum("ij,ij->j", Pg, A64 @ Pg)
    rq_err = np.max(np.abs(rq - wg))
    gap = np.array([np.min(np.abs(np.delete(tr, i) - tr[i])) for i in range(32)])
    sel = np.nonzero(gap >= 1e-2 * lmax)[0]
    dots = np.einsum("ij,ij->j", Pg[:, sel], Pr[:, sel])
    vec_err = np.linalg.norm(Pg[:, sel] - np.sign(dots) * Pr[:, sel], axis=0)
    bound = 1e-4 * lmax / gap[sel] + 1e-4
    print(f"[eigvecs] d={d} q={q} |dtheta| {err:.3g} orth {orth:.3g} rq {rq_err:.3g} "
          f"compared {sel.size} cols, max err/bound {np.max(vec_err / bound):.3g}", flush=True)
    assert err <= 1e-4 * lmax
    assert np.all(np.diff(wg) <= 0)
    assert orth <= 1e-4
    assert rq_err <= 1e-4 * lmax
    assert sel.size >= 4
    assert np.all(vec_err <= bound)
    assert torch.equal(Au[iu[1], iu[0]], Ad[iu[1], iu[0]])


def test_eigvecs_low_rank_subspace(spec):
    """Exactly rank 6 with distinct eigenvalues: the 6 leading Ritz vectors are
    the eigenvectors (up to sign) and span the column space of A."""
    import torch
    print_case("eigvecs_low_rank")
    rng = np.random.default_rng(11)
    d = 768
    lam = np.r_[[12.0, 9.0, 6.5, 4.0, 2.5, 1.0], np.zeros(d - 6)]
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    A = ((Q * lam) @ Q.T).astype(np.float32)
    Om = rng.standard_normal((d, 32)).astype(np.float32)
    w, P = spec.eigvecs_topk(dev(A), dev(Om), q=1)
    torch.cuda.synchronize()
    wg = w.cpu().numpy().astype(np.float64)
    Pg = P.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(wg[:6] - lam[:6])) <= 1e-4 * lam[0]
    dots = np.abs(np.einsum("ij,ij->j", Pg[:, :6], Q[:, :6]))
    assert np.all(dots >= 1 - 1e-4), dots


@pytest.mark.parametrize("case", ["min64", "ragged777", "zero", "identity"])
def test_eigvecs_edge_cases(spec, case):
    """The smallest size, a ragged size with a wider P, and two degenerate
    matrices: A = 0 (every Ritz value 0; P must still be orthonormal and
    finite) and A = I (every Ritz value 1, any orthonormal P is right)."""
    import torch
    print_case("eigvecs_edge", case=case)
    rng = np.random.default_rng({"min64": 64, "ragged777": 777, "zero": 5, "identity": 6}[case])
    d = {"min64": 64, "ragged777": 777, "zero": 256, "identity": 256}[case]
    if case == "zero":
        A = np.zeros((d, d), np.float32)
    elif case == "identity":
        A = np.eye(d, dtype=np.float32)
    else:
        A = _cov(rng, 2 * d, d, spikes=np.geomspace(30, 3, 6))
    Om = rng.standard_normal((d, 32)).astype(np.float32)
    ldp = 48 if case == "ragged777" else 32
    Pbuf = torch.full((d, ldp), 5.0, dtype=torch.float32, device="cuda")
    w, P = spec.eigvecs_topk(dev(A), dev(Om), q=2, P=Pbuf[:, :32])
    torch.cuda.synchronize()
    wg = w.cpu().numpy().astype(np.float64)
    Pb = Pbuf.cpu().numpy().astype(np.float64)
    Pg = Pb[:, :32]
    assert np.all(np.isfinite(wg)) and np.all(np.isfinite(Pg))
    assert np.all(Pb[:, 32:] == 5.0)
    assert np.max(np.abs(Pg.T @ Pg - np.eye(32))) <= 1e-4
    if case == "zero":
        assert np.all(wg == 0.0)
    elif case == "identity":
        assert np.max(np.abs(wg - 1.0)) <= 1e-5
    else:
        tr, Pr = oracle.topk_ritz_vectors(A.astype(np.float64), Om, 2)
        assert np.max(np.abs(wg - tr)) <= 1e-4 * tr[0]
        rq = np.einsum("ij,ij->j", Pg, A.astype(np.float64) @ Pg)
        assert np.max(np.abs(rq - wg)) <= 1e-4 * tr[0]


def test_eigvecs_non_finite_input_writes_every_output(spec):
    """A NaN in A makes Q^T A Q non-finite: info reports it and every value of w
    and of P's 32 columns is written (NaN), nothing left uninitialised; a finite
    input on the same buffers reports convergence."""
    import torch
    print_case("eigvecs_nonfinite")
    rng = np.random.default_rng(17)
    d = 256
    A = _cov(rng, 2 * d, d, spikes=np.geomspace(20, 3, 4))
    Om = dev(rng.standard_normal((d, 32)).astype(np.float32))
    info = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    w = torch.full((32,), 3.0, dtype=torch.float32, device="cuda")
    Pbuf = torch.full((d, 40), 3.0, dtype=torch.float32, device="cuda")
    spec.eigvecs_topk(dev(A), Om, q=2, w=w, P=Pbuf[:, :32], info=info)
    torch.cuda.synchronize()
    assert int(info.cpu()[0]) == 0
    assert np.all(np.isfinite(w.cpu().numpy()))
    A[17, 3] = np.nan
    spec.eigvecs_topk(dev(A), Om, q=2, w=w, P=Pbuf[:, :32], info=info)
    torch.cuda.synchronize()
    assert int(info.cpu()[0]) == 1
    assert np.all(np.isnan(w.cpu().numpy()))
    Pb = Pbuf.cpu().numpy()
    assert np.all(np.isnan(Pb[:, :32])) and np.all(Pb[:, 32:] == 3.0)
