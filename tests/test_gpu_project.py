"""Parity of the weight projection W' = P^T W P and the factor X = W P with the
fp64 oracle, through the C ABI, on seeded synthetic weights (bf16 bit patterns
and f32) and seeded orthonormal bases.

Bound: both products run in f32 with f32 accumulation over d terms, so each
entry is within the dot-product bound gamma_d = (d + 2) u of its absolute
products: |X - X*| <= gamma_d |W| |P| and |W' - W'*| <= 2 gamma_d |P|^T |W| |P|
(u = 2^-24; bf16 weights widen exactly, so the inputs are the oracle's).
"""
import numpy as np
import pytest

import oracle
from gpu_util import EPS32, dev, dev_bf16, print_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spec():
    import weights_bf16_fp32_amd as spec
    spec.lib()
    return spec


def _weight(rng, d, ldw, bf16):
    W = (rng.standard_normal((d, d)) / np.sqrt(d)).astype(np.float32)
    if bf16:
        bits = np.zeros((d, ldw), np.uint16)
        bits[:, :d] = W.view(np.uint32) >> 16
        bits[:, d:] = 0x7fc0  # NaN padding past column d is never read
        return bits, (bits[:, :d].astype(np.uint32) << 16).view(np.float32)
    buf = np.full((d, ldw), np.nan, np.float32)
    buf[:, :d] = W
    return buf, W


def _basis(rng, d, k, ldp):
    Q, _ = np.linalg.qr(rng.standard_normal((d, k)))
    buf = np.full((d, ldp), np.nan, np.float32)
    buf[:, :k] = Q.astype(np.float32)
    return buf, buf[:, :k].astype(np.float64)


def _run(spec, d, k, bf16, seed, want_factor=True, ldw=None, ldp=None, ldo=None, ldx=None):
    import torch
    print_case("project_weight", d=d, k=k, bf16=bf16, factor=want_factor)
    rng = np.random.default_rng(seed)
    ldw = ldw or d + (-d) % 8
    ldp, ldo, ldx = ldp or k, ldo or k, ldx or k
    Wbuf, W = _weight(rng, d, ldw, bf16)
    Pbuf, P = _basis(rng, d, k, ldp)
    Wd = (dev_bf16(Wbuf) if bf16 else dev(Wbuf))[:, :d]
    Pd = dev(Pbuf)[:, :k]
    Wp = torch.full((k, ldo), 3.0, dtype=torch.float32, device=Wd.device)
    X = torch.full((d, ldx), 3.0, dtype=torch.float32, device=Wd.device) if want_factor else None
    spec.project_weight(Wd, Pd, k=k, Wp=Wp[:, :k], X=None if X is None else X[:, :k], want_factor=want_factor)
    torch.cuda.synchronize()
    ref_wp, ref_x = oracle.project_weight(W, P)
    gam = (d + 2) * EPS32
    aW, aP = np.abs(W.astype(np.float64)), np.abs(P)
    g = Wp.cpu().numpy().astype(np.float64)
    assert np.all(g[:, k:] == 3.0)  # columns past k untouched
    err = np.abs(g[:, :k] - ref_wp)
    bound = 2 * gam * (aP.T @ (aW @ aP)) + 1e-30
    print(f"[project] d={d} k={k} bf16={bf16} max err/bound W' {np.max(err / bound):.3g}", flush=True)
    assert np.all(err <= bound)
    if want_factor:
        x = X.cpu().numpy().astype(np.float64)
        assert np.all(x[:, k:] == 3.0)
        errx = np.abs(x[:, :k] - ref_x)
        assert np.all(errx <= gam * (aW @ aP) + 1e-30)


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("d,k", [(64, 32), (100, 7), (777, 13), (1000, 1)])
def test_project_small(spec, d, k, bf16):
    _run(spec, d, k, bf16, seed=d * 3 + k)


def test_project_strides_and_no_factor(spec):
    _run(spec, 300, 20, True, seed=5, ldw=320, ldp=29, ldo=24, ldx=33)
    _run(spec, 300, 20, False, seed=6, ldw=308, want_factor=False)
    _run(spec, 8, 8, True, seed=7)  # a single partial tile


@pytest.mark.parametrize("bf16", [True, False])
def test_project_4096(spec, bf16):
    """The 4096 x 4096 weight on a 32-column basis, the launch bench.py times."""
    _run(spec, 4096, 32, bf16, seed=4096 + bf16)


def test_project_signal_subspace_end_to_end(spec):
    """Properties of the whole chain on the GPU: covariance of data with planted
    directions -> Ritz vectors -> W' of a weight that acts on those directions
    only.  W = U S U^T with U the planted directions: P spans U, so
    ||W'||_F = ||W||_F and the eigenvalues of W' are those of W."""
    import torch
    print_case("project_signal_subspace")
    rng = np.random.default_rng(12)
    d, n, kk = 1024, 4096, 6
    U, _ = np.linalg.qr(rng.standard_normal((d, kk)))
    Xd = rng.standard_normal((n, d)) + (rng.standard_normal((n, kk)) * np.sqrt([200, 160, 120, 90, 60, 40])) @ U.T
    C = dev(((Xd.T @ Xd) / n).astype(np.float32))
    s = np.array([3.0, -2.0, 1.5, 1.0, -0.5, 0.25])
    W = ((U * s) @ U.T).astype(np.float32)
    Om = dev(rng.standard_normal((d, 32)).astype(np.float32))
    w, P = spec.eigvecs_topk(C, Om, q=3)
    torch.cuda.synchronize()
    # the MP edge for sigma^2 = 1, c = d / n, with a 20 % margin over the
    # Tracy-Widom fluctuation of the largest bulk eigenvalue around it
    lam_plus = 1.0 * (1 + np.sqrt(d / n)) ** 2
    k = int(np.sum(w.cpu().numpy() > 1.2 * lam_plus))
    assert k == kk
    Wp, X = spec.project_weight(dev(W), P, k=k)
    torch.cuda.synchronize()
    wp = Wp.cpu().numpy().astype(np.float64)
    ev = np.sort(np.linalg.eigvalsh(0.5 * (wp + wp.T)))
    # the sample eigenvectors lean off U by sin^2 <= c / theta ~ 6e-3 (BBP): W' keeps
    # the spectrum of W to that relative level
    assert np.max(np.abs(ev - np.sort(s))) <= 0.05 * np.max(np.abs(s))
    assert abs(np.linalg.norm(wp) - np.linalg.norm(s)) <= 0.05 * np.linalg.norm(s)


def test_low_rank_factor_eckart_young(spec):
    """Swift-SVD-style rank-k factors from the library alone: C = W^T W
    (SYRK), the top Ritz vectors P of C (random projection), X = W P; then
    ||W - X P^T||_F^2 is within 1 % of the Eckart-Young optimum
    sum_{i > k} sigma_i^2, known here by construction (W = U diag(sigma) V^T
    with seeded orthogonal U, V)."""
    import torch
    print_case("low_rank_eckart_young")
    rng = np.random.default_rng(2)
    d, k = 1024, 16
    sig = 10.0 * 0.7 ** np.arange(d) + 1e-3
    U, _ = np.linalg.qr(rng.standard_normal((d, d)))
    V, _ = np.linalg.qr(rng.standard_normal((d, d)))
    W = ((U * sig) @ V.T).astype(np.float32)
    W64 = W.astype(np.float64)
    s_true = np.linalg.svd(W64, compute_uv=False)  # of the f32-rounded W actually used
    opt = float(np.sum(s_true[k:] ** 2))
    Wd = dev(W)
    C = torch.zeros((d, d), dtype=torch.float32, device=Wd.device)
    spec.cov_accumulate(Wd, C, alpha=1.0, beta=0.0)
    w, P = spec.eigvecs_topk(C, dev(rng.standard_normal((d, 32)).astype(np.float32)), q=2)
    Wp, X = spec.project_weight(Wd, P, k=k)
    torch.cuda.synchronize()
    Pk = P.cpu().numpy().astype(np.float64)[:, :k]
    Xk = X.cpu().numpy().astype(np.float64)
    err = float(np.sum((W64 - Xk @ Pk.T) ** 2))
    print(f"[eckart-young] k={k} error {err:.6g} optimum {opt:.6g} ratio {err / opt:.6f}", flush=True)
    assert opt <= err * (1 + 1e-9) + 1e-12  # no rank-k factor beats the optimum
    assert err <= 1.01 * opt
    # W' of the same basis against its fp64 value on the GPU's own P (a property
    # of the output, not an oracle input), within the f32 bound used above
    ref = Pk.T @ W64 @ Pk
    bound = 2 * (d + 2) * EPS32 * (np.abs(Pk).T @ np.abs(W64) @ np.abs(Pk))
    assert np.all(np.abs(Wp.cpu().numpy().astype(np.float64) - ref) <= bound)
