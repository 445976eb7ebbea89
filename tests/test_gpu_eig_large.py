"""GPU parity of the two-stage large eigensolver against the fp64 oracle.

Sizes cover the direct panel path (trailing rows fit in LDS), the TSQR panel
path (f32: more than 1024 trailing rows; f64: more than 512), ragged last
panels and blocks, and the degenerate cases (n < 3, zero, identity,
repeated and zero eigenvalues).  Tolerance: the benchmark spec's bound
1e-4 * lambda_max for f32 inputs; 1e-10 * lambda_max for f64, whose
reductions are done in fp64.
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


def _run(spec, A, dtype):
    import torch
    n = A.shape[0]
    Ad = dev(A.astype(dtype))
    info = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    w = spec.eigvalsh_large(Ad, info=info)
    torch.cuda.synchronize()
    return w.cpu().numpy().astype(np.float64), int(info.cpu().numpy()[0])


def _sym(rng, n):
    G = rng.standard_normal((n, n))
    return (G + G.T) / 2


@pytest.mark.parametrize("n", [1, 2, 3, 5, 32, 33, 34, 40, 64, 65, 100, 257, 1000, 1100, 2100])
def test_eig_large_f32_random(spec, n):
    print_case("eig_large_f32", n=n)
    rng = np.random.default_rng(1000 + n)
    A = _sym(rng, n).astype(np.float32)
    # garbage in the strict upper triangle must be ignored
    Ag = A.copy()
    Ag[np.triu_indices(n, 1)] = np.float32(1e30)
    w, info = _run(spec, Ag, np.float32)
    ref = oracle.eigvalsh_large(A.astype(np.float64))
    assert info == 0
    assert np.all(np.diff(w) <= 0)
    lmax = np.max(np.abs(ref))
    assert np.max(np.abs(w - ref)) <= 1e-4 * lmax


@pytest.mark.parametrize("n", [3, 40, 300, 600, 1100])
def test_eig_large_f64_random(spec, n):
    print_case("eig_large_f64", n=n)
    rng = np.random.default_rng(2000 + n)
    A = _sym(rng, n)
    w, info = _run(spec, A, np.float64)
    ref = oracle.eigvalsh_large(A)
    assert info == 0
    assert np.max(np.abs(w - ref)) <= 1e-10 * np.max(np.abs(ref))


def test_eig_large_covariance_structures(spec):
    rng = np.random.default_rng(7)
    n = 700
    # rank-deficient covariance (fewer samples than features)
    X = rng.standard_normal((200, n)).astype(np.float32)
    C = oracle.covariance(X, "f32", 1.0 / 200)
    w, info = _run(spec, C.astype(np.float32), np.float32)
    ref = oracle.eigvalsh_large(C.astype(np.float32).astype(np.float64))
    assert info == 0 and np.max(np.abs(w - ref)) <= 1e-4 * ref[0]
    # repeated eigenvalues and exact zeros
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    lam = np.concatenate([np.full(300, 2.0), np.zeros(200), np.linspace(0.1, 5.0, 200)])
    A = (Q * lam) @ Q.T
    w, info = _run(spec, A, np.float64)
    assert info == 0 and np.max(np.abs(w - np.sort(lam)[::-1])) <= 1e-10 * 5.0


@pytest.mark.parametrize("kind", ["zero", "identity", "diagonal"])
def test_eig_large_special(spec, kind):
    n = 150
    if kind == "zero":
        A = np.zeros((n, n))
    elif kind == "identity":
        A = np.eye(n)
    else:
        A = np.diag(np.linspace(-3, 7, n))
    for dt in (np.float32, np.float64):
        w, info = _run(spec, A, dt)
        ref = np.sort(np.diag(A))[::-1]
        assert info == 0
        assert np.max(np.abs(w - ref)) <= 1e-5 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("n", [1024, 4096])
def test_eig_large_f32_trace_preserved(spec, n):
    """An orthogonal similarity keeps the trace.  In fp32 each of the O(n^2 / 32)
    two-sided reflections moves it by rounding of either sign; a transformation
    that is not orthogonal to working precision (tau rounded apart from its v)
    shifts every eigenvalue the same way and the sum drifts by a multiple of
    n eps lambda_max (about 4 n eps lambda_max with such a tau on the FFN-width
    workload).  The unbiased reduction drifts by about n eps lambda_max / 10 on
    these inputs; the bound is n eps lambda_max / 4."""
    print_case("eig_large_f32_trace", n=n)
    rng = np.random.default_rng(4000 + n)
    Z = rng.standard_normal((2 * n, n)).astype(np.float32)
    A = (Z.T.astype(np.float64) @ Z.astype(np.float64) / (2 * n)).astype(np.float32)
    w, info = _run(spec, A, np.float32)
    assert info == 0
    tr = float(np.trace(A.astype(np.float64)))
    drift = abs(float(w.sum()) - tr)
    eps = float(np.finfo(np.float32).eps)
    print(f"[trace] n={n} |sum(lambda) - tr(A)| = {drift:.3g}, n eps lambda_max = {n * eps * w[0]:.3g}", flush=True)
    assert drift <= 0.25 * n * eps * float(w[0])


@pytest.mark.parametrize("kind", ["zero", "identity", "graded"])
def test_eig_large_panel_qr_paths(spec, kind):
    """Panels tall enough for the CholeskyQR panel factorisation (n = 600): zero
    and identity matrices give all-zero panels (the pivots fail and TSQR takes
    over), graded spectra over eight decades give ill-conditioned panels (the
    second pass, or TSQR), against the known eigenvalues."""
    n = 600
    rng = np.random.default_rng(31)
    if kind == "zero":
        lam = np.zeros(n)
    elif kind == "identity":
        lam = np.ones(n)
    else:
        lam = np.logspace(0, -8, n)
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    A = np.eye(n) * lam[0] if kind != "graded" else (Q * lam) @ Q.T
    if kind == "zero":
        A = np.zeros((n, n))
    ref = np.sort(lam)[::-1]
    for dt, tol in ((np.float32, 2e-5), (np.float64, 1e-11)):
        w, info = _run(spec, A, dt)
        assert info == 0
        assert np.max(np.abs(w - ref)) <= tol * max(1.0, ref[0]), (kind, dt)


def test_eig_large_concurrent_streams_match_one_at_a_time(spec):
    """Two solves in flight on two streams (each with its own panel helper
    stream at this size, which takes the look-ahead) give bit for bit the
    eigenvalues of the same solves run one at a time, and match LAPACK."""
    import torch
    n = 6400
    print_case("eig_large_two_streams", n=n)
    rng = np.random.default_rng(77)
    mats = [(_sym(rng, n) / np.sqrt(n)).astype(np.float32) for _ in range(2)]
    ref_seq = [_run(spec, M, np.float32) for M in mats]
    As = [dev(M) for M in mats]
    ws = [torch.empty(spec.eigvalsh_large_workspace(n, torch.float32), dtype=torch.uint8, device="cuda") for _ in range(2)]
    ws_out = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    infos = [torch.full((1,), -7, dtype=torch.int32, device="cuda") for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for j in range(2):
        with torch.cuda.stream(streams[j]):
            spec.eigvalsh_large(As[j], w=ws_out[j], ws=ws[j], info=infos[j])
    torch.cuda.synchronize()
    for j in range(2):
        assert int(infos[j].cpu()[0]) == 0 and ref_seq[j][1] == 0
        w = ws_out[j].cpu().numpy().astype(np.float64)
        assert np.array_equal(w, ref_seq[j][0])
        lap = np.linalg.eigvalsh(mats[j].astype(np.float64))[::-1]
        assert np.max(np.abs(w - lap)) <= 1e-4 * np.max(np.abs(lap))
