"""The fused window spectra + descriptors entry point (spec_eigvalsh_batched_desc)
against the two-call path (spec_eigvalsh_batched, then spec_descriptors) and the
oracle: the same eigenvalues bit for bit, descriptors within 1e-12 relative of
the two-call records (sums in another order) and within 1e-4 of the oracle's,
counts exact."""
import math

import numpy as np
import pytest

import oracle
from gpu_util import DESC_FLOAT_FIELDS, dev, dev_bf16, print_case
from gen import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spec():
    import weights_bf16_fp32_amd as spec
    spec.lib()
    return spec


def _same_records(a, b, rel=1e-12):
    for f in DESC_FLOAT_FIELDS:
        x, y = a[f].astype(np.float64), b[f].astype(np.float64)
        nan = np.isnan(y)
        assert np.array_equal(np.isnan(x), nan), f
        assert np.all(np.abs(x[~nan] - y[~nan]) <= rel * np.abs(y[~nan]) + 1e-300), f
    for f in ("n_above", "n_small", "r_pos", "flags"):
        assert np.array_equal(a[f], b[f]), f


@pytest.mark.parametrize("mode", ["given", "median", "mean"])
def test_fused_windows_match_two_calls_and_oracle(spec, mode):
    import torch
    print_case("fused_windows", mode=mode)
    S, T, d, N = 3, 64, 256, 30
    H = synth.eigentrack(streams=S, T=T, d=d)
    band = spec.gram_window(dev_bf16(H), N=N)
    s2m = {"given": spec.SIGMA2_GIVEN, "median": spec.SIGMA2_MEDIAN, "mean": spec.SIGMA2_MEAN}[mode]
    w2, i2 = spec.eigvalsh_batched_band(band, n=N, scale=1.0 / N)
    rec2 = spec.descriptors(w2, n_samples=N, p_dim=d, k=8, sigma2_mode=s2m)
    w1, i1, rec1 = spec.eigvalsh_batched_band_desc(band, n=N, scale=1.0 / N, n_samples=N, p_dim=d, k=8,
                                                   sigma2_mode=s2m)
    torch.cuda.synchronize()
    assert np.array_equal(w1.cpu().numpy(), w2.cpu().numpy())
    assert np.array_equal(i1.cpu().numpy(), i2.cpu().numpy())
    _same_records(rec1, rec2)
    W = T - N + 1
    om = {"given": oracle.SIGMA2_GIVEN, "median": oracle.SIGMA2_MEDIAN, "mean": oracle.SIGMA2_MEAN}[mode]
    for s in range(S):
        G = oracle.window_gram(H[s], "bf16", N)
        ref, _ = oracle.eigvalsh_small(G)
        for win in (0, W // 2, W - 1):
            o = oracle.descriptors(ref[win], n_samples=N, p_dim=d, k=8, sigma2_mode=om)
            g = rec1[s * W + win]
            for f in ("S", "H", "erank", "m1", "gk", "g1", "lambda_plus", "mp_w1"):
                assert abs(float(g[f]) - o[f]) <= 1e-4 * abs(o[f]), (f, float(g[f]), o[f])


@pytest.mark.parametrize("n,batch", [(17, 9), (32, 4), (2, 3)])
def test_fused_dense_sizes(spec, n, batch):
    """The padded 32-row kernel (n != 30), an odd batch, and the smallest n."""
    import torch
    print_case("fused_dense", n=n, batch=batch)
    rng = np.random.default_rng(n * 10 + batch)
    X = rng.standard_normal((batch, n + 5, n))
    A = np.einsum("bki,bkj->bij", X, X).astype(np.float32)
    Ad = dev(A)
    w2, i2 = spec.eigvalsh_batched_dense(Ad)
    rec2 = spec.descriptors(w2, n_samples=n + 5, p_dim=n, k=1)
    w1, i1, rec1 = spec.eigvalsh_batched_dense_desc(Ad, n_samples=n + 5, p_dim=n, k=1)
    torch.cuda.synchronize()
    assert np.array_equal(w1.cpu().numpy(), w2.cpu().numpy())
    _same_records(rec1, rec2)
    ref, _ = oracle.eigvalsh_small(A.astype(np.float64))
    for b in range(batch):
        o = oracle.descriptors(ref[b], n_samples=n + 5, p_dim=n, k=1)
        assert abs(float(rec1[b]["H"]) - o["H"]) <= 1e-4 * abs(o["H"]) + 1e-12
        assert int(rec1[b]["n_above"]) == o["n_above"] or \
            np.min(np.abs(ref[b] - o["lambda_plus"])) <= 1e-5 * ref[b][0]


def test_fused_nonfinite_matrix(spec):
    import torch
    print_case("fused_nonfinite")
    A = np.tile(np.eye(30, dtype=np.float32), (3, 1, 1))
    A[1, 7, 3] = np.nan
    w, info, rec = spec.eigvalsh_batched_dense_desc(dev(A), n_samples=60, p_dim=30, k=1)
    torch.cuda.synchronize()
    assert list(info.cpu().numpy() < 0) == [False, True, False]
    assert rec[1]["flags"] & spec.FLAG_NONFINITE and math.isnan(float(rec[1]["H"]))
    assert abs(float(rec[0]["H"]) - math.log(30)) <= 1e-12 and float(rec[2]["m1"]) == pytest.approx(1 / 30)
