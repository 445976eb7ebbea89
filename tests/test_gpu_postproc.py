"""Parity of the descriptor post-processing (exponential smoothing of descriptor
series; median, winsorised sigma^2, MAD, log-eigenvalue and KL-to-MP statistics
of spectra) with the fp64 oracle, through the C ABI.

Inputs are seeded synthetic records and oracle spectra, never values the GPU
path produced.  Both sides compute in fp64: order statistics (median, MAD),
counts and flags must match exactly; sums within 1e-12 relative; the KL value
within 1e-10 where every value lies clear of the bin edges (a value on an edge
may fall on either side when sigma^2 is itself a sum).
"""
import math
import os

import numpy as np
import pytest

import oracle
from gpu_util import DESC_FLOAT_FIELDS, dev, dev_bf16, print_case
from gen import synth

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ROBUST_F = ["median", "sigma2_winsor", "mad", "log_mean", "log_std", "sigma2", "kl_mp"]


@pytest.fixture(scope="module")
def spec():
    import weights_bf16_fp32_amd as spec
    spec.lib()
    return spec


def _records(streams, W, seed, holes=True):
    rng = np.random.default_rng(seed)
    rec = np.zeros((streams, W), dtype=oracle_desc_dtype())
    for f in DESC_FLOAT_FIELDS:
        rec[f] = rng.lognormal(0.0, 1.0, (streams, W)) * rng.choice([-1.0, 1.0], (streams, W))
    for f in ["n_above", "n_small", "r_pos"]:
        rec[f] = rng.integers(0, 30, (streams, W))
    rec["flags"] = rng.integers(0, 8, (streams, W))
    if holes:
        for f in DESC_FLOAT_FIELDS:
            m = rng.random((streams, W)) < 0.02
            rec[f][m] = rng.choice([np.nan, np.inf, -np.inf], m.sum())
        rec["H"][0, :5] = np.nan  # a series that starts with a gap
    return rec


def oracle_desc_dtype():
    import weights_bf16_fp32_amd as spec
    return spec.DESC_DTYPE


def _cmp_records(g, o, rec):
    """Smoothed values within 1e-12 of the series' largest finite input (each
    output is a convex combination of inputs, so rounding is relative to them)."""
    for f in DESC_FLOAT_FIELDS:
        a, b = g[f].astype(np.float64), o[f].astype(np.float64)
        assert np.array_equal(np.isnan(a), np.isnan(b)), f
        x = rec[f].astype(np.float64)
        scale = np.max(np.where(np.isfinite(x), np.abs(x), 0.0), axis=1, keepdims=True) * np.ones_like(b)
        ok = ~np.isnan(b)
        assert np.all(np.abs(a[ok] - b[ok]) <= 1e-12 * scale[ok] + 1e-300), f
    for f in ["n_above", "n_small", "r_pos", "flags"]:
        assert np.array_equal(g[f], o[f]), f


@pytest.mark.parametrize("alpha", [1.0, 0.3, 0.05])
def test_desc_smooth_small(spec, alpha):
    import torch
    print_case("desc_smooth_small", alpha=alpha)
    rec = _records(7, 33, seed=int(alpha * 100))
    d = torch.from_numpy(rec.view(np.uint8).reshape(-1, 144).copy()).cuda()
    g = spec.desc_smooth(d, streams=7, W=33, alpha=alpha)
    torch.cuda.synchronize()
    _cmp_records(g, oracle.smooth_descriptors(rec, alpha), rec)


def test_desc_smooth_eigentrack_shape(spec):
    """256 streams x 483 windows, the EigenTrack record layout bench.py smooths."""
    import torch
    print_case("desc_smooth_full", streams=256, W=483)
    rec = _records(256, 483, seed=5)
    d = torch.from_numpy(rec.view(np.uint8).reshape(-1, 144).copy()).cuda()
    g = spec.desc_smooth(d, streams=256, W=483, alpha=0.2)
    torch.cuda.synchronize()
    _cmp_records(g, oracle.smooth_descriptors(rec, 0.2), rec)


def _edge_clear(lam, n, p, s2, bins, rel=1e-9):
    """True if no value is within rel of a KL bin edge (the bin is then the same
    on both sides even if sigma^2 differs in its last bits)."""
    lam = np.maximum(np.asarray(lam, np.float64), 0.0)
    if p <= n:
        mu, c = lam, p / n
    else:
        mu, c = (n / p) * lam, n / p
    lm, lp = oracle.mp_edges(s2, c)
    t = (mu - lm) / (lp - lm) * bins
    inside = (t > 0) & (t < bins)
    return bool(np.all(np.abs(t[inside] - np.round(t[inside])) > rel * bins))


def _cmp_robust(g, lam, **kw):
    o = oracle.robust_stats(lam, **kw)
    assert int(g["flags"]) == o["flags"], (g["flags"], o["flags"])
    assert int(g["n_mad"]) == o["n_mad"]
    for f in ["median", "mad"]:  # order statistics: the same fp64 values
        if not math.isnan(o[f]):
            assert float(g[f]) == o[f], (f, float(g[f]), o[f])
    for f in ["sigma2_winsor", "log_mean", "log_std", "sigma2"]:
        a, b = float(g[f]), o[f]
        if math.isnan(b):
            assert math.isnan(a), f
        else:
            assert abs(a - b) <= 1e-12 * abs(b) + 1e-300, (f, a, b)
    a, b = float(g["kl_mp"]), o["kl_mp"]
    if math.isnan(b):
        assert math.isnan(a)
    elif kw.get("sigma2_mode", 0) in (oracle.SIGMA2_GIVEN, oracle.SIGMA2_MEDIAN) or \
            _edge_clear(lam, kw["n_samples"], kw["p_dim"], o["sigma2"], kw.get("bins", 16)):
        assert abs(a - b) <= 1e-10 * max(1.0, abs(b)), (a, b)


def _spectra(seed, batch, r, n, p):
    """Oracle eigenvalues (descending) of seeded covariances (1/n) X^T X of
    n x r Gaussian data with a few planted spikes, scaled to p/n."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(batch):
        X = rng.standard_normal((n, r))
        X[:, :2] *= rng.uniform(1.0, 4.0, 2)
        C = oracle.covariance(X.astype(np.float32), "f32", 1.0 / n)
        out.append(oracle.eigvalsh_large(C))
    return np.array(out)


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("r,n,p", [(30, 64, 30), (64, 200, 64), (31, 31, 4096)])
def test_spectrum_robust_modes(spec, mode, r, n, p):
    import torch
    print_case("spectrum_robust", mode=mode, r=r, n=n, p=p)
    lam = _spectra(r * 7 + mode, 12, r, max(n, r + 1), p)
    kw = dict(n_samples=n, p_dim=p, sigma2=1.0, sigma2_mode=mode, winsor_frac=0.1, mad_k=2.5, bins=12)
    for dt in (torch.float64, torch.float32):
        w = dev(lam).to(dt)
        g = spec.spectrum_robust(w, **kw)
        torch.cuda.synchronize()
        ref = lam if dt == torch.float64 else lam.astype(np.float32).astype(np.float64)
        for b in range(lam.shape[0]):
            _cmp_robust(g[b], ref[b], **kw)


def test_spectrum_robust_edge_cases(spec):
    import torch
    print_case("spectrum_robust_edges")
    cases = [
        np.array([2.0, 1.0]),                            # r = 2
        np.zeros(8),                                     # no positive value
        np.array([5.0, 4.0, np.nan, 1.0]),               # non-finite
        np.array([3.0, 3.0, 3.0, 3.0, 1.0, 1.0]),        # ties around the median
        np.array([9.0, 4.0, 3.0, 2.0, 1.0, -1e-9]),      # round-off below zero
        np.linspace(10.0, 0.5, 64),                      # bins 1 and 64, winsor at its cap
    ]
    for lam in cases:
        for bins, wf in [(1, 0.5), (64, 0.0), (7, 0.25)]:
            kw = dict(n_samples=100, p_dim=lam.size, sigma2=1.5, sigma2_mode=0, winsor_frac=wf, mad_k=1.0,
                      bins=bins)
            g = spec.spectrum_robust(dev(lam.reshape(1, -1)), **kw)
            torch.cuda.synchronize()
            _cmp_robust(g[0], lam, **kw)


def test_spectrum_robust_swiftsvd_4096(spec):
    """The 4096-eigenvalue Swift-SVD spectrum (oracle values, fp64 and f32)."""
    import torch
    print_case("spectrum_robust_4096")
    lam = np.load(os.path.join(GOLD, "swiftsvd.npz"))["eig"]
    for mode in (1, 3):
        kw = dict(n_samples=65536, p_dim=4096, sigma2_mode=mode, winsor_frac=0.05, mad_k=3.0, bins=32)
        for dt in (torch.float64, torch.float32):
            g = spec.spectrum_robust(dev(lam.reshape(1, -1)).to(dt), **kw)
            torch.cuda.synchronize()
            ref = lam if dt == torch.float64 else lam.astype(np.float32).astype(np.float64)
            _cmp_robust(g[0], ref, **kw)


def test_spectrum_robust_eigentrack_windows(spec):
    """All 123,648 window spectra of the EigenTrack workload in the launch bench.py
    times: sampled windows against the oracle on the oracle's own window
    spectra, and properties of every row at full size."""
    import torch
    print_case("spectrum_robust_windows", streams=256, T=512, N=30)
    S, T, d, N = 256, 512, 4096, 30
    W = T - N + 1
    H = synth.eigentrack(streams=S, T=T, d=d)
    rng = np.random.default_rng(77)
    picks = [(int(rng.integers(S)), int(rng.integers(W))) for _ in range(200)]
    G = np.array([oracle.window_gram(H[s][w:w + N], "bf16", N)[0] for s, w in picks])
    lam, _ = oracle.eigvalsh_small(G)
    kw = dict(n_samples=N, p_dim=d, sigma2_mode=oracle.SIGMA2_MEDIAN, winsor_frac=0.1, mad_k=3.0, bins=8)
    g = spec.spectrum_robust(dev(lam).to(torch.float32), **kw)
    torch.cuda.synchronize()
    ref = lam.astype(np.float32).astype(np.float64)
    for q in range(len(picks)):
        _cmp_robust(g[q], ref[q], **kw)
    # every window through the library's own path, checked by properties
    band = spec.gram_window(dev_bf16(H), N=N)
    w, _ = spec.eigvalsh_batched_band(band, n=N, scale=1.0 / N)
    rec = spec.spectrum_robust(w, **kw)
    torch.cuda.synchronize()
    wh = w.cpu().numpy().astype(np.float64).clip(min=0.0)
    assert rec.shape == (S * W,)
    assert np.array_equal(rec["median"], 0.5 * (wh[:, 14] + wh[:, 15]))
    assert np.all(rec["flags"] == 0) and np.all(rec["kl_mp"] >= -1e-12)
    assert np.all((rec["n_mad"] >= 0) & (rec["n_mad"] <= N))
