"""The sliding-window up/down-date (spec_eigvalsh_sliding) against the oracle:
every window's eigenvalues from the same f32 band, within 1e-6 * lambda_max
(fp64 updates, f32 output), on EigenTrack-shaped windows, strides, restart
periods that split streams raggedly, rank-deficient and repeated-row windows
(the deflation paths), windows of 1, 2, 32, 33 and 64 rows (both lane layouts),
a step with non-finite values, and the band from the GPU Gram kernel."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, dev_bf16, print_case
from gen import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spec():
    import weights_bf16_fp32_amd as spec
    spec.lib()
    return spec


def _oracle_spectra(band32, N, stride, scale):
    """[S * W, N] descending eigenvalues of the windows of the f32 band, fp64."""
    out = []
    for s in range(band32.shape[0]):
        K = oracle.band_window_gram(band32[s].astype(np.float64), N, scale, stride=stride)
        out.append(np.linalg.eigvalsh(K)[:, ::-1])
    return np.concatenate(out)


def _check(spec, band32, N, stride, scale, restart, tol=1e-6):
    import torch
    w, info = spec.eigvalsh_sliding(dev(band32), n=N, scale=scale, stride=stride, restart=restart)
    torch.cuda.synchronize()
    got, inf_ = w.cpu().numpy().astype(np.float64), info.cpu().numpy()
    ref = _oracle_spectra(band32, N, stride, scale)
    assert got.shape == ref.shape
    lmax = np.max(np.abs(ref), axis=1, keepdims=True)
    err = np.max(np.abs(got - ref) / np.maximum(lmax, 1e-300))
    print(f"[sliding] N={N} stride={stride} restart={restart}: max |dlambda|/lambda_max {err:.3g}, "
          f"iterations <= {inf_.max()}", flush=True)
    assert np.all(inf_ >= 0) and np.all(inf_ <= 40)
    assert err <= tol
    return got, inf_


def _band(H, N, dtype):
    return oracle.band_gram(H, dtype, N).astype(np.float32)


@pytest.mark.parametrize("restart", [1, 7, 64, 1000])
def test_sliding_eigentrack_windows(spec, restart):
    print_case("sliding_eigentrack", restart=restart)
    H = synth.eigentrack(streams=3, T=150, d=256)
    _check(spec, _band(H, 30, "bf16"), 30, 1, 1.0 / 30, restart)


def test_sliding_strides(spec):
    print_case("sliding_strides")
    H = synth.eigentrack(streams=2, T=131, d=96)
    for stride, N, R in [(3, 12, 5), (2, 30, 16), (40, 30, 4)]:
        _check(spec, _band(H, N, "bf16"), N, stride, 1.0 / N, R)


def test_sliding_deflation_paths(spec):
    """Rank 8 windows of 30 rows (22 zero eigenvalues: small weights and close
    poles), windows with zero rows, and runs of repeated rows."""
    print_case("sliding_deflation")
    rng = np.random.default_rng(11)
    low = rng.standard_normal((2, 120, 8)).astype(np.float32)
    _check(spec, _band(low, 30, "f32"), 30, 1, 1.0 / 30, 50)
    z = np.zeros((1, 90, 16), np.float32)
    z[0, 30:45] = rng.standard_normal((15, 16))
    _check(spec, _band(z, 30, "f32"), 30, 1, 1.0 / 30, 64)
    rep = np.repeat(rng.standard_normal((1, 40, 64)).astype(np.float32), 3, axis=1)
    _check(spec, _band(rep, 12, "f32"), 12, 1, 1.0 / 12, 64)


@pytest.mark.parametrize("N", [1, 2, 32, 33, 64])
def test_sliding_window_sizes(spec, N):
    print_case("sliding_sizes", N=N)
    H = synth.eigentrack(streams=2, T=N + 37, d=128)
    _check(spec, _band(H, N, "bf16"), N, 1, 1.0 / N, 16)


def test_sliding_non_finite_step(spec):
    """A NaN step: the windows holding it get NaN and info -1, the chain starts
    over once the step has left, and every other window matches the oracle."""
    import torch
    print_case("sliding_non_finite")
    N, T = 10, 60
    H = synth.eigentrack(streams=1, T=T, d=64)
    band = _band(H, N, "bf16")
    t_bad = 23
    band[0, t_bad, :] = np.nan                       # <h_t, h_{t-j}> for every j
    for j in range(1, N):
        band[0, t_bad + j, j] = np.nan               # <h_{t+j}, h_t>
    w, info = spec.eigvalsh_sliding(dev(band), n=N, scale=1.0 / N, restart=100)
    torch.cuda.synchronize()
    got, inf_ = w.cpu().numpy(), info.cpu().numpy()
    W = T - N + 1
    hit = np.array([wi <= t_bad < wi + N for wi in range(W)])
    assert np.all(np.isnan(got[hit])) and np.all(inf_[hit] == -1)
    clean = ~hit
    assert np.all(np.isfinite(got[clean])) and np.all(inf_[clean] >= 0)
    ok = np.nan_to_num(band, nan=0.0)
    ref = _oracle_spectra(ok, N, 1, 1.0 / N)
    err = np.max(np.abs(got[clean] - ref[clean])) / np.max(np.abs(ref[clean]))
    assert err <= 1e-6


def test_sliding_from_gpu_band_vs_oracle(spec):
    """End to end: the GPU band of bf16 activations, then the sliding spectra,
    against the oracle's window spectra straight from H (1e-4 * lambda_max),
    and against the batched solver on the same band."""
    import torch
    print_case("sliding_end_to_end")
    S, T, d, N = 4, 200, 512, 30
    H = synth.eigentrack(streams=S, T=T, d=d)
    band = spec.gram_window(dev_bf16(H), N=N)
    w, info = spec.eigvalsh_sliding(band, n=N, scale=1.0 / N, restart=64)
    wb, _ = spec.eigvalsh_batched_band(band, n=N, scale=1.0 / N)
    torch.cuda.synchronize()
    got, gb = w.cpu().numpy().astype(np.float64), wb.cpu().numpy().astype(np.float64)
    W = T - N + 1
    worst = 0.0
    for s in range(S):
        ref, _ = oracle.eigvalsh_small(oracle.window_gram(H[s], "bf16", N))
        e = np.max(np.abs(got[s * W:(s + 1) * W] - ref), axis=1) / ref[:, 0]
        worst = max(worst, float(e.max()))
    print(f"[sliding] end to end: max |dlambda|/lambda_max {worst:.3g}", flush=True)
    assert worst <= 1e-4
    assert np.max(np.abs(got - gb) / gb[:, :1]) <= 2e-5
