"""GPU parity of the S3 tail-pair screen (spec_tail_pair_screen) with the
oracle: the inner products within the fp64 dot-product bound, the kept mask
exact wherever |u_i^T v_j| is not within that bound of eps, the count exact."""
import numpy as np
import pytest

import oracle
from gpu_util import EPS64, dev, print_case
from gen import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spec():
    import weights_bf16_fp32_amd as spec
    spec.lib()
    return spec


def _check(spec, U, V, i0, t, head_dim, eps):
    import torch
    absdot, keep, count = spec.tail_pair_screen(dev(U), dev(V), i0=i0, t=t, head_dim=head_dim, eps=eps)
    torch.cuda.synchronize()
    ref_abs, ref_keep, ref_count = oracle.tail_pair_screen(U, V, i0=i0, t=t, head_dim=head_dim, eps=eps)
    Ut = np.abs(U[:, i0:i0 + t].astype(np.float64))
    Vt = np.abs(V[:, i0:i0 + t].astype(np.float64))
    bound = (U.shape[0] + 2) * EPS64 * (Ut.T @ Vt) + 1e-300
    got = absdot.cpu().numpy()
    assert np.all(np.abs(got - ref_abs) <= bound)
    clear = np.abs(ref_abs - eps) > bound
    kg = keep.cpu().numpy().astype(bool)
    assert np.array_equal(kg[clear], ref_keep[clear])
    if np.all(clear):
        assert int(count.cpu()[0]) == ref_count
    print(f"[screen] t={t} kept {ref_count} of {t * t}; {int(np.sum(~clear))} pairs within the bound of eps",
          flush=True)
    return int(count.cpu()[0])


def test_screen_s3_layer_factors(spec):
    """The S3 workload's own singular vectors (layer 0, d = 4096, f32), the
    page's tail (i >= 0.9 N) and 128-wide heads."""
    print_case("tail_pair_screen_s3", d=4096)
    U, _, V = synth.s3_factors(0, 4096)
    _check(spec, U.astype(np.float32), V.astype(np.float32), i0=3687, t=409, head_dim=128, eps=0.015)


def test_screen_identity_counts(spec):
    print_case("tail_pair_screen_identity")
    eye = np.eye(4096)
    c = _check(spec, eye, eye, i0=3687, t=409, head_dim=128, eps=0.015)
    assert c == sum(b * b - b for b in (25, 128, 128, 128))


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_screen_ragged(spec, dtype):
    """A row count, a tail and a head width that fit no tile, padded leading
    dimensions, and an eps that splits the products."""
    print_case("tail_pair_screen_ragged", dtype=dtype.__name__)
    rng = np.random.default_rng(41)
    n, cols, ld = 300, 150, 160
    U = np.zeros((n, ld), dtype=dtype)
    V = np.zeros((n, ld), dtype=dtype)
    U[:, :cols] = rng.standard_normal((n, cols)) / np.sqrt(n)
    V[:, :cols] = rng.standard_normal((n, cols)) / np.sqrt(n)
    _check(spec, U, V, i0=17, t=133, head_dim=7, eps=0.05)


def test_screen_planted_rotation(spec):
    print_case("tail_pair_screen_planted")
    rng = np.random.default_rng(5)
    Q, _ = np.linalg.qr(rng.standard_normal((64, 64)))
    for theta, kept in [(0.0149, 1), (0.0151, 0)]:
        R = np.eye(64)
        R[60, 60] = R[62, 62] = np.cos(theta)
        R[60, 62], R[62, 60] = -np.sin(theta), np.sin(theta)
        import torch
        absdot, keep, _ = spec.tail_pair_screen(dev(Q), dev(Q @ R), i0=58, t=6, head_dim=8)
        torch.cuda.synchronize()
        assert abs(float(absdot.cpu()[2, 4]) - np.sin(theta)) <= 1e-14
        assert int(keep.cpu()[2, 4]) == kept
