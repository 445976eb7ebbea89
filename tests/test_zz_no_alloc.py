"""The no-allocation descriptors entry point (spec_descriptors_static) against
spec_descriptors with a caller workspace: the same kernels on the same inputs,
so the records must agree bit for bit.  Two calls in a row on one GPU, the
second with a shorter spectrum and another aspect ratio, so a table left over
from the first call would show."""
import ctypes

import numpy as np
import pytest

from gpu_util import print_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spec():
    import torch
    import weights_bf16_fp32_amd as spec
    assert torch.cuda.is_available()
    spec.lib()
    return spec


def _records(spec, buf):
    return buf.cpu().numpy().view(spec.DESC_DTYPE).reshape(-1)


def _same(a, b):
    return a.tobytes() == b.tobytes()


def test_static_matches_workspace_entry_point_twice(spec):
    import torch
    L = spec.lib()
    rng = np.random.default_rng(71)
    cases = [(4096, 3, 65536, 4096, 8, spec.SIGMA2_GIVEN, torch.float32),   # first: the longer spectrum
             (30, 257, 30, 4096, 8, spec.SIGMA2_MEDIAN, torch.float64)]     # second: shorter, p > n
    for r, batch, n_s, p_d, k, s2m, dt in cases:
        print_case("descriptors_static", r=r, batch=batch, n=n_s, p=p_d)
        lam = np.sort(rng.gamma(2.0, 1.0, size=(batch, r)) * 1.7, axis=1)[:, ::-1].copy()
        lam[0, -3:] = 0.0  # zeros at the end of one spectrum
        w = torch.from_numpy(lam).to(dt).cuda()
        p = spec.DescParams(spec.MODE_EIG, s2m, 1.3, n_s, p_d, k, 0.2, 1e-2, 0.7)
        out_ws = torch.zeros((batch, spec.DESC_DTYPE.itemsize), dtype=torch.uint8, device="cuda")
        out_st = torch.full((batch, spec.DESC_DTYPE.itemsize), 255, dtype=torch.uint8, device="cuda")
        ws = torch.empty((spec.descriptors_workspace(r),), dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        wt = spec.F32 if dt == torch.float32 else spec.F64
        assert L.spec_descriptors_static(stream, w.data_ptr(), wt, batch, r, r, ctypes.byref(p),
                                         out_st.data_ptr()) == 0
        assert L.spec_descriptors(stream, w.data_ptr(), wt, batch, r, r, ctypes.byref(p), out_ws.data_ptr(),
                                  ws.data_ptr(), ws.numel()) == 0
        torch.cuda.synchronize()
        a, b = _records(spec, out_st), _records(spec, out_ws)
        assert _same(a, b)
        assert np.all(np.isfinite(a["H"])) and np.all(np.isfinite(a["mp_w1"]))


def test_static_rejects_longer_spectra_before_launch(spec):
    L = spec.lib()
    p = spec.DescParams(spec.MODE_EIG, spec.SIGMA2_GIVEN, 1.0, 100, 100, 1, 0.2, 1e-2, 0.7)
    fake = 1 << 20  # never dereferenced: the size check fails first
    assert L.spec_descriptors_static(None, fake, spec.F32, 1, 32769, 32769, ctypes.byref(p), fake) == -2
    assert L.spec_descriptors_static(None, fake, spec.F32, 1, 1, 1, ctypes.byref(p), fake) == -1
