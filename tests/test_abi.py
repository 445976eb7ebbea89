"""The C-ABI library loads, exports every entry point include/spec.h declares,
and rejects bad arguments on the host before anything is enqueued (no GPU
needed: every call here fails validation)."""
import ctypes
import os
import re

import pytest

import weights_bf16_fp32_amd as spec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec.h")

EINVAL, EUNSUPPORTED, EWORKSPACE = -1, -2, -3


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(spec.LIB_PATH):
        from weights_bf16_fp32_amd import build
        build.build()
    return spec.lib()


def test_exports_every_declared_symbol(L):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(spec_\w+)\s*\(", text, re.M))
    assert {"spec_cov_accumulate", "spec_gram_window", "spec_eigvalsh_batched", "spec_eigvalsh_large",
            "spec_descriptors"} <= declared
    for name in declared:
        assert hasattr(L, name), name
    assert set(spec.EXPORTS) == declared
    for name in spec.EXPORTS:  # every entry point is called with declared C types, never ctypes' int default
        assert getattr(L, name).argtypes is not None, name


def test_strerror_and_version(L):
    for s in (0, -1, -2, -3, -4, 7):
        assert len(L.spec_strerror(s)) > 0
    assert L.spec_version() == b"0.1.0"


def test_struct_layouts():
    assert ctypes.sizeof(spec.BatchSrc) == 56
    assert ctypes.sizeof(spec.DescParams) == 64
    assert spec.DESC_DTYPE.itemsize == 144


FAKE = 1 << 20  # an aligned non-null address; never dereferenced because validation fails first


def test_cov_accumulate_validation(L):
    f = L.spec_cov_accumulate
    assert f(None, FAKE, spec.BF16, 10, 8, 8, None, spec.F32, 8, 1.0, 0.0) == EINVAL  # C NULL
    assert f(None, None, spec.BF16, 10, 8, 8, FAKE, spec.F32, 8, 1.0, 0.0) == EINVAL  # X NULL, n > 0
    assert f(None, FAKE, spec.BF16, 10, 8, 4, FAKE, spec.F32, 8, 1.0, 0.0) == EINVAL  # ldx < d
    assert f(None, FAKE, spec.BF16, 10, 8, 8, FAKE, spec.F32, 7, 1.0, 0.0) == EINVAL  # ldc < d
    assert f(None, FAKE, spec.BF16, -1, 8, 8, FAKE, spec.F32, 8, 1.0, 0.0) == EINVAL
    assert f(None, FAKE, spec.BF16, 10, 0, 8, FAKE, spec.F32, 8, 1.0, 0.0) == EINVAL
    assert f(None, FAKE, spec.BF16, 10, 8, 8, FAKE, spec.F64, 8, 1.0, 0.0) == EUNSUPPORTED
    assert f(None, FAKE, spec.F64, 10, 8, 8, FAKE, spec.F64, 8, 1.0, 0.0) == EUNSUPPORTED
    assert f(None, FAKE + 1, spec.F32, 10, 8, 8, FAKE, spec.F32, 8, 1.0, 0.0) == EINVAL  # misaligned
    assert f(None, FAKE, spec.F32, 10, 8, 8, FAKE, spec.F32, 8, float("nan"), 0.0) == EINVAL


def test_gram_validation(L):
    f = L.spec_gram_window
    ok = (None, FAKE, spec.BF16, 2, 100, 64, 64, 6400, 30, 1, 1 / 30, spec.GRAM_BAND, FAKE)
    bad = [
        (5, 65), (5, 0), (8, 0), (1, 101),  # N > 64, N = 0, stride 0, T < N
    ]
    for idx, val in [(8, 65), (8, 0), (9, 0)]:
        a = list(ok); a[idx] = val
        assert f(*a) == EINVAL
    a = list(ok); a[4] = 20  # T < N
    assert f(*a) == EINVAL
    a = list(ok); a[6] = 32  # ld_t < d
    assert f(*a) == EINVAL
    a = list(ok); a[2] = spec.F64
    assert f(*a) == EUNSUPPORTED
    a = list(ok); a[11] = 7
    assert f(*a) == EINVAL
    a = list(ok); a[12] = None
    assert f(*a) == EINVAL


def test_batched_validation(L):
    f = L.spec_eigvalsh_batched
    src = spec.BatchSrc(spec.SRC_DENSE, FAKE, 30, 900, 0, 0, 1, 1.0)
    assert f(None, ctypes.byref(src), 4, 65, FAKE, None) == EUNSUPPORTED
    assert f(None, ctypes.byref(src), 4, 0, FAKE, None) == EINVAL
    assert f(None, ctypes.byref(src), 4, 31, FAKE, None) == EINVAL  # lda < n
    band = spec.BatchSrc(spec.SRC_BAND, FAKE, 0, 0, 2, 100, 1, 1 / 30)
    assert f(None, ctypes.byref(band), 2 * 70, 30, FAKE, None) == EINVAL  # batch != S * W
    assert f(None, None, 4, 30, FAKE, None) == EINVAL


def test_sliding_validation(L):
    f = L.spec_eigvalsh_sliding
    band = spec.BatchSrc(spec.SRC_BAND, FAKE, 0, 0, 2, 100, 1, 1 / 30)
    dense = spec.BatchSrc(spec.SRC_DENSE, FAKE, 30, 900, 0, 0, 1, 1.0)
    assert f(None, ctypes.byref(dense), 4, 30, 64, FAKE, None) == EINVAL  # band sources only
    assert f(None, ctypes.byref(band), 2 * 71, 30, 0, FAKE, None) == EINVAL  # restart < 1
    assert f(None, ctypes.byref(band), 2 * 70, 30, 64, FAKE, None) == EINVAL  # batch != S * W
    assert f(None, ctypes.byref(band), 2 * 71, 65, 64, FAKE, None) == EUNSUPPORTED
    assert f(None, ctypes.byref(band), 2 * 71, 0, 64, FAKE, None) == EINVAL
    assert f(None, ctypes.byref(band), 2 * 71, 30, 64, FAKE + 2, None) == EINVAL  # misaligned w
    assert f(None, ctypes.byref(band), 2 * 71, 30, 64, None, None) == EINVAL
    short = spec.BatchSrc(spec.SRC_BAND, FAKE, 0, 0, 2, 20, 1, 1 / 30)
    assert f(None, ctypes.byref(short), 0, 30, 64, FAKE, None) == EINVAL  # T < n


def test_eigh_batched_validation(L):
    f = L.spec_eigh_batched
    dense = spec.BatchSrc(spec.SRC_DENSE, FAKE, 30, 900, 0, 0, 1, 1.0)
    assert f(None, ctypes.byref(dense), 4, 30, FAKE, None, None) == EINVAL  # V NULL
    assert f(None, ctypes.byref(dense), 4, 33, FAKE, FAKE, None) == EUNSUPPORTED  # n > 32
    assert f(None, ctypes.byref(dense), 4, 0, FAKE, FAKE, None) == EINVAL
    assert f(None, ctypes.byref(dense), 4, 30, FAKE, FAKE + 2, None) == EINVAL  # misaligned V
    short = spec.BatchSrc(spec.SRC_DENSE, FAKE, 29, 900, 0, 0, 1, 1.0)
    assert f(None, ctypes.byref(short), 4, 30, FAKE, FAKE, None) == EINVAL  # lda < n
    band = spec.BatchSrc(spec.SRC_BAND, FAKE, 0, 0, 2, 100, 1, 1.0 / 30)
    assert f(None, ctypes.byref(band), 2 * 71 + 1, 30, FAKE, FAKE, None) == EINVAL  # batch != streams * W


def test_eigh_large_validation(L):
    b = ctypes.c_size_t(0)
    f = L.spec_eigh_large_workspace
    assert f(1000, spec.F32, 0, ctypes.byref(b)) == EINVAL  # k < 1
    assert f(1000, spec.F32, 1001, ctypes.byref(b)) == EINVAL  # k > n
    assert f(9000, spec.F32, 10, ctypes.byref(b)) == EUNSUPPORTED  # n past the vector path's limit
    assert f(1000, spec.BF16, 10, ctypes.byref(b)) == EUNSUPPORTED
    assert f(1000, spec.F32, 10, ctypes.byref(b)) == 0 and b.value > 0
    small = ctypes.c_size_t(0)
    assert L.spec_eigvalsh_large_workspace(1000, spec.F32, ctypes.byref(small)) == 0 and small.value < b.value
    g = L.spec_eigh_large
    need = b.value
    assert g(None, FAKE, spec.F32, 1000, 1000, FAKE, FAKE, 5, 10, FAKE, need, None) == EINVAL  # ldz < k
    assert g(None, FAKE, spec.F32, 1000, 1000, FAKE, None, 10, 10, FAKE, need, None) == EINVAL  # Z NULL
    assert g(None, FAKE, spec.F32, 1000, 1000, FAKE, FAKE, 10, 10, FAKE, need - 1, None) == EWORKSPACE
    assert g(None, FAKE, spec.F32, 1000, 1000, FAKE, FAKE + 2, 10, 10, FAKE, need, None) == EINVAL  # misaligned Z
    assert g(None, FAKE, spec.F32, 1000, 1000, FAKE, FAKE, 1 << 19, 10, FAKE, need, None) == EUNSUPPORTED  # Z past 2^31 bytes


def test_alignment_codes(L):
    """Every device pointer must be aligned to its element size, workspaces to 256
    bytes, and the large eigensolver's A to 16 bytes; anything less is SPEC_EINVAL."""
    cov = L.spec_cov_accumulate
    assert cov(None, FAKE + 1, spec.BF16, 10, 8, 8, FAKE, spec.F32, 8, 1.0, 0.0) == EINVAL  # bf16 X, odd
    assert cov(None, FAKE + 2, spec.F32, 10, 8, 8, FAKE, spec.F32, 8, 1.0, 0.0) == EINVAL   # f32 X, 2 bytes
    assert cov(None, FAKE, spec.F32, 10, 8, 8, FAKE + 4, spec.F64, 8, 1.0, 0.0) == EINVAL   # f64 C, 4 bytes
    gram = L.spec_gram_window
    assert gram(None, FAKE + 1, spec.BF16, 2, 100, 64, 64, 6400, 30, 1, 1.0, spec.GRAM_BAND, FAKE) == EINVAL
    assert gram(None, FAKE, spec.BF16, 2, 100, 64, 64, 6400, 30, 1, 1.0, spec.GRAM_BAND, FAKE + 2) == EINVAL
    bat = L.spec_eigvalsh_batched
    src = spec.BatchSrc(spec.SRC_DENSE, FAKE + 2, 30, 900, 0, 0, 1, 1.0)
    assert bat(None, ctypes.byref(src), 4, 30, FAKE, None) == EINVAL
    src = spec.BatchSrc(spec.SRC_DENSE, FAKE, 30, 900, 0, 0, 1, 1.0)
    assert bat(None, ctypes.byref(src), 4, 30, FAKE, FAKE + 2) == EINVAL  # info
    b = ctypes.c_size_t(0)
    L.spec_eigvalsh_large_workspace(512, spec.F32, ctypes.byref(b))
    big = L.spec_eigvalsh_large
    assert big(None, FAKE + 4, spec.F32, 512, 512, FAKE, FAKE, b.value, None) == EINVAL   # A: 16 bytes
    assert big(None, FAKE, spec.F32, 512, 512, FAKE + 2, FAKE, b.value, None) == EINVAL   # w
    assert big(None, FAKE, spec.F32, 512, 512, FAKE, FAKE + 128, b.value, None) == EINVAL  # ws: 256 bytes
    p = spec.DescParams(0, 0, 1.0, 64, 32, 1, 0.2, 1e-2, 0.7)
    L.spec_descriptors_workspace(32, ctypes.byref(b))
    desc = L.spec_descriptors
    assert desc(None, FAKE + 4, spec.F64, 1, 32, 32, ctypes.byref(p), FAKE, FAKE, b.value) == EINVAL  # w
    assert desc(None, FAKE, spec.F64, 1, 32, 32, ctypes.byref(p), FAKE + 4, FAKE, b.value) == EINVAL  # out
    assert desc(None, FAKE, spec.F64, 1, 32, 32, ctypes.byref(p), FAKE, FAKE + 8, b.value) == EINVAL  # ws


def test_large_validation(L):
    b = ctypes.c_size_t(0)
    assert L.spec_eigvalsh_large_workspace(4096, spec.F32, ctypes.byref(b)) == 0 and b.value > 0
    assert L.spec_eigvalsh_large_workspace(4096, spec.BF16, ctypes.byref(b)) == EUNSUPPORTED
    assert L.spec_eigvalsh_large_workspace(0, spec.F32, ctypes.byref(b)) == EINVAL
    assert L.spec_eigvalsh_large_workspace(40000, spec.F32, ctypes.byref(b)) == EUNSUPPORTED
    assert L.spec_eigvalsh_large_workspace(8193, spec.F64, ctypes.byref(b)) == EUNSUPPORTED
    L.spec_eigvalsh_large_workspace(512, spec.F64, ctypes.byref(b))
    f = L.spec_eigvalsh_large
    assert f(None, FAKE, spec.F64, 512, 512, FAKE, FAKE, b.value - 1, None) == EWORKSPACE
    assert f(None, FAKE, spec.F64, 512, 512, FAKE, None, b.value, None) == EWORKSPACE
    assert f(None, FAKE, spec.F64, 512, 500, FAKE, FAKE, b.value, None) == EINVAL
    assert f(None, FAKE, spec.F64, 512, 1 << 22, FAKE, FAKE, b.value, None) == EINVAL  # lda too large


def test_descriptors_validation(L):
    b = ctypes.c_size_t(0)
    assert L.spec_descriptors_workspace(30, ctypes.byref(b)) == 0 and b.value >= 30 * 8
    p = spec.DescParams(0, 0, 1.0, 64, 32, 1, 0.2, 1e-2, 0.7)
    f = L.spec_descriptors
    assert f(None, FAKE, spec.F32, 1, 32, 32, ctypes.byref(p), FAKE, FAKE, 8, ) == EWORKSPACE
    for field, val in [("k", 0), ("k", 32), ("n_samples", 0), ("top_frac", 1.5), ("sigma2", -1.0),
                       ("sigma2_mode", 5), ("small_rel", -1.0)]:
        q = spec.DescParams(0, 0, 1.0, 64, 32, 1, 0.2, 1e-2, 0.7)
        setattr(q, field, val)
        assert f(None, FAKE, spec.F32, 1, 32, 32, ctypes.byref(q), FAKE, FAKE, 4096) == EINVAL, field
    assert f(None, FAKE, spec.BF16, 1, 32, 32, ctypes.byref(p), FAKE, FAKE, 4096) == EUNSUPPORTED
    assert f(None, FAKE, spec.F32, 1, 1, 1, ctypes.byref(p), FAKE, FAKE, 4096) == EINVAL


def test_postproc_validation(L):
    f = L.spec_desc_smooth
    assert f(None, FAKE, 4, 10, 0.0, FAKE + 4096 * 144) == EINVAL  # alpha = 0
    assert f(None, FAKE, 4, 10, 1.5, FAKE + 4096 * 144) == EINVAL  # alpha > 1
    assert f(None, FAKE, 4, 0, 0.5, FAKE + 4096 * 144) == EINVAL   # W = 0
    assert f(None, FAKE, 4, 10, 0.5, FAKE + 144) == EINVAL         # out overlaps in
    assert f(None, None, 4, 10, 0.5, FAKE) == EINVAL
    g = L.spec_spectrum_robust
    ok = dict(sigma2_mode=0, bins=16, sigma2=1.0, n_samples=64, p_dim=32, winsor_frac=0.05, mad_k=3.0)
    for field, val in [("bins", 0), ("bins", 65), ("winsor_frac", 0.6), ("winsor_frac", -0.1), ("mad_k", 0.0),
                       ("sigma2_mode", 4), ("sigma2", 0.0), ("n_samples", 0), ("p_dim", 0)]:
        kw = dict(ok)
        kw[field] = val
        p = spec.RobustParams(*[kw[k] for k, _ in spec.RobustParams._fields_])
        assert g(None, FAKE, spec.F32, 1, 32, 32, ctypes.byref(p), FAKE) == EINVAL, field
    p = spec.RobustParams(*[ok[k] for k, _ in spec.RobustParams._fields_])
    assert g(None, FAKE, spec.BF16, 1, 32, 32, ctypes.byref(p), FAKE) == EUNSUPPORTED
    assert g(None, FAKE, spec.F32, 1, 1, 1, ctypes.byref(p), FAKE) == EINVAL   # r < 2
    assert g(None, FAKE, spec.F32, 1, 32, 31, ctypes.byref(p), FAKE) == EINVAL  # ldw < r


def test_topk_validation(L):
    b = ctypes.c_size_t(0)
    assert L.spec_eigvalsh_large_workspace(512, spec.F32, ctypes.byref(b)) == 0
    f = L.spec_eigvalsh_topk
    assert f(None, FAKE, spec.F64, 512, 512, FAKE, 2, FAKE, FAKE, b.value) == EUNSUPPORTED
    assert f(None, FAKE, spec.F32, 32, 32, FAKE, 2, FAKE, FAKE, b.value) == EINVAL     # n < 64
    assert f(None, FAKE, spec.F32, 512, 500, FAKE, 2, FAKE, FAKE, b.value) == EINVAL   # lda < n
    assert f(None, FAKE, spec.F32, 512, 512, FAKE, 17, FAKE, FAKE, b.value) == EINVAL  # q > 16
    assert f(None, FAKE, spec.F32, 512, 512, None, 2, FAKE, FAKE, b.value) == EINVAL
    assert f(None, FAKE, spec.F32, 512, 512, FAKE, 2, FAKE, FAKE, b.value - 1) == EWORKSPACE


def test_eigvecs_topk_validation(L):
    b = ctypes.c_size_t(0)
    assert L.spec_eigvalsh_large_workspace(512, spec.F32, ctypes.byref(b)) == 0
    f = L.spec_eigvecs_topk
    ok = (None, FAKE, spec.F32, 512, 512, FAKE, 2, FAKE, FAKE, 32, FAKE, b.value, None)
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a2=spec.F64) == EUNSUPPORTED
    assert call(a3=32, a4=32) == EINVAL          # n < 64
    assert call(a4=500) == EINVAL                # lda < n
    assert call(a6=17) == EINVAL                 # q > 16
    assert call(a6=-1) == EINVAL
    assert call(a8=None) == EINVAL               # no P
    assert call(a9=31) == EINVAL                 # ldp < 32
    assert call(a9=1 << 22) == EINVAL
    assert call(a11=b.value - 1) == EWORKSPACE
    assert call(a12=FAKE + 2) == EINVAL          # info not 4-byte aligned


def test_project_weight_validation(L):
    b = ctypes.c_size_t(0)
    assert L.spec_project_weight_workspace(4096, ctypes.byref(b)) == 0 and b.value > 4096 * 32 * 4
    assert L.spec_project_weight_workspace(0, ctypes.byref(b)) == EINVAL
    assert L.spec_project_weight_workspace(512, ctypes.byref(b)) == 0  # the size for d = 512 below
    f = L.spec_project_weight
    ok = [None, FAKE, spec.BF16, 512, 512, FAKE, 32, 32, FAKE, 32, FAKE, 32, FAKE, b.value]
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a2=spec.F64) == EUNSUPPORTED
    assert call(a1=None) == EINVAL
    assert call(a3=0) == EINVAL                   # d < 1
    assert call(a7=0) == EINVAL                   # k < 1
    assert call(a7=33) == EINVAL                  # k > 32
    assert call(a3=16, a4=16, a7=17) == EINVAL    # k > d
    assert call(a4=500) == EINVAL                 # ldw < d
    assert call(a4=516) == EINVAL                 # bf16 rows not 16-byte multiples
    assert call(a6=31) == EINVAL                  # ldp < k
    assert call(a9=31) == EINVAL                  # ldo < k
    assert call(a11=31) == EINVAL                 # ldx < k with X given
    assert call(a1=FAKE + 8) == EINVAL            # W not 16-byte aligned
    assert call(a13=b.value - 1) == EWORKSPACE


def test_tail_pair_screen_validation(L):
    f = L.spec_tail_pair_screen
    ok = [None, FAKE, FAKE, spec.F32, 4096, 4096, 4096, 3687, 409, 128, 0.015, FAKE, 409, FAKE, 409, FAKE]
    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a3=spec.BF16) == EUNSUPPORTED
    assert call(a8=410) == EINVAL             # i0 + t > ldu
    assert call(a8=0) == EINVAL               # t < 1
    assert call(a9=0) == EINVAL               # head_dim < 1
    assert call(a10=0.0) == EINVAL            # eps <= 0
    assert call(a10=float("inf")) == EINVAL
    assert call(a14=408) == EINVAL            # ldk < t
    assert call(a12=10) == EINVAL             # ldo < t with absdot given
    assert call(a13=None) == EINVAL           # keep NULL
    assert call(a1=FAKE + 2) == EINVAL        # f32 U misaligned
    assert call(a15=FAKE + 4) == EINVAL       # count misaligned
