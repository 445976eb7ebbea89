"""Python binding of the gfx950 spectral library (libspec.so, C ABI in include/spec.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  The library
is loaded on first use and a missing library raises immediately; there is no
fallback of any kind.

    import weights_bf16_fp32_amd as spec
    spec.cov_accumulate(X, C, alpha=1/n, beta=0.0)          # C <- beta C + alpha X^T X (lower)
    band = spec.gram_window(H, N=30)                          # [S, T, N] <h_t, h_{t-j}>
    w, info = spec.eigvalsh_batched_band(band, n=30, scale=1/30)
    w = spec.eigvalsh_large(C)                                # destroys C
    rec = spec.descriptors(w, n_samples=n, p_dim=d, k=1)      # structured numpy array
    sm = spec.desc_smooth(raw_records, streams=S, W=W, alpha=0.3)  # smoothed descriptor series
    rb = spec.spectrum_robust(w, n_samples=n, p_dim=d)        # median/MAD/winsor/log/KL statistics
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "SpecError", "lib", "cov_accumulate", "gram_window", "eigvalsh_batched_dense",
    "eigvalsh_batched_band", "eigvalsh_large", "eigvalsh_large_workspace", "descriptors",
    "descriptors_workspace", "DESC_DTYPE", "desc_smooth", "spectrum_robust", "ROBUST_DTYPE", "eigvalsh_topk",
    "eigvecs_topk", "project_weight", "project_weight_workspace",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspec.so")

BF16, F32, F64 = 0, 1, 2
GRAM_BAND, GRAM_DENSE = 0, 1
SRC_DENSE, SRC_BAND = 0, 1
MODE_EIG, MODE_SINGULAR = 0, 1
SIGMA2_GIVEN, SIGMA2_MEDIAN, SIGMA2_MEAN, SIGMA2_WINSOR = 0, 1, 2, 3
FLAG_NONFINITE, FLAG_GK_UNDEF, FLAG_S_ZERO, FLAG_HELD = 1, 2, 4, 8

_DESC_FIELDS_F = ["S", "H", "erank", "m1", "gk", "g1", "sigma2", "lambda_plus", "mp_w1",
                  "top_energy", "top_sigma_share", "tail_head", "tail_min", "sigma1"]
_DESC_FIELDS_I = ["n_above", "n_small", "r_pos", "flags"]
DESC_DTYPE = np.dtype([(f, "<f8") for f in _DESC_FIELDS_F] + [(f, "<i8") for f in _DESC_FIELDS_I])
assert DESC_DTYPE.itemsize == 144
_ROBUST_FIELDS_F = ["median", "sigma2_winsor", "mad", "log_mean", "log_std", "sigma2", "kl_mp"]
ROBUST_DTYPE = np.dtype([(f, "<f8") for f in _ROBUST_FIELDS_F] + [("n_mad", "<i8"), ("flags", "<i8")])
assert ROBUST_DTYPE.itemsize == 72


KT = {"syrk": 0, "gram": 1, "small_eig": 2, "desc": 3, "symm": 4, "syr2k": 5, "panel": 6, "bulge": 7,
      "tridiag": 8}


def timing_enable(kernels) -> None:
    """Start timing every launch of the named kernels (keys of KT) with HIP
    events on their own stream; an empty list stops."""
    m = 0
    for k in kernels:
        m |= 1 << KT[k]
    _check(lib().spec_timing_enable(m))


def timing_read(kernel: str):
    """(total device ms, timed launches) of one kernel since timing_enable."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(lib().spec_timing_read(KT[kernel], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


class SpecError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"spec status {status}: {msg}")
        self.status = status


class BatchSrc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("a", ctypes.c_void_p), ("lda", ctypes.c_int64),
                ("stride_a", ctypes.c_int64), ("streams", ctypes.c_int64), ("T", ctypes.c_int64),
                ("stride", ctypes.c_int), ("scale", ctypes.c_float)]


class DescParams(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("sigma2_mode", ctypes.c_int), ("sigma2", ctypes.c_double),
                ("n_samples", ctypes.c_int64), ("p_dim", ctypes.c_int64), ("k", ctypes.c_int64),
                ("top_frac", ctypes.c_double), ("small_rel", ctypes.c_double),
                ("tail_frac", ctypes.c_double)]


class RobustParams(ctypes.Structure):
    _fields_ = [("sigma2_mode", ctypes.c_int32), ("bins", ctypes.c_int32), ("sigma2", ctypes.c_double),
                ("n_samples", ctypes.c_int64), ("p_dim", ctypes.c_int64), ("winsor_frac", ctypes.c_double),
                ("mad_k", ctypes.c_double)]


EXPORTS = ["spec_strerror", "spec_version", "spec_cov_accumulate", "spec_gram_window",
           "spec_eigvalsh_batched", "spec_eigvalsh_large_workspace", "spec_eigvalsh_large",
           "spec_descriptors_workspace", "spec_descriptors", "spec_desc_smooth", "spec_spectrum_robust",
           "spec_eigvalsh_topk", "spec_eigvecs_topk", "spec_project_weight_workspace",
           "spec_project_weight", "spec_timing_enable", "spec_timing_read", "spec_descriptors_static", "spec_tail_pair_screen", "spec_eigvalsh_batched_desc",
           "spec_eigvalsh_sliding", "spec_eigh_large_workspace", "spec_eigh_large", "spec_eigh_batched"]

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libspec.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(weights_bf16_fp32_amd/build.py); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.spec_strerror.argtypes = [i32]
        L.spec_strerror.restype = ctypes.c_char_p
        L.spec_version.argtypes = []
        L.spec_version.restype = ctypes.c_char_p
        L.spec_cov_accumulate.argtypes = [vp, vp, i32, i64, i64, i64, vp, i32, i64, dbl, dbl]
        L.spec_gram_window.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, i32, i32, dbl, i32, vp]
        L.spec_eigvalsh_batched.argtypes = [vp, ctypes.POINTER(BatchSrc), i64, i32, vp, vp]
        L.spec_eigvalsh_large_workspace.argtypes = [i64, i32, ctypes.POINTER(ctypes.c_size_t)]
        L.spec_eigvalsh_large.argtypes = [vp, vp, i32, i64, i64, vp, vp, ctypes.c_size_t, vp]
        L.spec_eigh_large_workspace.argtypes = [i64, i32, i64, ctypes.POINTER(ctypes.c_size_t)]
        L.spec_eigh_large.argtypes = [vp, vp, i32, i64, i64, vp, vp, i64, i64, vp, ctypes.c_size_t, vp]
        L.spec_descriptors_workspace.argtypes = [i64, ctypes.POINTER(ctypes.c_size_t)]
        L.spec_descriptors.argtypes = [vp, vp, i32, i64, i64, i64, ctypes.POINTER(DescParams), vp, vp,
                                       ctypes.c_size_t]
        L.spec_desc_smooth.argtypes = [vp, vp, i64, i64, dbl, vp]
        L.spec_eigvalsh_topk.argtypes = [vp, vp, i32, i64, i64, vp, i32, vp, vp, ctypes.c_size_t]
        L.spec_eigvecs_topk.argtypes = [vp, vp, i32, i64, i64, vp, i32, vp, vp, i64, vp, ctypes.c_size_t, vp]
        L.spec_project_weight_workspace.argtypes = [i64, ctypes.POINTER(ctypes.c_size_t)]
        L.spec_project_weight.argtypes = [vp, vp, i32, i64, i64, vp, i64, i32, vp, i64, vp, i64, vp,
                                          ctypes.c_size_t]
        L.spec_spectrum_robust.argtypes = [vp, vp, i32, i64, i64, i64, ctypes.POINTER(RobustParams), vp]
        L.spec_eigvalsh_batched_desc.argtypes = [vp, ctypes.POINTER(BatchSrc), i64, i32, vp, vp,
                                                  ctypes.POINTER(DescParams), vp, vp, ctypes.c_size_t]
        L.spec_tail_pair_screen.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, i64, dbl, vp, i64, vp, i64,
                                             vp]
        L.spec_descriptors_static.argtypes = [vp, vp, i32, i64, i64, i64, ctypes.POINTER(DescParams), vp]
        L.spec_eigvalsh_sliding.argtypes = [vp, ctypes.POINTER(BatchSrc), i64, i32, i32, vp, vp]
        L.spec_eigh_batched.argtypes = [vp, ctypes.POINTER(BatchSrc), i64, i32, vp, vp, vp]
        L.spec_timing_enable.argtypes = [ctypes.c_uint]
        L.spec_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        for f in EXPORTS[2:]:
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise SpecError(status, lib().spec_strerror(status).decode())


def _torch():
    import torch
    return torch


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float64:
        return F64
    raise SpecError(-2, f"unsupported dtype {t.dtype}")


def _dev(t):
    if not t.is_cuda:
        raise SpecError(-1, "tensor must be on the GPU")
    return t.data_ptr()


def cov_accumulate(X, C, alpha: float = 1.0, beta: float = 0.0):
    """C <- beta C + alpha X^T X on the lower triangle of C (X: [n, d], C: [d, d])."""
    n, d = X.shape
    if X.stride(1) != 1 or C.stride(1) != 1:
        raise SpecError(-1, "inner dimension must be contiguous")
    _check(lib().spec_cov_accumulate(_stream(), _dev(X), _dt(X), n, d, X.stride(0), _dev(C), _dt(C),
                                     C.stride(0), float(alpha), float(beta)))
    return C


def gram_window(H, N: int, stride: int = 1, scale: float = 1.0, layout: int = GRAM_BAND, out=None):
    """Band <h_t, h_{t-j}> [S, T, N] (layout BAND) or dense scale*H_w H_w^T [S*W, N, N]."""
    torch = _torch()
    if H.dim() == 2:
        H = H.unsqueeze(0)
    S, T, d = H.shape
    if H.stride(2) != 1:
        raise SpecError(-1, "feature dimension must be contiguous")
    if out is None:
        if layout == GRAM_BAND:
            out = torch.empty((S, T, N), dtype=torch.float32, device=H.device)
        else:
            W = (T - N) // stride + 1
            out = torch.empty((S * W, N, N), dtype=torch.float32, device=H.device)
    _check(lib().spec_gram_window(_stream(), _dev(H), _dt(H), S, T, d, H.stride(1), H.stride(0), N, stride,
                                  float(scale), layout, _dev(out)))
    return out


def _batched(src: BatchSrc, batch: int, n: int, w, info, device):
    torch = _torch()
    if w is None:
        w = torch.empty((batch, n), dtype=torch.float32, device=device)
    if info is None:
        info = torch.empty((batch,), dtype=torch.int32, device=device)
    _check(lib().spec_eigvalsh_batched(_stream(), ctypes.byref(src), batch, n, _dev(w), _dev(info)))
    return w, info


def eigvalsh_batched_dense(A, w=None, info=None):
    """Eigenvalues (descending) of A [batch, n, n] f32 (lower triangle read).
    info[b] = bisection rounds, or -1 for a matrix with a non-finite entry."""
    if A.dim() == 2:
        A = A.unsqueeze(0)
    batch, n, _ = A.shape
    src = BatchSrc(SRC_DENSE, _dev(A), A.stride(1), A.stride(0), 0, 0, 1, 1.0)
    return _batched(src, batch, n, w, info, A.device)


def eigvalsh_batched_band(band, n: int, scale: float, stride: int = 1, w=None, info=None):
    """Eigenvalues of every window's Gram scale * G_w from the band [S, T, n] of gram_window."""
    S, T, N = band.shape
    if N != n or not band.is_contiguous():
        raise SpecError(-1, "band must be a contiguous [streams, T, n] tensor")
    batch = S * ((T - n) // stride + 1)
    src = BatchSrc(SRC_BAND, _dev(band), 0, 0, S, T, stride, float(scale))
    return _batched(src, batch, n, w, info, band.device)


def _eigh_batched(src, batch, n, w, V, info, device):
    torch = _torch()
    if w is None:
        w = torch.empty((batch, n), dtype=torch.float32, device=device)
    if V is None:
        V = torch.empty((batch, n, n), dtype=torch.float32, device=device)
    if info is None:
        info = torch.empty((batch,), dtype=torch.int32, device=device)
    _check(lib().spec_eigh_batched(_stream(), ctypes.byref(src), batch, n, _dev(w), _dev(V), _dev(info)))
    return w, V, info


def eigh_batched_dense(A, w=None, V=None, info=None):
    """Eigenvalues (descending) and eigenvectors of A [batch, n, n] f32 (lower
    triangle read, n <= 32): V[b][:, j] belongs to w[b][j].  info[b] = Jacobi
    sweeps, -2 (sweep limit) or -1 (non-finite entry)."""
    if A.dim() == 2:
        A = A.unsqueeze(0)
    batch, n, _ = A.shape
    src = BatchSrc(SRC_DENSE, _dev(A), A.stride(1), A.stride(0), 0, 0, 1, 1.0)
    return _eigh_batched(src, batch, n, w, V, info, A.device)


def eigh_batched_band(band, n: int, scale: float, stride: int = 1, w=None, V=None, info=None):
    """Eigenpairs of every window's Gram scale * G_w from the band [S, T, n] of gram_window."""
    S, T, N = band.shape
    if N != n or not band.is_contiguous():
        raise SpecError(-1, "band must be a contiguous [streams, T, n] tensor")
    batch = S * ((T - n) // stride + 1)
    src = BatchSrc(SRC_BAND, _dev(band), 0, 0, S, T, stride, float(scale))
    return _eigh_batched(src, batch, n, w, V, info, band.device)


def eigvalsh_sliding(band, n: int, scale: float, stride: int = 1, restart: int = 64, w=None, info=None):
    """The spectra of eigvalsh_batched_band by rank-one down/up-dates along each
    stream (fp64, a fresh start every `restart` windows).  info[b] = largest
    secular iteration count of the window's updates, or -1 (non-finite step)."""
    torch = _torch()
    S, T, N = band.shape
    if N != n or not band.is_contiguous():
        raise SpecError(-1, "band must be a contiguous [streams, T, n] tensor")
    batch = S * ((T - n) // stride + 1)
    src = BatchSrc(SRC_BAND, _dev(band), 0, 0, S, T, stride, float(scale))
    if w is None:
        w = torch.empty((batch, n), dtype=torch.float32, device=band.device)
    if info is None:
        info = torch.empty((batch,), dtype=torch.int32, device=band.device)
    _check(lib().spec_eigvalsh_sliding(_stream(), ctypes.byref(src), batch, n, int(restart), _dev(w), _dev(info)))
    return w, info


def eigh_large_workspace(n: int, dtype, k: int) -> int:
    torch = _torch()
    t = F32 if dtype == torch.float32 else F64
    b = ctypes.c_size_t(0)
    _check(lib().spec_eigh_large_workspace(n, t, k, ctypes.byref(b)))
    return b.value


def eigh_large(A, k: int, w=None, Z=None, ws=None, info=None):
    """All eigenvalues (descending) of the symmetric A [n, n] (lower triangle
    read, A destroyed) and the eigenvectors of the k largest, Z [n, k] (column j
    for w[j])."""
    torch = _torch()
    n = A.shape[0]
    if A.stride(1) != 1:
        raise SpecError(-1, "A must be row-major")
    if w is None:
        w = torch.empty((n,), dtype=A.dtype, device=A.device)
    if Z is None:
        Z = torch.empty((n, k), dtype=A.dtype, device=A.device)
    if ws is None:
        ws = torch.empty((eigh_large_workspace(n, A.dtype, k),), dtype=torch.uint8, device=A.device)
    ip = _dev(info) if info is not None else None
    _check(lib().spec_eigh_large(_stream(), _dev(A), _dt(A), n, A.stride(0), _dev(w), _dev(Z), Z.stride(0), k,
                                 _dev(ws), ws.numel(), ip))
    return w, Z


def eigvalsh_large_workspace(n: int, dtype) -> int:
    torch = _torch()
    t = F32 if dtype == torch.float32 else F64
    b = ctypes.c_size_t(0)
    _check(lib().spec_eigvalsh_large_workspace(n, t, ctypes.byref(b)))
    return b.value


def eigvalsh_large(A, w=None, ws=None, info=None):
    """Eigenvalues (descending) of the symmetric A [n, n] (lower triangle read, A destroyed)."""
    torch = _torch()
    n = A.shape[0]
    if A.stride(1) != 1:
        raise SpecError(-1, "A must be row-major")
    if w is None:
        w = torch.empty((n,), dtype=A.dtype, device=A.device)
    if ws is None:
        ws = torch.empty((eigvalsh_large_workspace(n, A.dtype),), dtype=torch.uint8, device=A.device)
    ip = _dev(info) if info is not None else None
    _check(lib().spec_eigvalsh_large(_stream(), _dev(A), _dt(A), n, A.stride(0), _dev(w), _dev(ws),
                                     ws.numel(), ip))
    return w


def descriptors_workspace(r: int) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().spec_descriptors_workspace(r, ctypes.byref(b)))
    return b.value


def descriptors(w, *, n_samples: int, p_dim: int, k: int = 1, mode: int = MODE_EIG,
                sigma2: float = 1.0, sigma2_mode: int = SIGMA2_GIVEN, top_frac: float = 0.2,
                small_rel: float = 1e-2, tail_frac: float = 0.7, out=None, ws=None, to_host: bool = True):
    """Descriptors of each row of w [batch, r] (sorted descending).  Returns a numpy
    structured array of DESC_DTYPE (or the raw device buffer if to_host is False)."""
    torch = _torch()
    if w.dim() == 1:
        w = w.unsqueeze(0)
    batch, r = w.shape
    if out is None:
        out = torch.empty((batch, DESC_DTYPE.itemsize), dtype=torch.uint8, device=w.device)
    if ws is None:
        ws = torch.empty((descriptors_workspace(r),), dtype=torch.uint8, device=w.device)
    p = DescParams(mode, sigma2_mode, float(sigma2), int(n_samples), int(p_dim), int(k), float(top_frac),
                   float(small_rel), float(tail_frac))
    _check(lib().spec_descriptors(_stream(), _dev(w), _dt(w), batch, r, w.stride(0), ctypes.byref(p),
                                  _dev(out), _dev(ws), ws.numel()))
    if not to_host:
        return out
    return out.cpu().numpy().view(DESC_DTYPE).reshape(batch)


def descriptors_static(w, *, n_samples: int, p_dim: int, k: int = 1, mode: int = MODE_EIG,
                       sigma2: float = 1.0, sigma2_mode: int = SIGMA2_GIVEN, top_frac: float = 0.2,
                       small_rel: float = 1e-2, tail_frac: float = 0.7, out=None, to_host: bool = True):
    """descriptors() without a workspace: the library's own per-GPU table is used
    (spec_descriptors_static; r <= 32768; overlapping calls on one GPU race)."""
    torch = _torch()
    if w.dim() == 1:
        w = w.unsqueeze(0)
    batch, r = w.shape
    if out is None:
        out = torch.empty((batch, DESC_DTYPE.itemsize), dtype=torch.uint8, device=w.device)
    p = DescParams(mode, sigma2_mode, float(sigma2), int(n_samples), int(p_dim), int(k), float(top_frac),
                   float(small_rel), float(tail_frac))
    _check(lib().spec_descriptors_static(_stream(), _dev(w), _dt(w), batch, r, w.stride(0), ctypes.byref(p),
                                         _dev(out)))
    if not to_host:
        return out
    return out.cpu().numpy().view(DESC_DTYPE).reshape(batch)


def desc_smooth(rec, *, streams: int, W: int, alpha: float, out=None, to_host: bool = True):
    """Exponential smoothing along W of the descriptor records rec (a device uint8
    buffer of streams * W records, as descriptors(..., to_host=False) returns).
    Returns a numpy structured array [streams, W] of DESC_DTYPE (or the device
    buffer if to_host is False)."""
    torch = _torch()
    if out is None:
        out = torch.empty((streams * W, DESC_DTYPE.itemsize), dtype=torch.uint8, device=rec.device)
    _check(lib().spec_desc_smooth(_stream(), _dev(rec), streams, W, float(alpha), _dev(out)))
    if not to_host:
        return out
    return out.cpu().numpy().view(DESC_DTYPE).reshape(streams, W)


def spectrum_robust(w, *, n_samples: int, p_dim: int, sigma2: float = 1.0, sigma2_mode: int = SIGMA2_GIVEN,
                    winsor_frac: float = 0.05, mad_k: float = 3.0, bins: int = 16, out=None,
                    to_host: bool = True):
    """Median, winsorised sigma^2, MAD and MAD outlier count, log-eigenvalue mean
    and spread, and the KL form of the MP deviation of each row of w [batch, r]
    (sorted descending).  Returns a numpy structured array of ROBUST_DTYPE (or
    the device buffer if to_host is False)."""
    torch = _torch()
    if w.dim() == 1:
        w = w.unsqueeze(0)
    batch, r = w.shape
    if out is None:
        out = torch.empty((batch, ROBUST_DTYPE.itemsize), dtype=torch.uint8, device=w.device)
    p = RobustParams(int(sigma2_mode), int(bins), float(sigma2), int(n_samples), int(p_dim), float(winsor_frac),
                     float(mad_k))
    _check(lib().spec_spectrum_robust(_stream(), _dev(w), _dt(w), batch, r, w.stride(0), ctypes.byref(p),
                                      _dev(out)))
    if not to_host:
        return out
    return out.cpu().numpy().view(ROBUST_DTYPE).reshape(batch)


def eigvalsh_topk(A, Omega, q: int = 2, w=None, ws=None):
    """The 32 Ritz values (descending) of the symmetric A [n, n] (lower triangle
    read, A kept) on the range of A Omega after q subspace iterations; Omega is
    the caller's random test matrix [n, 32] (float32, contiguous)."""
    torch = _torch()
    n = A.shape[0]
    if A.stride(1) != 1 or not Omega.is_contiguous() or tuple(Omega.shape) != (n, 32):
        raise SpecError(-1, "A must be row-major and Omega a contiguous [n, 32] tensor")
    if w is None:
        w = torch.empty((32,), dtype=torch.float32, device=A.device)
    if ws is None:
        ws = torch.empty((eigvalsh_large_workspace(n, torch.float32),), dtype=torch.uint8, device=A.device)
    _check(lib().spec_eigvalsh_topk(_stream(), _dev(A), _dt(A), n, A.stride(0), _dev(Omega), int(q), _dev(w),
                                    _dev(ws), ws.numel()))
    return w


def eigvecs_topk(A, Omega, q: int = 2, w=None, P=None, ws=None, info=None):
    """Ritz values (descending, [32]) and Ritz vectors P [n, 32] (column i for
    value i, orthonormal columns, arbitrary signs) of the same projection as
    eigvalsh_topk; the columns with a value above the MP edge span the signal
    subspace.  ``info`` (int32 [1] device tensor, optional) receives 0
    (converged), 1 (non-finite input) or 2 (sweep limit reached)."""
    torch = _torch()
    n = A.shape[0]
    if A.stride(1) != 1 or not Omega.is_contiguous() or tuple(Omega.shape) != (n, 32):
        raise SpecError(-1, "A must be row-major and Omega a contiguous [n, 32] tensor")
    if w is None:
        w = torch.empty((32,), dtype=torch.float32, device=A.device)
    if P is None:
        P = torch.empty((n, 32), dtype=torch.float32, device=A.device)
    if P.dim() != 2 or P.shape[0] != n or P.shape[1] < 32 or P.stride(1) != 1 or P.dtype != torch.float32:
        raise SpecError(-1, "P must be a row-major float32 [n, >= 32] tensor")
    if ws is None:
        ws = torch.empty((eigvalsh_large_workspace(n, torch.float32),), dtype=torch.uint8, device=A.device)
    _check(lib().spec_eigvecs_topk(_stream(), _dev(A), _dt(A), n, A.stride(0), _dev(Omega), int(q), _dev(w),
                                   _dev(P), P.stride(0), _dev(ws), ws.numel(), _dev(info) if info is not None else None))
    return w, P


def project_weight_workspace(d: int) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().spec_project_weight_workspace(d, ctypes.byref(b)))
    return b.value


def project_weight(W, P, k=None, Wp=None, X=None, want_factor: bool = True, ws=None):
    """W' = P^T W P ([k, k]) and, if want_factor, X = W P ([d, k]) for a square
    weight W [d, d] (bf16 or float32, row-major) and the basis P [d, >= k]
    (float32, row-major; the first k columns are used)."""
    torch = _torch()
    d = W.shape[0]
    if W.dim() != 2 or W.shape[1] != d or W.stride(1) != 1:
        raise SpecError(-1, "W must be a row-major square tensor")
    if P.dim() != 2 or P.shape[0] != d or P.stride(1) != 1 or P.dtype != torch.float32:
        raise SpecError(-1, "P must be a row-major float32 [d, k] tensor")
    k = P.shape[1] if k is None else int(k)
    if k > P.shape[1]:
        raise SpecError(-1, "k exceeds the columns of P")
    if Wp is None:
        Wp = torch.empty((k, k), dtype=torch.float32, device=W.device)
    if want_factor and X is None:
        X = torch.empty((d, k), dtype=torch.float32, device=W.device)
    if not want_factor:
        X = None
    if ws is None:
        ws = torch.empty((project_weight_workspace(d),), dtype=torch.uint8, device=W.device)
    _check(lib().spec_project_weight(_stream(), _dev(W), _dt(W), d, W.stride(0), _dev(P), P.stride(0), k, _dev(Wp),
                                     Wp.stride(0), None if X is None else _dev(X), 0 if X is None else X.stride(0),
                                     _dev(ws), ws.numel()))
    return Wp, X


def tail_pair_screen(U, V, *, i0: int | None = None, t: int | None = None, head_dim: int = 128,
                     eps: float = 0.015, absdot=None, keep=None, count=None):
    """S3 swap-candidate screen: |u_i^T v_j| for the tail columns [i0, i0 + t) of
    U and V (singular vectors as columns; default tail: i >= 0.9 N), and the
    same-head pairs below eps.  Returns (absdot [t, t] f64, keep [t, t] uint8,
    count [1] int64), device tensors."""
    import math
    torch = _torch()
    N = U.shape[1]
    if i0 is None:
        i0 = int(math.ceil(0.9 * N))
    if t is None:
        t = N - i0
    if U.dtype != V.dtype or U.stride(1) != 1 or V.stride(1) != 1 or U.shape[0] != V.shape[0]:
        raise SpecError(-1, "U and V must be row-major with the same dtype and row count")
    dev = U.device
    if absdot is None:
        absdot = torch.empty((t, t), dtype=torch.float64, device=dev)
    if keep is None:
        keep = torch.empty((t, t), dtype=torch.uint8, device=dev)
    if count is None:
        count = torch.empty((1,), dtype=torch.int64, device=dev)
    _check(lib().spec_tail_pair_screen(_stream(), _dev(U), _dev(V), _dt(U), U.shape[0], U.stride(0), V.stride(0),
                                       int(i0), int(t), int(head_dim), float(eps), _dev(absdot), absdot.stride(0),
                                       _dev(keep), keep.stride(0), _dev(count)))
    return absdot, keep, count


def eigvalsh_batched_band_desc(band, n: int, scale: float, *, n_samples: int, p_dim: int, k: int = 1,
                               stride: int = 1, mode: int = MODE_EIG, sigma2: float = 1.0,
                               sigma2_mode: int = SIGMA2_GIVEN, top_frac: float = 0.2, small_rel: float = 1e-2,
                               tail_frac: float = 0.7, w=None, keep_w: bool = True, info=None, out=None, ws=None,
                               to_host: bool = True):
    """Window spectra and their descriptors in one pass (spec_eigvalsh_batched_desc)
    from the band [S, T, n] of gram_window.  Returns (w or None, info, records)."""
    torch = _torch()
    S, T, N = band.shape
    if N != n or not band.is_contiguous():
        raise SpecError(-1, "band must be a contiguous [streams, T, n] tensor")
    batch = S * ((T - n) // stride + 1)
    src = BatchSrc(SRC_BAND, _dev(band), 0, 0, S, T, stride, float(scale))
    dev = band.device
    if w is None and keep_w:
        w = torch.empty((batch, n), dtype=torch.float32, device=dev)
    if info is None:
        info = torch.empty((batch,), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((batch, DESC_DTYPE.itemsize), dtype=torch.uint8, device=dev)
    if ws is None:
        ws = torch.empty((descriptors_workspace(n),), dtype=torch.uint8, device=dev)
    p = DescParams(mode, sigma2_mode, float(sigma2), int(n_samples), int(p_dim), int(k), float(top_frac),
                   float(small_rel), float(tail_frac))
    _check(lib().spec_eigvalsh_batched_desc(_stream(), ctypes.byref(src), batch, n,
                                            _dev(w) if w is not None else None, _dev(info), ctypes.byref(p),
                                            _dev(out), _dev(ws), ws.numel()))
    rec = out.cpu().numpy().view(DESC_DTYPE).reshape(batch) if to_host else out
    return w, info, rec


def eigvalsh_batched_dense_desc(A, *, n_samples: int, p_dim: int, k: int = 1, w=None, info=None, out=None,
                                ws=None, **kw):
    """Dense batch [batch, n, n] (lower read): spectra and descriptors in one pass."""
    torch = _torch()
    if A.dim() == 2:
        A = A.unsqueeze(0)
    batch, n, _ = A.shape
    src = BatchSrc(SRC_DENSE, _dev(A), A.stride(1), A.stride(0), 0, 0, 1, 1.0)
    dev = A.device
    if w is None:
        w = torch.empty((batch, n), dtype=torch.float32, device=dev)
    if info is None:
        info = torch.empty((batch,), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((batch, DESC_DTYPE.itemsize), dtype=torch.uint8, device=dev)
    if ws is None:
        ws = torch.empty((descriptors_workspace(n),), dtype=torch.uint8, device=dev)
    p = DescParams(kw.get("mode", MODE_EIG), kw.get("sigma2_mode", SIGMA2_GIVEN), float(kw.get("sigma2", 1.0)),
                   int(n_samples), int(p_dim), int(k), float(kw.get("top_frac", 0.2)),
                   float(kw.get("small_rel", 1e-2)), float(kw.get("tail_frac", 0.7)))
    _check(lib().spec_eigvalsh_batched_desc(_stream(), ctypes.byref(src), batch, n, _dev(w), _dev(info),
                                            ctypes.byref(p), _dev(out), _dev(ws), ws.numel()))
    return w, info, out.cpu().numpy().view(DESC_DTYPE).reshape(batch)
