"""Seeded synthetic inputs for the spectral hot path.

This module is the only code the tests of the GPU path, the fp64 oracle's
stored expected values and the benchmark share.  It draws random matrices with
the shapes and value distributions of the workloads the pages describe and
holds none of the method's arithmetic (no covariance, no eigen-solve, no
descriptor); the library itself never imports it.

Workloads (all seeded from ``numpy.random.SeedSequence(0).spawn(5)[i]`` with
PCG64, in a fixed draw order):

* ``tiny``       X f32 [64, 32]: N(0,1) plus two planted rank-1 spikes
                 (theta = 4, 8) along orthonormalised random directions.
                 Spiked covariance model, "Random matrix theory spectral
                 methods" page, section 2.2.
* ``eigentrack`` H bf16 [streams, T, d]: per-stream decode-step activations
                 h_t = z_t + sqrt(a_s) B_s g_t with a rank-8 orthonormal basis
                 B_s and strength a_s ~ U(0, 3); the EigenTrack sliding window,
                 same page, section 3.1.
* ``swiftsvd``   32 chunks X bf16 [2048, 4096] of Student-t(4) entries, 16
                 outlier channels scaled by 20 (shared by all chunks); the
                 incremental covariance of the Swift-SVD page, sections 2 and 7.
* ``ffn``        X bf16 [65536, 14336]: N(0,1) plus a rank-64 additive spike
                 with theta log-uniform in [0.5, 50] (FFN width 14336 from the
                 S3 page, section 5.1); generated bit-identically on any host.
* ``s3``         32 layers W f32 [4096, 4096] = U diag(sigma) V^T with Haar
                 U, V and sigma_i = (2i-1)^(-a), a = 3 / log10(2d-1), so that
                 sigma_1 = 1, sigma_d = 1e-3 (S3 page, section 2).

bf16 values are produced once on the host by round-to-nearest-even from f32 and
handed to both sides as raw uint16 bit patterns.
"""
from __future__ import annotations

import hashlib
import math

import numpy as np

CONFIG_INDEX = {"tiny": 0, "eigentrack": 1, "swiftsvd": 2, "ffn": 3, "s3": 4}

# Full-size shapes of the five workloads.
FULL = {
    "tiny": dict(n=64, d=32, thetas=(4.0, 8.0)),
    "eigentrack": dict(streams=256, T=512, d=4096, N=30, rank=8, amax=3.0),
    "swiftsvd": dict(chunks=32, n=2048, d=4096, outliers=16, scale=20.0, nu=4.0),
    "ffn": dict(n=65536, d=14336, rank=64, theta_lo=0.5, theta_hi=50.0),
    "s3": dict(layers=32, d=4096, sigma_min=1e-3),
}


def rng_for(config: str, sub: int = 0) -> np.random.Generator:
    """Generator for one workload; ``sub`` separates independent draws."""
    ss = np.random.SeedSequence(0).spawn(5)[CONFIG_INDEX[config]]
    if sub:
        ss = ss.spawn(sub + 1)[sub]
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round f32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to f32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def orthonormal(rng: np.random.Generator, d: int, k: int) -> np.ndarray:
    """d x k matrix with orthonormal columns (QR of a Gaussian, signs fixed)."""
    g = rng.standard_normal((d, k))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))


def orthonormal_exact(rng: np.random.Generator, d: int, k: int) -> np.ndarray:
    """d x k orthonormal columns by twice-applied modified Gram-Schmidt on a
    Gaussian, every inner product an exactly rounded sum (math.fsum), so the
    result has the same bits on any host (BLAS and LAPACK round differently on
    different CPUs)."""
    g = rng.standard_normal((d, k))
    q = np.empty((d, k))
    for j in range(k):
        v = g[:, j].copy()
        for _ in range(2):
            for i in range(j):
                v = v - math.fsum(v * q[:, i]) * q[:, i]
        q[:, j] = v / math.sqrt(math.fsum(v * v))
    return q


def haar_orthogonal(rng: np.random.Generator, d: int) -> np.ndarray:
    """Haar-distributed d x d orthogonal matrix: QR of N(0,1) with the signs of
    diag(R) folded into Q (Mezzadri, Notices AMS 54, 2007)."""
    return orthonormal(rng, d, d)


def tiny(n: int = 64, d: int = 32, thetas=(4.0, 8.0)) -> np.ndarray:
    """X = Z + sum_k sqrt(theta_k) s_k u_k^T, f32 [n, d]."""
    rng = rng_for("tiny")
    z = rng.standard_normal((n, d))
    u = orthonormal(rng, d, len(thetas))
    s = rng.standard_normal((n, len(thetas)))
    x = z + (s * np.sqrt(np.asarray(thetas))) @ u.T
    return x.astype(np.float32)


def eigentrack(streams: int = 256, T: int = 512, d: int = 4096, rank: int = 8,
               amax: float = 3.0, seed_sub: int = 0) -> np.ndarray:
    """bf16 bits [streams, T, d]: h_t = z_t + sqrt(a_s) B_s g_t per stream."""
    rng = rng_for("eigentrack", seed_sub)
    a = rng.uniform(0.0, amax, size=streams)
    out = np.empty((streams, T, d), dtype=np.uint16)
    for s in range(streams):
        b = orthonormal(rng, d, rank)
        g = rng.standard_normal((T, rank))
        z = rng.standard_normal((T, d), dtype=np.float32)
        h = z + ((math.sqrt(a[s]) * g) @ b.T).astype(np.float32)
        out[s] = f32_to_bf16_bits(h)
    return out


def eigentrack_strengths(streams: int = 256, amax: float = 3.0, seed_sub: int = 0) -> np.ndarray:
    """The per-stream signal strengths a_s drawn first by :func:`eigentrack`."""
    return rng_for("eigentrack", seed_sub).uniform(0.0, amax, size=streams)


def swiftsvd_outlier_channels(d: int = 4096, outliers: int = 16) -> np.ndarray:
    rng = rng_for("swiftsvd")
    return np.sort(rng.choice(d, size=outliers, replace=False))


def swiftsvd_chunk(k: int, n: int = 2048, d: int = 4096, outliers: int = 16,
                   scale: float = 20.0, nu: float = 4.0) -> np.ndarray:
    """bf16 bits [n, d] of chunk k: Student-t(nu) entries, outlier columns x scale."""
    cols = swiftsvd_outlier_channels(d, outliers)
    rng = rng_for("swiftsvd", 1 + k)
    x = rng.standard_t(nu, size=(n, d)).astype(np.float32)
    x[:, cols] *= np.float32(scale)
    return f32_to_bf16_bits(x)


def swiftsvd(chunks: int = 32, n: int = 2048, d: int = 4096, outliers: int = 16,
             scale: float = 20.0, nu: float = 4.0) -> np.ndarray:
    """bf16 bits [chunks, n, d]."""
    out = np.empty((chunks, n, d), dtype=np.uint16)
    for k in range(chunks):
        out[k] = swiftsvd_chunk(k, n, d, outliers, scale, nu)
    return out


def ffn_spikes(d: int = 14336, rank: int = 64, theta_lo: float = 0.5, theta_hi: float = 50.0):
    """(theta [rank], U [d, rank]) of the FFN-width spiked covariance, and the
    spike loadings L = sqrt(theta_k) u_k rounded to the grid 2^-20 ([rank, d])."""
    rng = rng_for("ffn")
    u01 = rng.uniform(0.0, 1.0, size=rank)
    theta = theta_lo * (theta_hi / theta_lo) ** u01
    U = orthonormal_exact(rng, d, rank)
    L = np.round(np.sqrt(theta)[:, None] * U.T * 2.0 ** 20) / 2.0 ** 20
    return theta, U, L


def ffn(n: int = 65536, d: int = 14336, rank: int = 64, theta_lo: float = 0.5,
        theta_hi: float = 50.0, row_block: int = 4096) -> np.ndarray:
    """bf16 bits [n, d]: X = Z + S L with Z ~ N(0, 1), S ~ +-1 (Rademacher; mean 0,
    variance 1, so E[x x^T] = I + sum_k theta_k u_k u_k^T).  L sits on the grid
    2^-20 and S is +-1, so every entry of S L is an integer multiple of 2^-20 below
    2^26 ulps and the fp64 product is exact in any summation order: the same bits
    on every host."""
    _, _, L = ffn_spikes(d, rank, theta_lo, theta_hi)
    out = np.empty((n, d), dtype=np.uint16)
    for i, r0 in enumerate(range(0, n, row_block)):
        r1 = min(n, r0 + row_block)
        rng = rng_for("ffn", 1 + i)
        z = rng.standard_normal((r1 - r0, d), dtype=np.float32)
        s = rng.integers(0, 2, size=(r1 - r0, rank)).astype(np.float64) * 2.0 - 1.0
        x = z.astype(np.float64) + s @ L
        out[r0:r1] = f32_to_bf16_bits(x.astype(np.float32))
    return out


def s3_sigma(d: int = 4096, sigma_min: float = 1e-3) -> np.ndarray:
    """Planted singular values sigma_i = (2i-1)^(-a), sigma_1 = 1, sigma_d = sigma_min."""
    a = -math.log10(sigma_min) / math.log10(2 * d - 1)
    i = np.arange(1, d + 1, dtype=np.float64)
    return (2.0 * i - 1.0) ** (-a)


def s3_layer_f64(layer: int, d: int = 4096, sigma_min: float = 1e-3) -> np.ndarray:
    """W = U diag(sigma) V^T in fp64 for one layer (before rounding to f32)."""
    rng = rng_for("s3", 1 + layer)
    U = haar_orthogonal(rng, d)
    V = haar_orthogonal(rng, d)
    return (U * s3_sigma(d, sigma_min)) @ V.T


def s3_factors(layer: int, d: int = 4096, sigma_min: float = 1e-3):
    """(U, sigma, V) of one layer, fp64: W = U diag(sigma) V^T (the singular
    vectors the S3 tail-pair screen takes)."""
    rng = rng_for("s3", 1 + layer)
    U = haar_orthogonal(rng, d)
    V = haar_orthogonal(rng, d)
    return U, s3_sigma(d, sigma_min), V


def s3_layer(layer: int, d: int = 4096, sigma_min: float = 1e-3) -> np.ndarray:
    """f32 [d, d] weight of one layer (fp64 product rounded to nearest f32)."""
    return s3_layer_f64(layer, d, sigma_min).astype(np.float32)


def s3(layers: int = 32, d: int = 4096, sigma_min: float = 1e-3) -> np.ndarray:
    out = np.empty((layers, d, d), dtype=np.float32)
    for l in range(layers):
        out[l] = s3_layer(l, d, sigma_min)
    return out


def s3_layers_device(layers: int = 32, d: int = 4096, sigma_min: float = 1e-3, device="cuda", seed: int = 0):
    """The S3 weight workload drawn on the GPU with torch (for timing runs, where
    64 host QRs of d x d would take minutes): the same recipe as s3_layer --
    Haar U, V from QR of N(0,1) fp64 matrices with the signs of diag(R) folded
    in, W = U diag(sigma) V^T in fp64, rounded to f32 -- from torch's seeded
    device generator, so the values differ from s3_layer's while the planted
    spectrum is the same.  Returns a [layers, d, d] float32 device tensor."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    sig = torch.from_numpy(s3_sigma(d, sigma_min)).to(device)
    out = torch.empty((layers, d, d), dtype=torch.float32, device=device)
    for l in range(layers):
        hs = []
        for _ in range(2):
            q, r = torch.linalg.qr(torch.randn((d, d), dtype=torch.float64, device=device, generator=g))
            hs.append(q * torch.sign(torch.diagonal(r)))
        out[l] = ((hs[0] * sig) @ hs[1].T).to(torch.float32)
        del hs, q, r
    return out


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
