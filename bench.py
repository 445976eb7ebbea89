"""Benchmark of the spectral hot path on one MI355X.

One step is one pass of the whole path over the FFN-width covariance workload
(65536 tokens x 14336 features, bf16, N(0,1) plus a rank-64 spike):
  SYRK aggregation C = X^T X / 65536 (one call, lower triangle, fp32)
  -> all 14336 eigenvalues of C (reduction to band, bulge chasing, multisection)
  -> descriptors of the spectrum (entropy, leading mass, eigengap, MP edge and
     outlier count, W1 to MP, energy shares).
value = covariance eigensolves per second of that whole step (one per step).

The other workloads are timed after the steps as phase rows (not part of
value): the 64 x 32 tiny case, the EigenTrack sliding windows (256 streams x
512 steps x 4096, N = 30), the Swift-SVD covariance (32 chunks of 2048 x 4096
bf16 -> eigvalsh 4096 f32) and the S3 weight spectra (32 layers of 4096^2 f32,
fp64 Gram and fp64 eigvalsh).  Inputs are resident in HBM before any timing.

The roofline row is the kernel with the most device time per step, timed live
with HIP events that the library records around each of its launches on the
stream it launches on (spec.timing_enable).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-phases] [--no-postproc]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # B/s
PEAK_BF16_MFMA = 2.5e15    # dense flop/s
PEAK_F32_MFMA = 157.3e12   # dense fp32 matrix-core flop/s
PEAK_F64_MFMA = 78.6e12    # dense fp64 matrix-core flop/s
PEAK_F32_VALU = 78.6e12    # non-packed fp32 FMA: 256 CU x 64 lanes x 2 flop x 2.4 GHz

FFN = dict(n=65536, d=14336)
NB = 32  # bandwidth of the reduction to band (the library's stage-1 block)

METRIC = "covariance SYRK TFLOP/s + eigensolves/sec; % of MFMA/HBM roofline, 1 GPU"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- algorithmic work

def panel_sizes(n):
    """Trailing sizes m of the reduction's panels (one SYMM and one SYR2K each)."""
    out, c0 = [], 0
    while n - (c0 + NB) >= 2:
        out.append(n - (c0 + NB))
        c0 += NB
    return out


def bulge_flops(n, b=NB):
    """Bulge chasing: sweep s (0 <= s < n - 2) runs (n - 2 - s) // b + 1 tasks;
    the first applies a length-b reflector two-sided to a b x b diagonal block
    (D v and the rank-2 update, 4 b^2 flops), every later one also applies the
    previous reflector from the right and the new one from the left to the
    b x b off-diagonal block (8 b^2 more): 12 b^2."""
    tot = 0
    for s in range(n - 2):
        t = (n - 2 - s) // b + 1
        tot += 4 * b * b + 12 * b * b * (t - 1)
    return float(tot)


def kernel_work(kernel, n, n_rows=None):
    """(algorithmic flops, algorithmic HBM bytes) summed over the launches one
    eigensolve (or one SYRK call) makes, per the design notes."""
    if kernel == "syrk":
        return float(n_rows) * n * (n + 1), 2.0 * n_rows * n + 4.0 * n * (n + 1) / 2
    if kernel == "symm":
        ms = np.array(panel_sizes(n), dtype=np.float64)
        return float(np.sum(2.0 * ms * ms * NB)), float(np.sum(4.0 * ms * (ms + 1) / 2 + 2 * 4.0 * ms * NB))
    if kernel == "syr2k":
        ms = np.array(panel_sizes(n), dtype=np.float64)
        return float(np.sum(2.0 * NB * ms * (ms + 1))), float(np.sum(2 * 4.0 * ms * (ms + 1) / 2))
    if kernel == "bulge":
        return bulge_flops(n), 2 * 4.0 * n * 2 * NB
    raise KeyError(kernel)


def roofline_row(kernel, total_ms, launches, n, n_rows=None, traffic=None):
    flops, bytes_ = kernel_work(kernel, n, n_rows)
    t = total_ms / 1e3
    if kernel == "syrk":
        bound, peak, ach, unit = "mfma", PEAK_BF16_MFMA, flops / t, "TFLOP/s"
    elif kernel in ("symm", "syr2k"):
        bound, peak, ach, unit = "mfma", PEAK_F32_MFMA, flops / t, "TFLOP/s"
    else:  # bulge chasing: scalar fp32 arithmetic in registers
        bound, peak, ach, unit = "alu", PEAK_F32_VALU, flops / t, "TFLOP/s"
    return {"kernel": kernel, "bound": bound, "achieved": ach / 1e12, "peak": peak / 1e12, "unit": unit,
            "frac": ach / peak, "traffic": traffic, "launches": launches, "avg_launch_ms": total_ms / max(1, launches),
            "algorithmic_flops": flops, "algorithmic_bytes": bytes_,
            "achieved_GBs": bytes_ / t / 1e9}


def counter_traffic(kernel):
    """HBM bytes per launch of one kernel at the headline workload from the
    committed counter summary, or None when its source changed since."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"{kernel}_ffn_14336_hbm_traffic.md")
    try:
        rec = json.loads(re.search(r"```json\n(.*?)\n```", open(path).read(), re.S).group(1))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, AttributeError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    return float(rec["hbm_bytes_per_launch"])


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(X):
    """The oracle as it stands on a bounded sample of the headline step, scaled
    to eigensolves/s of the whole step: the fp64 covariance of 2048 of the 65536
    rows (x 32), the fp64 Householder + bisection eigensolve of the leading 4096 x
    4096 block of that covariance (x (14336/4096)^3, the cubic cost), and the
    descriptors of a 14336-value spectrum."""
    import oracle
    n, d = FFN["n"], FFN["d"]
    rows = 2048
    t0 = time.perf_counter()
    C = oracle.covariance(X[:rows], "bf16", 1.0 / rows)
    t_cov = (time.perf_counter() - t0) * (n / rows)
    t0 = time.perf_counter()
    w = oracle.eigvalsh_large(C[:4096, :4096])
    t_eig = (time.perf_counter() - t0) * (d / 4096) ** 3
    wd = np.concatenate([w, np.linspace(0.0, float(w[-1]), d - 4096)])
    t0 = time.perf_counter()
    oracle.descriptors(wd, n_samples=n, p_dim=d, k=1)
    t_desc = time.perf_counter() - t0
    total = t_cov + t_eig + t_desc
    return {"value": 1.0 / total, "unit": "eigensolves/s", "cores": os.cpu_count(), "kind": "oracle",
            "sample": ("fp64 covariance of 2048 of 65536 rows x 32; fp64 eigensolve of the leading 4096 x 4096 "
                       "block x (14336/4096)^3; descriptors of one 14336-value spectrum"),
            "seconds_per_step_est": total, "phases_s": {"covariance": t_cov, "eig14336": t_eig, "desc": t_desc}}


# ----------------------------------------------------------------------------- phase rows

def ev_pair(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def timed(torch, fn, reps):
    fn()
    torch.cuda.synchronize()
    a, b = ev_pair(torch)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def phase_rows(torch, spec, synth, dev, with_cpu, which=("tiny", "eigentrack", "swiftsvd", "s3")):
    rows = {}
    if "tiny" in which:
        # ---- tiny: 64 x 32 f32 -> C (alpha = 1/64) -> 32 eigenvalues -> descriptors
        X1 = torch.from_numpy(synth.tiny()).to(dev)
        C1 = torch.empty((32, 32), dtype=torch.float32, device=dev)
        w1 = torch.empty((1, 32), dtype=torch.float32, device=dev)
        i1 = torch.empty((1,), dtype=torch.int32, device=dev)
        d1 = torch.empty((1, spec.DESC_DTYPE.itemsize), dtype=torch.uint8, device=dev)
        ws1 = torch.empty((spec.descriptors_workspace(32),), dtype=torch.uint8, device=dev)

        def tiny():
            spec.cov_accumulate(X1, C1, alpha=1.0 / 64, beta=0.0)
            spec.eigvalsh_batched_dense(C1, w=w1, info=i1)
            spec.descriptors(w1, n_samples=64, p_dim=32, k=1, out=d1, ws=ws1, to_host=False)
        ms = timed(torch, tiny, 200)
        rows["tiny_64x32"] = {"ms": ms, "eigensolves_per_s": 1e3 / ms, "bound": "launch latency (4 kernels)"}
        log(f"tiny: {ms * 1e3:.1f} us per pass")
    if "eigentrack" in which:
        # ---- EigenTrack windows: band Gram -> 123,648 window spectra -> descriptors
        S, T, d, N = 256, 512, 4096, 30
        W = T - N + 1
        H = synth.eigentrack(streams=S, T=T, d=d)
        Hd = torch.from_numpy(H.view(np.int16)).to(dev).view(torch.bfloat16)
        band = torch.empty((S, T, N), dtype=torch.float32, device=dev)
        ww = torch.empty((S * W, N), dtype=torch.float32, device=dev)
        iw = torch.empty((S * W,), dtype=torch.int32, device=dev)
        dw = torch.empty((S * W, spec.DESC_DTYPE.itemsize), dtype=torch.uint8, device=dev)
        wsw = torch.empty((spec.descriptors_workspace(N),), dtype=torch.uint8, device=dev)
        part = {}
        for name, fn in [("gram_band", lambda: spec.gram_window(Hd, N=N, out=band)),
                         ("eig_windows", lambda: spec.eigvalsh_batched_band(band, n=N, scale=1.0 / N, w=ww, info=iw)),
                         ("desc_windows", lambda: spec.descriptors(ww, n_samples=N, p_dim=d, k=8, out=dw, ws=wsw,
                                                                    to_host=False))]:
            part[name] = timed(torch, fn, 10)
        # the same spectra and records from the fused entry point (one kernel after the band)
        fused = timed(torch, lambda: spec.eigvalsh_batched_band_desc(band, n=N, scale=1.0 / N, n_samples=N, p_dim=d,
                                                                    k=8, w=ww, info=iw, out=dw, ws=wsw,
                                                                    to_host=False), 10)
        tot = sum(part.values())
        rounds = float(iw.float().mean())
        rows["eigentrack_256x512x4096_N30"] = {
            "ms": tot, "phases_ms": part, "windows": S * W, "window_spectra_per_s": S * W / (tot / 1e3),
            "eig_desc_fused_ms": fused, "ms_fused_path": part["gram_band"] + fused,
            "gram_band": {"bound": "hbm", "achieved_GBs": (H.nbytes + S * T * N * 4) / (part["gram_band"] / 1e3) / 1e9,
                          "frac": (H.nbytes + S * T * N * 4) / (part["gram_band"] / 1e3) / PEAK_HBM},
            # per window: Householder (4/3) N^3, then Sturm counts of 4 flop per step
            # of N: 64 multisection points and N bisections of `rounds` counts each
            "eig_windows": {"bound": "alu",
                            "achieved_TFLOPs": S * W * (4.0 / 3.0 * N ** 3 + 4.0 * N * (64 + rounds * N)) / (part["eig_windows"] / 1e3) / 1e12,
                            "mean_bisection_rounds": rounds},
            "desc_windows": {"bound": "hbm", "achieved_GBs": S * W * (N * 4 + 144) / (part["desc_windows"] / 1e3) / 1e9}}
        rows["eigentrack_256x512x4096_N30"]["eig_windows"]["frac"] = \
            rows["eigentrack_256x512x4096_N30"]["eig_windows"]["achieved_TFLOPs"] * 1e12 / PEAK_F32_VALU
        log(f"eigentrack: {tot:.3f} ms ({part}); fused eig+desc {fused:.3f} ms")
        if with_cpu:
            import oracle
            t0 = time.perf_counter()
            for s in range(2):
                G = oracle.window_gram(H[s], "bf16", N)
                w, _ = oracle.eigvalsh_small(G)
                for b in range(w.shape[0]):
                    oracle.descriptors(w[b], n_samples=N, p_dim=d, k=8)
            t = (time.perf_counter() - t0) * S / 2
            rows["eigentrack_256x512x4096_N30"]["cpu_baseline"] = {
                "value": S * W / t, "unit": "window spectra/s", "cores": os.cpu_count(), "kind": "oracle",
                "sample": "2 of 256 streams (966 windows: fp64 Gram, Jacobi, descriptors) x 128"}
        del Hd, band, ww, iw, dw, H
    if "swiftsvd" in which:
        # ---- Swift-SVD: 32 chunks -> C 4096^2 -> eigvalsh 4096 f32 -> descriptors
        Xs = synth.swiftsvd(chunks=32, n=2048, d=4096)
        Xsd = torch.from_numpy(Xs.view(np.int16)).to(dev).view(torch.bfloat16)
        Cs = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
        wsb = torch.empty((4096,), dtype=torch.float32, device=dev)
        wss = torch.empty((spec.eigvalsh_large_workspace(4096, torch.float32),), dtype=torch.uint8, device=dev)
        infos = torch.zeros((1,), dtype=torch.int32, device=dev)
        ds = torch.empty((1, spec.DESC_DTYPE.itemsize), dtype=torch.uint8, device=dev)
        dss = torch.empty((spec.descriptors_workspace(4096),), dtype=torch.uint8, device=dev)

        def sw_syrk():
            for k in range(32):
                spec.cov_accumulate(Xsd[k], Cs, alpha=1.0, beta=0.0 if k == 0 else 1.0)
        part = {"syrk": timed(torch, sw_syrk, 5)}
        # the same C in one call: the 32 chunks are contiguous, so sum_k X_k^T X_k
        # is one SYRK over the stacked 65536 rows (C written once, not 32 times)
        Xstack = Xsd.reshape(32 * 2048, 4096)
        syrk_stacked = timed(torch, lambda: spec.cov_accumulate(Xstack, Cs, alpha=1.0, beta=0.0), 5)
        part["eig_large"] = timed(torch, lambda: (sw_syrk(), spec.eigvalsh_large(Cs, w=wsb, ws=wss, info=infos)), 3) \
            - part["syrk"]
        part["desc"] = timed(torch, lambda: spec.descriptors(wsb, n_samples=65536, p_dim=4096, k=1,
                                                             sigma2_mode=spec.SIGMA2_MEAN, out=ds, ws=dss,
                                                             to_host=False), 10)
        tot = sum(part.values())
        f = 65536.0 * 4096 * 4097
        rows["swiftsvd_32x2048x4096"] = {
            "ms": tot, "phases_ms": part, "eigensolves_per_s": 1e3 / tot,
            "syrk": {"bound": "mfma", "achieved_TFLOPs": f / (part["syrk"] / 1e3) / 1e12,
                     "frac": f / (part["syrk"] / 1e3) / PEAK_BF16_MFMA},
            "syrk_one_call": {"ms": syrk_stacked, "achieved_TFLOPs": f / (syrk_stacked / 1e3) / 1e12,
                              "frac": f / (syrk_stacked / 1e3) / PEAK_BF16_MFMA},
            "eig_4096_f32_per_s": 1e3 / part["eig_large"]}
        assert int(infos.cpu()[0]) == 0
        log(f"swiftsvd: {tot:.3f} ms ({part})")
        del Xsd, Xs, Cs, wss
    if "s3" in which:
        # ---- S3: 32 layers W (4096^2 f32) -> fp64 Gram -> fp64 eigvalsh -> singular descriptors
        t0 = time.time()
        Wl = synth.s3_layers_device(32, 4096, device=dev)
        torch.cuda.synchronize()
        log(f"s3 layers generated on the GPU in {time.time() - t0:.1f} s")
        C5 = torch.empty((4096, 4096), dtype=torch.float64, device=dev)
        w5 = torch.empty((32, 4096), dtype=torch.float64, device=dev)
        ws5 = torch.empty((spec.eigvalsh_large_workspace(4096, torch.float64),), dtype=torch.uint8, device=dev)
        i5 = torch.zeros((1,), dtype=torch.int32, device=dev)
        d5 = torch.empty((32, spec.DESC_DTYPE.itemsize), dtype=torch.uint8, device=dev)
        dss5 = torch.empty((spec.descriptors_workspace(4096),), dtype=torch.uint8, device=dev)
        acc = {"syrk_f64": 0.0, "eig_large_f64": 0.0}
        spec.cov_accumulate(Wl[0], C5, alpha=1.0, beta=0.0)  # warm-up
        spec.eigvalsh_large(C5, w=w5[0], ws=ws5, info=i5)
        torch.cuda.synchronize()
        for l in range(32):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            spec.cov_accumulate(Wl[l], C5, alpha=1.0, beta=0.0)
            e[1].record()
            spec.eigvalsh_large(C5, w=w5[l], ws=ws5, info=i5)
            e[2].record()
            torch.cuda.synchronize()
            acc["syrk_f64"] += e[0].elapsed_time(e[1])
            acc["eig_large_f64"] += e[1].elapsed_time(e[2])
        acc["desc"] = timed(torch, lambda: spec.descriptors(w5, mode=spec.MODE_SINGULAR, n_samples=4096, p_dim=4096,
                                                            k=1, out=d5, ws=dss5, to_host=False), 5)
        tot_seq = sum(acc.values())
        # the 32 layers as one batch with two solves in flight: layer l runs on
        # stream l % 2 with its own C and workspace (each solve is a latency
        # chain, two of them share the GPU), descriptors of all 32 spectra after
        C5b, ws5b, i5b = [C5, torch.empty_like(C5)], [ws5, torch.empty_like(ws5)], [i5, torch.zeros_like(i5)]
        st5 = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority

        def s3_batch():
            cur = torch.cuda.current_stream()
            for s_ in st5:
                s_.wait_stream(cur)
            for l in range(32):
                j = l % 2
                with torch.cuda.stream(st5[j]):
                    spec.cov_accumulate(Wl[l], C5b[j], alpha=1.0, beta=0.0)
                    spec.eigvalsh_large(C5b[j], w=w5[l], ws=ws5b[j], info=i5b[j])
            for s_ in st5:
                cur.wait_stream(s_)
            spec.descriptors(w5, mode=spec.MODE_SINGULAR, n_samples=4096, p_dim=4096, k=1, out=d5, ws=dss5,
                             to_host=False)

        s3_batch()  # warm-up (creates the second stream's state)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        s3_batch()
        torch.cuda.synchronize()
        tot = (time.perf_counter() - t0) * 1e3
        assert all(int(x.cpu()[0]) == 0 for x in i5b)
        f = 32 * 4096.0 * 4096 * 4097
        rows["s3_32x4096x4096"] = {
            "ms": tot, "two_in_flight": True, "ms_one_at_a_time": tot_seq, "phases_ms_one_at_a_time": acc,
            "layers": 32, "layer_spectra_per_s": 32e3 / tot,
            "syrk_f64": {"bound": "mfma", "achieved_TFLOPs": f / (acc["syrk_f64"] / 1e3) / 1e12,
                         "frac": f / (acc["syrk_f64"] / 1e3) / PEAK_F64_MFMA},
            "eig_4096_f64_per_s": 32e3 / acc["eig_large_f64"]}
        assert int(i5.cpu()[0]) == 0
        log(f"s3: {tot:.1f} ms two in flight, {tot_seq:.1f} ms one at a time ({acc})")
        del Wl, C5, w5, ws5
    return rows


def postproc_rows(torch, spec, dev):
    """The rows beyond the hot path (descriptor post-processing, randomised
    top-k, Ritz vectors, weight projection) on a 4096 covariance."""
    d = 4096
    rng = np.random.default_rng(2024)
    Xr = torch.from_numpy(rng.standard_normal((8192, d)).astype(np.float32)).to(dev).to(torch.bfloat16)
    C = torch.empty((d, d), dtype=torch.float32, device=dev)
    spec.cov_accumulate(Xr, C, alpha=1.0 / 8192, beta=0.0)
    ws = torch.empty((spec.eigvalsh_large_workspace(d, torch.float32),), dtype=torch.uint8, device=dev)
    Om = torch.from_numpy(rng.standard_normal((d, 32)).astype(np.float32)).to(dev)
    w_top = torch.empty((32,), dtype=torch.float32, device=dev)
    P_top = torch.empty((d, 32), dtype=torch.float32, device=dev)
    Wb = torch.from_numpy((rng.standard_normal((d, d)).astype(np.float32) / np.sqrt(d))).to(dev).to(torch.bfloat16)
    Wp_out = torch.empty((32, 32), dtype=torch.float32, device=dev)
    X_out = torch.empty((d, 32), dtype=torch.float32, device=dev)
    ws_proj = torch.empty((spec.project_weight_workspace(d),), dtype=torch.uint8, device=dev)
    S, W, N = 256, 483, 30
    wwin = torch.rand((S * W, N), device=dev).sort(dim=1, descending=True).values.contiguous()
    dwin = torch.empty((S * W, spec.DESC_DTYPE.itemsize), dtype=torch.uint8, device=dev)
    wsd = torch.empty((spec.descriptors_workspace(N),), dtype=torch.uint8, device=dev)
    spec.descriptors(wwin, n_samples=N, p_dim=4096, k=8, out=dwin, ws=wsd, to_host=False)
    sm_out = torch.empty_like(dwin)
    rb_win = torch.empty((S * W, spec.ROBUST_DTYPE.itemsize), dtype=torch.uint8, device=dev)
    # eigenvalues and the eigenvectors of the 0.8 d largest (the keep set of a
    # 0.8 keep ratio) on the same covariance; the solver destroys its input, so
    # each call starts from a copy (a 64 MB device copy, ~20 us)
    # the window eigenpairs at the EigenTrack shape: 256 streams x 512 steps,
    # N = 30, from a band of the same shape (positive window Grams)
    Hw = torch.from_numpy(rng.standard_normal((S, 512, 64)).astype(np.float32)).to(dev).to(torch.bfloat16)
    bandw = spec.gram_window(Hw, N=N)
    ww_e = torch.empty((S * W, N), dtype=torch.float32, device=dev)
    Vw_e = torch.empty((S * W, N, N), dtype=torch.float32, device=dev)
    iw_e = torch.empty((S * W,), dtype=torch.int32, device=dev)
    k_e = int(0.8 * d)
    Ce = torch.empty_like(C)
    w_e = torch.empty((d,), dtype=torch.float32, device=dev)
    Z_e = torch.empty((d, k_e), dtype=torch.float32, device=dev)
    ws_e = torch.empty((spec.eigh_large_workspace(d, torch.float32, k_e),), dtype=torch.uint8, device=dev)
    post = {
        "sliding_windows_123648_N30_r64": lambda: spec.eigvalsh_sliding(bandw, n=N, scale=1.0 / N, restart=64,
                                                                       w=ww_e, info=iw_e),
        "eigh_windows_123648_N30": lambda: spec.eigh_batched_band(bandw, n=N, scale=1.0 / N, w=ww_e, V=Vw_e,
                                                                   info=iw_e),
        "eigvalsh_large_4096_f32": lambda: (Ce.copy_(C), spec.eigvalsh_large(Ce, w=w_e, ws=ws)),
        "eigh_4096_f32_k3276": lambda: (Ce.copy_(C), spec.eigh_large(Ce, k_e, w=w_e, Z=Z_e, ws=ws_e)),
        "desc_smooth_123648": lambda: spec.desc_smooth(dwin, streams=S, W=W, alpha=0.2, out=sm_out, to_host=False),
        "robust_windows_123648": lambda: spec.spectrum_robust(wwin, n_samples=N, p_dim=4096,
                                                              sigma2_mode=spec.SIGMA2_MEDIAN, bins=8, out=rb_win,
                                                              to_host=False),
        "topk_4096_q2": lambda: spec.eigvalsh_topk(C, Om, q=2, w=w_top, ws=ws),
        "eigvecs_topk_4096_q2": lambda: spec.eigvecs_topk(C, Om, q=2, w=w_top, P=P_top, ws=ws),
        "project_weight_4096_bf16_k32": lambda: spec.project_weight(Wb, P_top, k=32, Wp=Wp_out, X=X_out, ws=ws_proj),
    }
    return {k: {"ms": timed(torch, fn, 10)} for k, fn in post.items()}


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--in-flight", type=int, default=2, help="batches in flight on their own streams in the timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-phases", action="store_true", help="skip the other workloads' phase rows")
    ap.add_argument("--no-postproc", action="store_true", help="skip the rows beyond the hot path")
    ap.add_argument("--phases", default="tiny,eigentrack,swiftsvd,s3",
                    help="comma-separated phase rows to run (tiny, eigentrack, swiftsvd, s3)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the workloads shard without communication; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import weights_bf16_fp32_amd as spec
    from gen import synth

    dev = torch.device("cuda:0")
    n, d = FFN["n"], FFN["d"]
    t0 = time.time()
    X = synth.ffn(n=n, d=d)
    log(f"ffn input generated in {time.time() - t0:.1f} s")
    Xd = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
    # F batches in flight: step i runs on stream i % F with buffer set i % F,
    # so one step's SYRK and band reduction run beside the previous steps' bulge
    # chases (latency chains on a quarter of the CUs) and panel factorisations;
    # every step is the whole path over its batch
    def buffers():
        return {"C": torch.empty((d, d), dtype=torch.float32, device=dev),
                "w": torch.empty((d,), dtype=torch.float32, device=dev),
                "ws": torch.empty((spec.eigvalsh_large_workspace(d, torch.float32),), dtype=torch.uint8, device=dev),
                "info": torch.zeros((1,), dtype=torch.int32, device=dev),
                "desc": torch.empty((1, spec.DESC_DTYPE.itemsize), dtype=torch.uint8, device=dev),
                "dws": torch.empty((spec.descriptors_workspace(d),), dtype=torch.uint8, device=dev)}
    F = args.in_flight
    sets = [buffers() for _ in range(F)]
    streams = [torch.cuda.Stream() for _ in range(F)]  # default priority

    phases = ["syrk", "eig_large", "desc"]
    ev = {p: ev_pair(torch) for p in phases}

    def step(b, events=False):
        def mark(p, i):
            if events:
                ev[p][i].record()
        mark("syrk", 0)
        spec.cov_accumulate(Xd, b["C"], alpha=1.0 / n, beta=0.0)
        mark("syrk", 1)
        mark("eig_large", 0)
        spec.eigvalsh_large(b["C"], w=b["w"], ws=b["ws"], info=b["info"])
        mark("eig_large", 1)
        mark("desc", 0)
        spec.descriptors(b["w"], n_samples=n, p_dim=d, k=1, out=b["desc"], ws=b["dws"], to_host=False)
        mark("desc", 1)

    def pipelined(i):
        with torch.cuda.stream(streams[i % F]):
            step(sets[i % F])

    # every stream of the pipeline runs at least once before the timed steps
    # (its first solve creates the stream's helper for the panel factorisations)
    W = max(args.warmup, F)
    for i in range(W):
        pipelined(i)
        log(f"warmup step {i + 1}/{W} enqueued")
    torch.cuda.synchronize()
    log("warmup done")
    # inside the timed steps only the kernels launched once per step carry HIP
    # events (an event pair costs a few microseconds of device time, and the
    # reduction launches ~900 panel kernels per step); the per-launch kernels of
    # the reduction are timed in one census step after them, and the phases of
    # one batch alone in a step of their own before it
    single = ["syrk", "bulge", "tridiag", "desc"]
    multi = ["symm", "syr2k", "panel"]
    spec.timing_enable(single)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        pipelined(W + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kt = {k: spec.timing_read(k) for k in single}
    spec.timing_enable([])
    step(sets[0], events=True)  # one batch alone, phase events only
    torch.cuda.synchronize()
    acc = {p: ev[p][0].elapsed_time(ev[p][1]) for p in phases}
    spec.timing_enable(multi)
    step(sets[0])
    torch.cuda.synchronize()
    kt.update({k: tuple(x * args.steps for x in spec.timing_read(k)) for k in multi})  # as if over K steps
    spec.timing_enable([])
    # the SYRK alone (in the timed steps it shares the GPU with a bulge chase)
    syrk_alone_ms = timed(torch, lambda: spec.cov_accumulate(Xd, sets[0]["C"], alpha=1.0 / n, beta=0.0), 3)
    log(f"{args.steps} timed steps in {wall:.3f} s")
    info, desc = sets[0]["info"], sets[0]["desc"]
    assert all(int(b["info"].cpu()[0]) == 0 for b in sets), "large eigensolver reported a failure"
    ms = dict(acc)  # one batch alone (the census step)
    ms_step = wall * 1e3 / args.steps
    rec = np.frombuffer(desc.cpu().numpy().tobytes(), dtype=spec.DESC_DTYPE)[0]

    per_step = {k: {"ms_per_step": v[0] / args.steps, "launches_per_step": v[1] / args.steps,
                    "timed_in": "timed steps" if k in single else "census step"}
                for k, v in kt.items()}
    rows = {}
    for k in ("syrk", "symm", "syr2k", "bulge"):
        tot, launches = kt[k]
        rows[k] = roofline_row(k, tot / args.steps, launches / args.steps, d, n_rows=n,
                               traffic=counter_traffic(k))
    dominant = max(rows, key=lambda k: rows[k]["avg_launch_ms"] * rows[k]["launches"])
    roof = dict(rows[dominant])
    roof["timed_in"] = per_step[dominant]["timed_in"]
    for k in ("launches", "avg_launch_ms", "algorithmic_flops", "algorithmic_bytes", "achieved_GBs"):
        roof.pop(k, None)
    syrk_tflops = rows["syrk"]["achieved"]

    phase = None
    if not args.no_phases:
        phase = phase_rows(torch, spec, synth, dev, not args.no_cpu_baseline, tuple(args.phases.split(",")))
    post = None
    if not args.no_postproc:
        post = postproc_rows(torch, spec, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample (cpu_baseline)")
        cpu = cpu_baseline(X)

    out = {
        "metric": METRIC,
        "value": 1e3 / ms_step,
        "unit": "eigensolves/s (65536x14336 bf16 -> 14336^2 f32 covariance -> all eigenvalues + descriptors)",
        "n_gpus": 1, "steps": args.steps, "warmup": W,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->f32", "data": "synthetic (seeded generator shaped like the FFN-width workload)",
        "config": {"workload": "ffn 65536x14336 bf16 -> SYRK C = X^T X / 65536 (f32) -> eigvalsh 14336 f32 "
                               "-> descriptors", "covariance_rows": n, "covariance_dim": d,
                   "batches_in_flight": F},
        "ms_per_step_one_batch_in_flight": sum(ms.values()),
        "syrk_tflops": syrk_tflops,
        "syrk_alone": {"ms": syrk_alone_ms, "TFLOPs": n * d * (d + 1) / (syrk_alone_ms / 1e3) / 1e12,
                       "frac_bf16_mfma": n * d * (d + 1) / (syrk_alone_ms / 1e3) / PEAK_BF16_MFMA},
        "eigensolves_per_s": 1e3 / ms_step,
        "phases_ms_one_batch": ms,
        "kernels_per_step": per_step,
        "n_above": int(rec["n_above"]),
        "roofline": roof,
        "roofline_all": rows,
        "phase_rows": phase,
        "postproc": post,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
