"""Benchmark of the spectral hot path on one MI355X.

One step is one pass of every hot-path stage over one batch of synthetic input:
  * Swift-SVD covariance: 32 incremental SYRK calls (2048 x 4096 bf16 chunks,
    fp32 C, beta = 0 then 1), the eigenvalues of the 4096 x 4096 result
    (two-stage tridiagonalisation + multisection) and their descriptors;
  * EigenTrack monitor: the band Gram of 256 streams x 512 steps x 4096 bf16
    activations (N = 30 window), the spectra of all 256 x 483 windows (batched
    Householder + bisection, one wave per window) and their descriptors.
value = spectra per second over the whole step (123,648 windows + 1 covariance).
Inputs are resident in HBM before timing.  Phase times come from HIP events on
the stream the library launches on.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # B/s
PEAK_BF16_MFMA = 2.5e15    # dense flop/s
PEAK_F32_MFMA = 157.3e12   # dense fp32 matrix-core flop/s
PEAK_F32_VALU = 78.6e12    # non-packed fp32 FMA: 256 CU x 64 lanes x 2 flop x 2.4 GHz

SW = dict(chunks=32, n=2048, d=4096)
ET = dict(streams=256, T=512, d=4096, N=30)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def make_inputs():
    from weights_bf16_fp32_amd import synth
    t = time.time()
    H = synth.eigentrack(streams=ET["streams"], T=ET["T"], d=ET["d"])
    log(f"eigentrack input generated in {time.time() - t:.1f} s")
    t = time.time()
    X = synth.swiftsvd(chunks=SW["chunks"], n=SW["n"], d=SW["d"])
    log(f"swiftsvd input generated in {time.time() - t:.1f} s")
    return H, X


def eig_traffic():
    """HBM bytes per large-eigensolver call from the committed counter summary, or
    None when the eigensolver source has changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "eig_large_4096_f32_hbm_traffic.md")
    try:
        rec = json.loads(re.search(r"```json\n(.*?)\n```", open(path).read(), re.S).group(1))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, AttributeError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    return float(rec["hbm_bytes_per_call"])


def cpu_baseline(H, X):
    """The oracle as it stands, on a bounded sample of the same step, scaled to
    spectra/s of a whole step: 4 streams of windows (Gram + Jacobi +
    descriptors), 1 of the 32 covariance chunks (x 32), the 4096 eigensolve."""
    import oracle
    cores = os.cpu_count()
    N = ET["N"]
    t0 = time.perf_counter()
    ns = 4
    for s in range(ns):
        G = oracle.window_gram(H[s], "bf16", N)
        w, _ = oracle.eigvalsh_small(G)
        for b in range(w.shape[0]):
            oracle.descriptors(w[b], n_samples=N, p_dim=ET["d"], k=8)
    t_et = (time.perf_counter() - t0) * ET["streams"] / ns
    t0 = time.perf_counter()
    C = oracle.covariance(X[0], "bf16", 1.0)
    t_cov = (time.perf_counter() - t0) * SW["chunks"]
    C = C * SW["chunks"]  # a full-size covariance for the eigensolve timing
    t0 = time.perf_counter()
    w = oracle.eigvalsh_large(C)
    oracle.descriptors(w, n_samples=SW["chunks"] * SW["n"], p_dim=SW["d"], k=1)
    t_eig = time.perf_counter() - t0
    total = t_et + t_cov + t_eig
    spectra = ET["streams"] * (ET["T"] - N + 1) + 1
    return {"value": spectra / total, "unit": "spectra/s", "cores": cores, "kind": "oracle",
            "sample": (f"4 of 256 EigenTrack streams (1932 windows: fp64 Gram, Jacobi, descriptors) x 64; "
                       f"1 of 32 covariance chunks x 32; one 4096 fp64 Householder+bisection eigensolve"),
            "seconds_per_step_est": total,
            "phases_s": {"eigentrack": t_et, "covariance": t_cov, "eig4096": t_eig}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-postproc", action="store_true",
                    help="skip the timing of the rows beyond the hot path (post-processing, top-k)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the workloads shard without communication; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import weights_bf16_fp32_amd as spec

    H, X = make_inputs()
    dev = torch.device("cuda:0")
    Hd = torch.from_numpy(H.view(np.int16)).to(dev).view(torch.bfloat16)
    Xd = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
    d, N = SW["d"], ET["N"]
    C = torch.empty((d, d), dtype=torch.float32, device=dev)
    w_big = torch.empty((d,), dtype=torch.float32, device=dev)
    ws_big = torch.empty((spec.eigvalsh_large_workspace(d, torch.float32),), dtype=torch.uint8, device=dev)
    info_big = torch.zeros((1,), dtype=torch.int32, device=dev)
    S, T = ET["streams"], ET["T"]
    W = T - N + 1
    band = torch.empty((S, T, N), dtype=torch.float32, device=dev)
    w_win = torch.empty((S * W, N), dtype=torch.float32, device=dev)
    info_win = torch.empty((S * W,), dtype=torch.int32, device=dev)
    desc_big = torch.empty((1, spec.DESC_DTYPE.itemsize), dtype=torch.uint8, device=dev)
    desc_win = torch.empty((S * W, spec.DESC_DTYPE.itemsize), dtype=torch.uint8, device=dev)
    dws_big = torch.empty((spec.descriptors_workspace(d),), dtype=torch.uint8, device=dev)
    dws_win = torch.empty((spec.descriptors_workspace(N),), dtype=torch.uint8, device=dev)
    n_total = SW["chunks"] * SW["n"]

    phases = ["syrk", "eig_large", "desc_large", "gram_band", "eig_windows", "desc_windows"]
    ev = {p: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for p in phases}

    def step(timed):
        def mark(p, i):
            if timed:
                ev[p][i].record()
        mark("syrk", 0)
        for k in range(SW["chunks"]):
            spec.cov_accumulate(Xd[k], C, alpha=1.0, beta=0.0 if k == 0 else 1.0)
        mark("syrk", 1)
        mark("eig_large", 0)
        spec.eigvalsh_large(C, w=w_big, ws=ws_big, info=info_big)
        mark("eig_large", 1)
        mark("desc_large", 0)
        spec.descriptors(w_big, n_samples=n_total, p_dim=d, k=1, out=desc_big, ws=dws_big, to_host=False)
        mark("desc_large", 1)
        mark("gram_band", 0)
        spec.gram_window(Hd, N=N, out=band)
        mark("gram_band", 1)
        mark("eig_windows", 0)
        spec.eigvalsh_batched_band(band, n=N, scale=1.0 / N, w=w_win, info=info_win)
        mark("eig_windows", 1)
        mark("desc_windows", 0)
        spec.descriptors(w_win, n_samples=N, p_dim=ET["d"], k=8, out=desc_win, ws=dws_win, to_host=False)
        mark("desc_windows", 1)

    for i in range(args.warmup):
        step(False)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    acc = {p: 0.0 for p in phases}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        for p in phases:
            acc[p] += ev[p][0].elapsed_time(ev[p][1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"{args.steps} timed steps in {wall:.3f} s")
    ms = {p: acc[p] / args.steps for p in phases}
    ms_step = wall * 1e3 / args.steps
    spectra = S * W + 1
    assert int(info_big.cpu()[0]) == 0, "large eigensolver reported a failure"
    rounds = info_win.cpu().numpy()
    assert np.all(rounds >= 0), "a window's eigensolve reported a failure"
    mean_rounds = float(rounds.mean())

    # roofline rows (algorithmic work per launch / average launch time)
    syrk_flops = SW["n"] * d * (d + 1)                  # symmetric half, per chunk launch
    syrk_t = ms["syrk"] / 1e3 / SW["chunks"]
    gram_bytes = H.nbytes + S * T * N * 4
    # per window: (4/3) n^3 for the reduction, 4 flops per Sturm step at 2 points per bisection round
    win_flops = S * W * (4.0 / 3.0 * N ** 3 + 2 * mean_rounds * N * 4)
    eig_flops = 4.0 / 3.0 * d ** 3                      # reduction to band; stages 2-3 are O(n^2 b)
    rows = {
        "eig_large": {"bound": "mfma", "achieved": eig_flops / (ms["eig_large"] / 1e3) / 1e12,
                      "peak": PEAK_F32_MFMA / 1e12, "unit": "TFLOP/s",
                      "kernels": "one call: reduction to band (TSQR panels, SYMM, SYR2K), bulge chasing, "
                                 "multisection; per-kernel times in the kernel-stats profile"},
        "syrk": {"bound": "mfma", "achieved": syrk_flops / syrk_t / 1e12, "peak": PEAK_BF16_MFMA / 1e12,
                 "unit": "TFLOP/s"},
        "gram_band": {"bound": "hbm", "achieved": gram_bytes / (ms["gram_band"] / 1e3) / 1e9,
                      "peak": PEAK_HBM / 1e9, "unit": "GB/s"},
        "eig_windows": {"bound": "alu", "achieved": win_flops / (ms["eig_windows"] / 1e3) / 1e12,
                   "peak": PEAK_F32_VALU / 1e12, "unit": "TFLOP/s"},
    }
    for r in rows.values():
        r["frac"] = r["achieved"] / r["peak"]
        r["traffic"] = None
    rows["eig_large"]["traffic"] = eig_traffic()  # HBM bytes per call (counter runs), or None if stale
    dominant = max(rows, key=lambda p: ms[p])  # the phase that takes the most time
    roof = dict(rows[dominant])
    roof["kernel"] = dominant

    post_rows = None
    if not args.no_postproc:
        # descriptor post-processing (a row beyond the hot path, timed on its own):
        # smoothing of the window descriptor series, robust / log / KL statistics of
        # the window spectra and of the 4096 spectrum
        sm_out = torch.empty_like(desc_win)
        rb_win = torch.empty((S * W, spec.ROBUST_DTYPE.itemsize), dtype=torch.uint8, device=dev)
        rb_big = torch.empty((1, spec.ROBUST_DTYPE.itemsize), dtype=torch.uint8, device=dev)
        post = {
            "desc_smooth": lambda: spec.desc_smooth(desc_win, streams=S, W=W, alpha=0.2, out=sm_out, to_host=False),
            "robust_windows": lambda: spec.spectrum_robust(w_win, n_samples=N, p_dim=ET["d"],
                                                           sigma2_mode=spec.SIGMA2_MEDIAN, bins=8, out=rb_win,
                                                           to_host=False),
            "robust_4096": lambda: spec.spectrum_robust(w_big, n_samples=n_total, p_dim=d,
                                                        sigma2_mode=spec.SIGMA2_WINSOR, bins=32, out=rb_big,
                                                        to_host=False),
        }
        # leading eigenvalues of the 4096 covariance by random projection (q = 2), on
        # the covariance rebuilt by the SYRK chunks (the eigensolve overwrote it)
        for k in range(SW["chunks"]):
            spec.cov_accumulate(Xd[k], C, alpha=1.0, beta=0.0 if k == 0 else 1.0)
        Om = torch.from_numpy(np.random.default_rng(2024).standard_normal((d, 32)).astype(np.float32)).to(dev)
        w_top = torch.empty((32,), dtype=torch.float32, device=dev)
        post["topk_4096_q2"] = lambda: spec.eigvalsh_topk(C, Om, q=2, w=w_top, ws=ws_big)
        P_top = torch.empty((d, 32), dtype=torch.float32, device=dev)
        post["eigvecs_topk_4096_q2"] = lambda: spec.eigvecs_topk(C, Om, q=2, w=w_top, P=P_top, ws=ws_big)
        Wb = torch.from_numpy((np.random.default_rng(2025).standard_normal((d, d)).astype(np.float32)
                               / np.sqrt(d))).to(dev).to(torch.bfloat16)
        Wp_out = torch.empty((32, 32), dtype=torch.float32, device=dev)
        X_out = torch.empty((d, 32), dtype=torch.float32, device=dev)
        ws_proj = torch.empty((spec.project_weight_workspace(d),), dtype=torch.uint8, device=dev)
        post["project_weight_4096_bf16_k32"] = lambda: spec.project_weight(Wb, P_top, k=32, Wp=Wp_out, X=X_out,
                                                                           ws=ws_proj)
        post_ms = {}
        for name, fn in post.items():
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                fn()
            e1.record()
            torch.cuda.synchronize()
            post_ms[name] = e0.elapsed_time(e1) / 10
        smooth_bytes = 2 * S * W * spec.DESC_DTYPE.itemsize
        robust_bytes = S * W * (N * 4 + spec.ROBUST_DTYPE.itemsize)
        post_rows = {
            "desc_smooth": {"ms": post_ms["desc_smooth"], "records": S * W, "bound": "hbm",
                            "achieved_GBs": smooth_bytes / (post_ms["desc_smooth"] / 1e3) / 1e9},
            "robust_windows": {"ms": post_ms["robust_windows"], "spectra": S * W, "bound": "hbm",
                               "achieved_GBs": robust_bytes / (post_ms["robust_windows"] / 1e3) / 1e9},
            "robust_4096": {"ms": post_ms["robust_4096"], "spectra": 1},
            # 4 products A Q (2 n^2 32 flop each, the symmetric half read twice) + 3 TSQRs
            "topk_4096_q2": {"ms": post_ms["topk_4096_q2"], "ritz_values": 32, "bound": "mfma",
                             "achieved_TFLOPs": 4 * 2.0 * d * d * 32 / (post_ms["topk_4096_q2"] / 1e3) / 1e12},
            # the same plus the 32 x 32 Jacobi and P = Q U (signal-subspace basis)
            "eigvecs_topk_4096_q2": {"ms": post_ms["eigvecs_topk_4096_q2"], "ritz_vectors": 32},
            # W' = P^T W P and W P: the bf16 weight read once (2 d^2 bytes), 2 d^2 32 flop
            "project_weight_4096_bf16_k32": {
                "ms": post_ms["project_weight_4096_bf16_k32"], "bound": "hbm",
                "achieved_GBs": 2.0 * d * d / (post_ms["project_weight_4096_bf16_k32"] / 1e3) / 1e9,
                "achieved_TFLOPs_f32": 2.0 * d * d * 32 / (post_ms["project_weight_4096_bf16_k32"] / 1e3) / 1e12},
        }
        for r in post_rows.values():
            if "achieved_GBs" in r:
                r["frac"] = r["achieved_GBs"] * 1e9 / PEAK_HBM
            if "achieved_TFLOPs" in r:
                r["frac"] = r["achieved_TFLOPs"] * 1e12 / PEAK_F32_MFMA

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample (cpu_baseline)")
        cpu = cpu_baseline(H, X)

    out = {
        "metric": "covariance SYRK TFLOP/s + eigensolves/sec; % of MFMA/HBM roofline, 1 GPU",
        "value": spectra / (ms_step / 1e3),
        "unit": "spectra/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->f32", "data": "synthetic (seeded generators shaped like the pages' workloads)",
        "config": {"workload": "eigentrack 256x512x4096 bf16 N=30 + swiftsvd 32x2048x4096 bf16 -> eig 4096 f32",
                   "windows": S * W, "covariance_dim": d, "covariance_rows": n_total},
        "syrk_tflops": rows["syrk"]["achieved"],
        "eigensolves_per_s": spectra / (ms_step / 1e3),
        "phases_ms": ms,
        "window_mean_bisection_rounds": mean_rounds,
        "roofline": roof,
        "roofline_all": rows,
        "postproc": post_rows,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
