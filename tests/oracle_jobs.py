"""Oracle jobs the GPU parity tests hand to child processes (spawned, so they
never touch the GPU).  Test infrastructure only: imports nothing from the
product library except the seeded input generators."""
import numpy as np

ET_FIELDS = ["S", "H", "erank", "m1", "gk", "g1", "lambda_plus", "mp_w1"]


def oracle_windows(worker, nworkers):
    """Oracle spectra and descriptors of every window of the streams s with
    s % nworkers == worker (run in a child process: it regenerates the input).
    Window Grams come from the oracle's band of inner products, which the CPU
    pins tie to the windows' definition."""
    import oracle as orc
    from gen import synth as syn
    S, T, d, N = 256, 512, 4096, 30
    W = T - N + 1
    H = syn.eigentrack(streams=S, T=T, d=d)
    idx = np.arange(N)
    lag = np.abs(idx[:, None] - idx[None, :])
    far = np.maximum(idx[:, None], idx[None, :])
    out = {}
    for s in range(worker, S, nworkers):
        B = orc.band_gram(H[s], "bf16", N)[0]
        G = np.stack([B[w + far, lag] / N for w in range(W)])
        ev, _ = orc.eigvalsh_small(G)
        rec = [orc.descriptors(ev[w], n_samples=N, p_dim=d, k=8) for w in range(W)]
        desc = {f: np.array([r[f] for r in rec]) for f in ET_FIELDS + ["n_above"]}
        out[s] = (ev, desc)
    return out


