"""Write the oracle's expected values for the full-size workloads.

Calls only the fp64 oracle (``oracle/``) and the seeded input generators; no
value here comes from the GPU path.  For each workload it records the SHA-256
of the generated input (so a test can confirm it regenerated the same bits),
the oracle's eigenvalues (descending) and the oracle's descriptors.

    python tests/golden/make_golden.py swiftsvd      # 32 x 2048 x 4096 bf16 chunks
    python tests/golden/make_golden.py ffn           # 65536 x 14336 bf16

Outputs: tests/golden/<workload>[_<layer>].npz with arrays ``eig`` (fp64),
``desc_json`` (the descriptor dict as JSON text) and ``sha256``.
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from gen import synth  # noqa: E402

DESC_KW = {
    "swiftsvd": dict(n_samples=32 * 2048, p_dim=4096, k=1),
    "ffn": dict(n_samples=65536, p_dim=14336, k=1),
    "s3": dict(mode=oracle.SINGULAR, n_samples=4096, p_dim=4096, k=1),
}


def save(name, eig, desc, sha, extra=None):
    path = os.path.join(HERE, name + ".npz")
    arrays = dict(eig=np.asarray(eig, np.float64), desc_json=np.array(json.dumps(desc)), sha256=np.array(sha))
    for k, v in (extra or {}).items():
        arrays[k] = np.asarray(v)
    np.savez_compressed(path, **arrays)
    print("wrote", path, flush=True)


def swiftsvd():
    t = time.time()
    d = 4096
    acc = np.zeros((d, d))
    hashes = []
    for k in range(32):
        X = synth.swiftsvd_chunk(k)
        hashes.append(synth.sha256(X))
        acc = oracle.covariance(X, "bf16", 1.0, C0=acc, beta=1.0)
    print("covariance", time.time() - t, flush=True)
    w = oracle.eigvalsh_large(acc)
    print("eig", time.time() - t, flush=True)
    desc = oracle.descriptors(w, **DESC_KW["swiftsvd"])
    save("swiftsvd", w, desc, ",".join(hashes), {"trace": np.trace(acc)})


def s3(layers):
    for l in layers:
        t = time.time()
        W = synth.s3_layer(l)
        C = oracle.covariance(W, "f32", 1.0)
        w = oracle.eigvalsh_large(C)
        desc = oracle.descriptors(w, **DESC_KW["s3"])
        save(f"s3_{l}", w, desc, synth.sha256(W))
        print("layer", l, time.time() - t, flush=True)


def ffn():
    t = time.time()
    X = synth.ffn()
    sha = synth.sha256(X)
    print("generated", time.time() - t, flush=True)
    C = oracle.covariance(X, "bf16", 1.0 / 65536)
    del X
    print("covariance", time.time() - t, flush=True)
    w = oracle.eigvalsh_large(C)
    print("eig", time.time() - t, flush=True)
    desc = oracle.descriptors(w, **DESC_KW["ffn"])
    lp = desc["lambda_plus"]
    # independent exact count from the inertia of C - lambda_plus I (Sylvester)
    inertia_above = C.shape[0] - oracle.count_below_dense(C, lp)
    print("inertia", time.time() - t, flush=True)
    save("ffn", w, desc, sha, {"n_above_inertia": inertia_above})


if __name__ == "__main__":
    what = sys.argv[1]
    if what == "swiftsvd":
        swiftsvd()
    elif what == "s3":
        s3([int(a) for a in sys.argv[2:]] or [0])
    elif what == "ffn":
        ffn()
    else:
        raise SystemExit("unknown workload " + what)
