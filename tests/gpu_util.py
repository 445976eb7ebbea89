"""Helpers shared by the GPU parity tests (device transfer and tolerance bounds)."""
import numpy as np

EPS32 = 2.0 ** -24
EPS64 = 2.0 ** -53

DESC_FLOAT_FIELDS = ["S", "H", "erank", "m1", "gk", "g1", "sigma2", "lambda_plus", "mp_w1",
                     "top_energy", "top_sigma_share", "tail_head", "tail_min", "sigma1"]
DESC_INT_FIELDS = ["n_above", "n_small", "r_pos"]


def dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def lower(M: np.ndarray) -> np.ndarray:
    return np.tril(M)


def syrk_bound(Xabs64: np.ndarray, alpha: float, eps: float, C0abs=None, beta: float = 0.0) -> np.ndarray:
    """Worst-case elementwise error of a floating-point C = beta C0 + alpha X^T X
    accumulated in precision eps over n terms: (n + 2) eps (|alpha| |X|^T |X| + |beta C0|)."""
    n = Xabs64.shape[0]
    b = abs(alpha) * (Xabs64.T @ Xabs64)
    if C0abs is not None and beta != 0.0:
        b = b + abs(beta) * C0abs
    return (n + 2) * eps * b + 1e-300


def print_case(name: str, **kw):
    """Name the case before a GPU step so a fault report says which one ran."""
    print(f"[gpu case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)
