"""Shared helpers of the GPU parity tests."""
import numpy as np
import torch

DEV = "cuda:0"
TOL_BF16 = 1e-2      # max|y - y_ref| / max|y_ref| for bf16 inputs
TOL_F32 = 1e-5       # same, fp32 inputs


def dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def wdtype(inp):
    return torch.bfloat16 if inp.dtype == "bf16" else torch.float32


def tol(inp):
    return TOL_BF16 if inp.dtype == "bf16" else TOL_F32


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.abs(ref).max()
    if scale == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / scale)


def host(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def sample_rows(T: int, n: int, k: int, seed: int = 0) -> np.ndarray:
    """Rows for sampled checks: the whole first and last chunk plus k random rows."""
    rng = np.random.default_rng(seed)
    first = np.arange(0, min(n, T))
    last = np.arange(max(0, T - n), T)
    rand = rng.choice(T, size=min(k, T), replace=False)
    return np.unique(np.concatenate([first, last, rand]))
