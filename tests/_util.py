"""Shared helpers of the tests: host <-> device conversions and the tolerance checks."""
import numpy as np
import torch

import gen

DEV = "cuda:0"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def check_float(gpu: np.ndarray, ref: np.ndarray, allow: np.ndarray, tol: float = 2e-3, what: str = ""):
    """|gpu - ref| <= tol * rms(ref) + allow elementwise (allow: the oracle's flip allowance)."""
    rms = float(np.sqrt(np.mean(np.square(ref))))
    err = np.abs(gpu.astype(np.float64) - ref)
    bound = tol * rms + (allow if allow is not None else 0.0)
    bad = err > bound
    assert not bad.any(), "%s: %d of %d outside tol (max err/rms %.3g, rms %.3g)" % (
        what, int(bad.sum()), bad.size, float(err.max() / rms), rms)
    return float(err.max() / rms)


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = a.astype(np.float64).ravel()
    b = b.astype(np.float64).ravel()
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))
