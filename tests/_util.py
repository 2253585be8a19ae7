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


def check_float(gpu: np.ndarray, ref: np.ndarray, allow: np.ndarray, tol: float = 2e-3, what: str = "",
                run: np.ndarray = None):
    """|gpu - ref| <= tol * rms(ref) + allow elementwise (allow: the oracle's flip allowance, plus for FP8 P.V the
    allowance of the FP8 dot-product reading, whose part alone is run when given). Prints how many elements lie
    beyond tol * rms (accepted only through the allowances) and, given run, how many of them need its part."""
    rms = float(np.sqrt(np.mean(np.square(ref))))
    err = np.abs(gpu.astype(np.float64) - ref)
    allow = allow if allow is not None else 0.0
    bound = tol * rms + allow
    bad = err > bound
    over = err > tol * rms
    msg = "%s: max err/rms %.3g; %d of %d elements beyond %.0e rms (accepted by the allowances)" % (
        what, float(err.max() / rms), int(over.sum()), err.size, tol)
    if run is not None:
        need_run = err > tol * rms + (allow - run)
        msg += ", %d of them only through the FP8 run allowance (their max err/rms %.3g)" % (
            int(need_run.sum()), float(err[need_run].max() / rms) if need_run.any() else 0.0)
    print(msg, flush=True)
    assert not bad.any(), "%s: %d of %d outside tol (max err/rms %.3g, rms %.3g)" % (
        what, int(bad.sum()), bad.size, float(err.max() / rms), rms)
    return float(err.max() / rms)


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = a.astype(np.float64).ravel()
    b = b.astype(np.float64).ravel()
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))
