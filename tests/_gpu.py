"""Helpers for the GPU parity tests (imported only by tests marked ``gpu``)."""
import sys

import numpy as np
import torch

DEV = torch.device("cuda", 0)
REL_TOL = 1e-4   # |y_gpu - y_oracle| <= 1e-4 * sum_k |w_ik| |x_tk| per element


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_parity(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, what: str = ""):
    """Element-wise fp32 parity against the fp64 oracle (exact 0 where the bound is 0)."""
    y_gpu = np.asarray(y_gpu, np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), what
    err = np.abs(y_gpu - y_ref)
    tol = REL_TOL * bound
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; worst at {i}: "
            f"gpu={y_gpu[i]!r} ref={y_ref[i]!r} err={err[i]:.3e} tol={tol[i]:.3e}")
    zero = bound == 0
    assert np.all(y_gpu[zero] == 0), what
