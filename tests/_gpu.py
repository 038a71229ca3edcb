"""Shared helpers of the GPU parity tests: moving stored inputs to the device,
reading results back as exact float64, and the tolerance checks.

Tolerances: fp32 I/O |err| <= 1e-5 + 1e-5*|ref| (out, last, grad_b); bf16 I/O
|err| <= 1e-5 + 1e-2*|ref|.  grad_a = lambda*h_{t-1} is a product of two
checked quantities, so its bound is the first-order propagation of theirs:
atol*(1 + |lambda| + |h_{t-1}|) + 2*rtol*|grad_a|.
"""
import sys

import numpy as np
import torch

TOL = {"f32": (1e-5, 1e-5), "bf16": (1e-2, 1e-5)}  # (rtol, atol)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_close(name, got, ref, dtype):
    rtol, atol = TOL[dtype]
    err = np.abs(got - ref)
    tol = atol + rtol * np.abs(ref)
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / tol, 0)), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} outside |err| <= {atol} + {rtol}|ref|;"
                             f" worst at {i}: got {got[i]!r} ref {ref[i]!r}")
    return float(np.max(err / tol)) if err.size else 0.0


def check_grad_a(got, ref, lam, hprev, dtype):
    rtol, atol = TOL[dtype]
    err = np.abs(got - ref)
    tol = atol * (1 + np.abs(lam) + np.abs(hprev)) + 2 * rtol * np.abs(ref)
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / tol, 0)), err.shape)
        raise AssertionError(f"grad_a: {int(bad.sum())} of {bad.size} outside the propagated bound;"
                             f" worst at {i}: got {got[i]!r} ref {ref[i]!r}")
    return float(np.max(err / tol)) if err.size else 0.0


def prev_state(h, h0=None):
    """h_{t-1} for every t (h0 or zero at t = 0)."""
    B, T, D = h.shape
    first = np.zeros((B, 1, D)) if h0 is None else np.asarray(h0, np.float64)[:, None, :]
    return np.concatenate([first, h[:, :-1]], axis=1)
