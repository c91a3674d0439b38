"""Shared helpers for the GPU parity tests (HIP path vs the oracle)."""

import sys

import numpy as np

# The fp64-oracle tolerance for matmul outputs: per output row,
# max_n |y - ref| / max_n |ref| <= 2e-3 (tolerance reading).
TOL = 2e-3


def torch_mod():
    import torch

    return torch


def dev(a, dtype=None):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def u32(a):
    """uint32 numpy array -> int32 device tensor holding the same bits."""
    return dev(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32))


def host(t):
    torch = torch_mod()
    torch.cuda.synchronize()
    return t.cpu().numpy()


def row_rel_err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.max(np.abs(ref), axis=1)
    denom = np.where(denom == 0, 1.0, denom)
    return np.max(np.abs(y - ref), axis=1) / denom


def assert_close_rows(y, ref, tol=TOL, what=""):
    err = row_rel_err(y, ref)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert err.max() <= tol, f"{what}: row-normalized max error {err.max():.3e} > {tol} (row {int(err.argmax())})"
    say(f"  {what}: worst row error {err.max():.2e}")
    return float(err.max())


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
