"""Shared helpers for the GPU parity tests (HIP path vs the oracle)."""

import sys

import numpy as np

# The fp64-oracle tolerance for matmul outputs: per output row,
# max_n |y - ref| / max_n |ref| <= 2e-3 (the pages' maximum relative error read per
# row: an element-wise relative error is unbounded near zero outputs).
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


def glu_bound(g, u, act, f16, tol=TOL):
    """Per-element bound for the GLU product act(g) * u from the matmul bar.

    g and u are the fp64 oracle gate and up products [M, N].  Each may err by
    tol times its row's largest magnitude (the matmul bar), eg and eu.  The
    activation then moves by at most da = the larger of |act(g +- eg) -
    act(g)| and |act'(g)| eg (the endpoints cover its exponential tails), and
    the product by da (|u| + eu) + |act(g)| eu.  Added: for a float16 output
    the two roundings the op defines (the activation, then the product: 2^-11
    each, relative) and float16's smallest subnormal step; for float32 a few
    ulps; and a floor at float32 resolution of the row's largest product.
    """
    from oracle import matmul

    name = {"silu": "silu", "gelu_tanh": "gelu", "gelu": "gelu"}[act]
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    one = np.ones_like(g)
    a = matmul.glu_act(name, g, one)
    h = 1e-6 * np.maximum(1.0, np.abs(g))
    slope = (matmul.glu_act(name, g + h, one) - matmul.glu_act(name, g - h, one)) / (2 * h)
    eg = tol * np.max(np.abs(g), axis=1, keepdims=True)
    eu = tol * np.max(np.abs(u), axis=1, keepdims=True)
    da = np.maximum.reduce([np.abs(matmul.glu_act(name, g + eg, one) - a),
                            np.abs(matmul.glu_act(name, g - eg, one) - a), np.abs(slope) * eg])
    b = da * (np.abs(u) + eu) + np.abs(a) * eu
    rel = 2.0 ** -11 if f16 else 2.0 ** -22
    floor = 2.0 ** -22 * np.max(np.abs(a * u), axis=1, keepdims=True) + (2.0 ** -24 if f16 else 0.0)
    return b + rel * (2 * np.abs(a) * np.abs(u) + np.abs(a * u)) + floor + 1e-30


def assert_glu_close(y, ref, g, u, act, f16, what=""):
    """y within glu_bound of the oracle's GLU product ref; reports the largest
    fraction of the bound used and the row-normalized error."""
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    bound = glu_bound(g, u, act, f16)
    frac = np.abs(y - ref) / bound
    i = np.unravel_index(int(frac.argmax()), frac.shape)
    assert frac.max() <= 1.0, f"{what}: error {abs(y[i] - ref[i]):.3e} at {i} exceeds its bound {bound[i]:.3e}"
    say(f"  {what}: bound use {frac.max():.2f}, row-normalized error {row_rel_err(y, ref).max():.2e}")
    return float(frac.max())


def bf16_bound(ref, out, tol=TOL):
    """Per-element bound for bfloat16-activation products: the row bar (tol of
    the row's largest |ref|) plus, for a bfloat16 store, the one rounding the
    store defines (at most 2^-8 of the element: bfloat16 keeps 8 significant
    bits); float16 and float32 stores need nothing beyond the row bar."""
    ref = np.asarray(ref, np.float64)
    row = tol * np.max(np.abs(ref), axis=1, keepdims=True)
    return row + (2.0 ** -8 * np.abs(ref) if out == "bf16" else 0.0)


def assert_close_bf16(y, ref, out, what=""):
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - ref)
    b = bf16_bound(ref, out)
    i = np.unravel_index(int((err / b).argmax()), err.shape)
    assert np.all(err <= b), f"{what}: error {err[i]:.3e} at {i} exceeds its bound {b[i]:.3e}"
    say(f"  {what}: row-normalized error {row_rel_err(y, ref).max():.2e}, bound use {(err / b).max():.2f}")
