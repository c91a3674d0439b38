"""The GLU product's tolerance (the matmul bar carried through act and the
product): it admits the error the float16-weight matrix cores produce and
rejects plausible mistakes.  CPU only: the kernel's arithmetic is emulated in
float64 with each weight rounded to float16 (the matrix-core operand)."""

import numpy as np
import pytest

from _gpu import glu_bound
from oracle import codecs, encode, matmul


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
def test_glu_bound_admits_f16_weights_and_rejects_mistakes(act):
    rng = np.random.default_rng(5)
    m, n, k = 64, 40, 1024
    w = encode.quantize("q4_k", (rng.standard_normal((2 * n, k)) * 0.02).astype(np.float32))
    wg, wu = w[:n], w[n:]
    x = rng.standard_normal((m, k)).astype(np.float16)
    ref = matmul.quantized_matmul_glu("q4_k", wg, wu, k, x, act, "f16")
    g0, u0 = matmul.qmatmul("q4_k", wg, k, x), matmul.qmatmul("q4_k", wu, k, x)
    bound = glu_bound(g0, u0, act, True)
    name = "silu" if act == "silu" else "gelu"

    def emulate(wa, wb, activation=True):
        da = codecs.dequantize("q4_k", wa, k).astype(np.float16).astype(np.float64)
        db = codecs.dequantize("q4_k", wb, k).astype(np.float16).astype(np.float64)
        g = x.astype(np.float64) @ da.T
        u = x.astype(np.float64) @ db.T
        a = matmul.glu_act(name, g, np.ones_like(g)) if activation else g
        return matmul.round_out(matmul.round_out(a, "f16") * u, "f16")

    assert np.all(np.abs(emulate(wg, wu) - ref) <= bound)
    assert np.any(np.abs(emulate(wu, wg) - ref) > bound)                     # gate and up swapped
    assert np.any(np.abs(emulate(wg, wu, activation=False) - ref) > bound)   # activation dropped
    shifted = np.roll(emulate(wg, wu), 1, axis=1)                            # columns off by one
    assert np.any(np.abs(shifted - ref) > bound)
