"""libkq launches captured in a HIP graph: every replay equals the eager result.

The tile map and the expert-segment GEMM are meant to run back to back with no
host sync, so they are captured together.  Replays are interleaved with eager
work and synchronizations, and each replay's outputs are checked.
"""

import numpy as np
import pytest

from _gpu import dev, u32
from oracle import encode

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch

    from gguf_quant_matmul_amd import kq

    rng = np.random.default_rng(77)
    n, k, e = 160, 1024, 5
    w = dev(encode.quantize("q4_k", (rng.standard_normal((n, k)) * 0.02).astype(np.float32)))
    we = dev(encode.quantize("q6_k", (rng.standard_normal((e, n, k)) * 0.02).astype(np.float32)))
    xv = dev(rng.standard_normal((3, k)).astype(np.float16))
    xm = dev(rng.standard_normal((300, k)).astype(np.float16))
    ids = np.sort(rng.integers(0, e, 300)).astype(np.uint32)
    ids_d = u32(ids)
    cap = kq.kq_expert_tile_map_capacity(300, e)
    map_ = torch.zeros((cap, 3), dtype=torch.int32, device="cuda")
    counts = torch.zeros((1,), dtype=torch.int32, device="cuda")
    yv = torch.zeros((3, n), dtype=torch.float32, device="cuda")
    ym = torch.zeros((300, n), dtype=torch.float16, device="cuda")
    ys = torch.zeros((300, n), dtype=torch.float16, device="cuda")

    def work():
        kq.kq_qmv("q4_k", w, n, k, xv, yv)
        kq.kq_qmm("q4_k", w, n, k, xm, ym)
        kq.kq_expert_tile_map(ids_d, e, map_, counts)
        kq.kq_gather_qmm_seg("q6_k", we, e, n, k, xm, map_, counts, ys)

    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (yv, ym, ys, map_, counts)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (yv, ym, ys, map_, counts):
            t.zero_()
        _ = (xm.float() @ xm.float().T).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((yv, ym, ys, map_, counts), ref):
            assert torch.equal(got, want), f"replay {rep} differs"


def test_graph_replays_fused_and_other_codecs():
    # the two-pass GLU GEMM (the up pass reads what the gate pass stored), the
    # residual epilogue on the GEMV body, the GEMVs of other codecs, and the
    # wide matrix-core GEMV (plain, residual, and the GLU's two passes)
    import torch

    from gguf_quant_matmul_amd import kq

    rng = np.random.default_rng(78)
    n, k = 160, 1024

    def wq(codec, shape):
        return dev(encode.quantize(codec, (rng.standard_normal(shape + (k,)) * 0.05).astype(np.float32)))

    wg, wu, wr, wl, w2 = wq("q5_k", (n,)), wq("q5_k", (n,)), wq("q3_k", (n,)), wq("q4_1", (n,)), wq("q2_k", (n,))
    xm = dev(rng.standard_normal((130, k)).astype(np.float16))
    xr = dev(rng.standard_normal((5, k)).astype(np.float16))
    res = dev(rng.standard_normal((5, n)).astype(np.float32))
    gate = dev(rng.standard_normal(n).astype(np.float32))
    y_glu = torch.zeros((130, n), dtype=torch.float16, device="cuda")
    y_res = torch.zeros((5, n), dtype=torch.float32, device="cuda")
    y_l = torch.zeros((5, n), dtype=torch.float32, device="cuda")
    y_2 = torch.zeros((130, n), dtype=torch.float16, device="cuda")
    xw = dev(rng.standard_normal((40, k)).astype(np.float16))
    res_w = dev(rng.standard_normal((40, n)).astype(np.float16))
    y_wglu = torch.zeros((24, n), dtype=torch.float16, device="cuda")
    y_wres = torch.zeros((40, n), dtype=torch.float16, device="cuda")
    y_w = torch.zeros((40, n), dtype=torch.float32, device="cuda")
    outs = (y_glu, y_res, y_l, y_2, y_wglu, y_wres, y_w)

    def work():
        kq.kq_quantized_matmul_glu("q5_k", wg, wu, n, k, xm, y_glu, "gelu_tanh")
        kq.kq_quantized_matmul_residual("q3_k", wr, n, k, xr, res, y_res, gate)
        kq.kq_qmv("q4_1", wl, n, k, xr, y_l)
        kq.kq_qmm("q2_k", w2, n, k, xm, y_2)
        kq.kq_quantized_matmul_glu("q5_k", wg, wu, n, k, xw[:24], y_wglu, "silu")
        kq.kq_quantized_matmul_residual("q2_k", w2, n, k, xw, res_w, y_wres)
        kq.kq_quantized_matmul("q4_1", wl, n, k, xw, y_w)

    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.zero_()
        _ = (xm.float() @ xm.float().T).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got, want), f"replay {rep} differs"
