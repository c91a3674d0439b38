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
