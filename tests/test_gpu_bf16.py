"""GPU parity of the bfloat16-activation entry points (kq_qmv_bf16,
kq_qmm_bf16, kq_gather_qmm_seg_bf16) against the fp64 oracle.

The oracle is the same fp64 product: a bfloat16 activation is exact in
float64.  Bar: per row, max |y - ref| <= 2e-3 of the row's largest |ref|,
plus for a bfloat16 store the one rounding it defines (2^-8 of the element);
see tests/_gpu.py bf16_bound.  Shapes span several 64-row column blocks with
ragged tails, 1 to 16 GEMV rows, row tiles of 16 / 64 / 128 GEMM rows, and
activations far outside float16's range.
"""

import numpy as np
import pytest

import _full as F
from _gpu import assert_close_bf16, dev, host, say, u32
from gguf_quant_matmul_amd import workloads as W
from oracle import codecs, encode, matmul

pytestmark = pytest.mark.gpu

CODECS = ("q4_k", "q6_k", "q8_0", "q4_0", "q5_k", "q4_1", "q5_0", "q5_1", "q2_k", "q3_k")
SUPER = ("q4_k", "q5_k", "q6_k", "q2_k", "q3_k")
OUTS = ("f32", "f16", "bf16")


@pytest.fixture(scope="module")
def kq():
    from gguf_quant_matmul_amd import kq as mod

    return mod


def _tdt(out):
    import torch

    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out]


def _xb(m, k, seed, scale=1.0):
    return W.to_bf16((np.random.default_rng(seed).standard_normal((m, k)) * scale).astype(np.float32))


def _devb(a):
    import torch

    return dev(a).to(torch.bfloat16)


def _got(y):
    import torch

    return host(y.to(torch.float32)).astype(np.float64)


@pytest.mark.parametrize("codec", CODECS)
def test_bf16_qmv_qmm_parity(kq, codec):
    import torch

    k = 512 if codec in SUPER else 320
    for m, n in ((1, 100), (3, 1000), (16, 200), (17, 130), (130, 200), (300, 70)):
        w = F.random_bytes(codec, n, k, 51 + n)
        x = _xb(m, k, 52 + m)
        ref = F.qmatmul(codec, w, k, x)
        for out in OUTS:
            say(f"bf16 {codec} m={m} n={n} k={k} out={out}")
            y = torch.full((m, n), float("nan"), dtype=_tdt(out), device="cuda")
            fn = kq.kq_qmv if m <= 16 else kq.kq_qmm
            fn(codec, dev(w), n, k, _devb(x), y)
            assert_close_bf16(_got(y), ref, out, what=f"bf16 {codec} m={m} n={n} {out}")
        # kq_quantized_matmul routes bfloat16 activations the same way
        yq = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        kq.kq_quantized_matmul(codec, dev(w), n, k, _devb(x), yq)
        assert_close_bf16(_got(yq), ref, "f32", what=f"bf16 quantized_matmul {codec} m={m}")


@pytest.mark.parametrize("codec", ["q4_k", "q6_k", "q8_0", "q4_0"])
def test_bf16_long_k(kq, codec):
    # K = 14336 (a down projection): the GEMV's sixteen waves each walk seven
    # groups of four K steps, the matmul tile 112 staged chunks
    import torch

    k, n = 14336, 72
    w = F.random_bytes(codec, n, k, 81)
    for m in (2, 40):
        x = _xb(m, k, 82 + m)
        ref = F.qmatmul(codec, w, k, x)
        say(f"bf16 long K {codec} m={m}")
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        (kq.kq_qmv if m <= 16 else kq.kq_qmm)(codec, dev(w), n, k, _devb(x), y)
        assert_close_bf16(_got(y), ref, "f32", what=f"bf16 long K {codec} m={m}")


@pytest.mark.parametrize("scale", [2.0 ** -60, 2.0 ** 60])
def test_bf16_activations_outside_f16_range(kq, scale):
    import torch

    for codec in ("q4_k", "q8_0"):
        k, n, m = 256, 96, 20
        w = F.random_bytes(codec, n, k, 61)
        x = _xb(m, k, 62, scale)
        ref = F.qmatmul(codec, w, k, x)
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        kq.kq_qmm(codec, dev(w), n, k, _devb(x), y)
        assert_close_bf16(_got(y), ref, "f32", what=f"bf16 x scale {scale} {codec}")


@pytest.mark.parametrize("codec", CODECS)
def test_bf16_seg_parity(kq, codec):
    import torch

    rng = np.random.default_rng(71)
    e, n = 4, 150
    k = 512 if codec in SUPER else 320
    sizes = [96, 20, 64, 133]
    ids = np.concatenate([np.full(c, i, np.uint32) for i, c in enumerate(sizes)] + [np.full(3, e + 1, np.uint32)])
    rows = ids.size
    w = encode.quantize(codec, (rng.standard_normal((e, n, k)) * 0.02).astype(np.float32))
    x = _xb(rows, k, 72)
    cap = kq.kq_expert_tile_map_capacity(rows, e)
    map_ = torch.full((cap, 3), -1, dtype=torch.int32, device="cuda")
    counts = torch.zeros((1,), dtype=torch.int32, device="cuda")
    kq.kq_expert_tile_map(u32(ids), e, map_, counts)
    count = int(host(counts)[0])
    tiles = host(map_)[:count].view(np.uint32)
    ref = matmul.gather_qmm_seg(codec, w, k, x, tiles)
    covered = ids < e
    for out in OUTS:
        say(f"bf16 seg {codec} {out}")
        y = torch.full((rows, n), float("nan"), dtype=_tdt(out), device="cuda")
        kq.kq_gather_qmm_seg(codec, dev(w), e, n, k, _devb(x), map_, counts, y)
        got = _got(y)
        assert np.all(np.isnan(got[~covered])), "uncovered rows must stay unwritten"
        assert_close_bf16(got[covered], ref[covered], out, what=f"bf16 seg {codec} {out}")


def _encoded(kq, codec, seed, n, k, dist="normal"):
    import torch

    wdev = dev(W.weight_rows(seed, n, k, dist))
    wq = torch.empty((n, codecs.row_bytes(codec, k)), dtype=torch.uint8, device="cuda")
    kq.kq_quantize(codec, wdev, wq)
    del wdev
    ob = F.oracle_bytes(codec, seed, n, k, dist)
    assert torch.equal(wq, dev(ob))
    return wq, ob


@pytest.mark.parametrize("which", ["gemv", "gemm", "seg"])
def test_bf16_workloads_full(kq, which):
    # the q4_K decode GEMV (f32 out), prefill GEMM and MoE segment GEMM
    # (bfloat16 out, x's dtype) with the workloads' activations rounded to
    # bfloat16; every output compared
    import torch

    if which in ("gemv", "gemm"):
        c = W.Q4K_DECODE_GEMV if which == "gemv" else W.Q4K_PREFILL_GEMM
        wq, ob = _encoded(kq, c.codec, c.seed, c.n, c.k)
        x = W.activations_bf16(c.seed, c.m, c.k)
        out = "f32" if which == "gemv" else "bf16"
        y = torch.full((c.m, c.n), float("nan"), dtype=_tdt(out), device="cuda")
        say(f"bf16 workload {c.name}")
        (kq.kq_qmv if which == "gemv" else kq.kq_qmm)(c.codec, wq, c.n, c.k, _devb(x), y)
        assert_close_bf16(_got(y), F.qmatmul(c.codec, ob, c.k, x), out, what=f"bf16 {c.name}")
    else:
        c = W.MOE_SEG_Q4K
        wq, ob = _encoded(kq, c.codec, c.seed, c.n_experts * c.n, c.k)
        r = W.routing(c.seed, c.tokens, c.top_k, c.n_experts)
        x = W.activations_bf16(c.seed, c.tokens, c.k)[r.token_of_row]
        rows = x.shape[0]
        cap = kq.kq_expert_tile_map_capacity(rows, c.n_experts)
        map_ = torch.empty((cap, 3), dtype=torch.int32, device="cuda")
        counts = torch.empty((1,), dtype=torch.int32, device="cuda")
        kq.kq_expert_tile_map(u32(r.sorted_ids), c.n_experts, map_, counts)
        tiles, _ = matmul.expert_tile_map(r.sorted_ids, c.n_experts)
        y = torch.full((rows, c.n), float("nan"), dtype=torch.bfloat16, device="cuda")
        say(f"bf16 workload {c.name}")
        kq.kq_gather_qmm_seg(c.codec, wq, c.n_experts, c.n, c.k, _devb(x), map_, counts, y)
        ref = F.gather_qmm_seg(c.codec, ob.reshape(c.n_experts, c.n, -1), c.k, x, tiles)
        assert_close_bf16(_got(y), ref, "bf16", what=f"bf16 {c.name}")
    F.clear()
    torch.cuda.empty_cache()
