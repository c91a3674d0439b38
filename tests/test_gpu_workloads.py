"""GPU parity at the workloads' full sizes (the five configurations, the other
codecs' rows and the fused epilogues' prefill rows), in the launch
configuration the benchmark times, with EVERY output compared.

For each workload: the float32 weights are drawn (seeded, see
gguf_quant_matmul_amd/workloads.py) and encoded twice, on the GPU by
kq_quantize and on the host by the oracle encoder (tests/_full.py runs it in
row chunks on a thread pool); all bytes must be equal.  The kernel runs over
the whole tensor into an output filled with NaN beforehand, and every output
element is compared with the fp64 oracle computed from the oracle's own bytes
(a skipped or duplicated tile, or an unwritten row, shows up as NaN or as an
error).  Dequantize is compared bit for bit on every row (in row chunks).
"""

import numpy as np
import pytest

import _full as F
from _gpu import assert_close_rows, assert_glu_close, dev, host, say, u32
from gguf_quant_matmul_amd import workloads as W
from oracle import codecs, matmul

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kq():
    from gguf_quant_matmul_amd import kq as mod

    yield mod
    F.clear()


def _nan(shape, dtype):
    import torch

    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def _encoded(kq, codec, seed, n, k, dist="normal"):
    """(GPU-encoded device bytes, oracle bytes), checked equal over every row."""
    import torch

    wdev = dev(W.weight_rows(seed, n, k, dist))
    wq = torch.empty((n, codecs.row_bytes(codec, k)), dtype=torch.uint8, device="cuda")
    kq.kq_quantize(codec, wdev, wq)
    del wdev
    ob = F.oracle_bytes(codec, seed, n, k, dist)
    same = torch.equal(wq, dev(ob))
    assert same, f"kq_quantize bytes differ from the oracle encoder ({codec}, {n}x{k}, seed {seed})"
    return wq, ob


GEMV_CFGS = [W.Q4K_DECODE_GEMV, *W.Q8_0_Q4_0_GEMVS, W.Q6K_LMHEAD_GEMV, W.Q4K_PREFILL_GEMM,
             W.Q5K_GEMV, W.Q5K_GEMM, *W.LEGACY_GEMV, W.Q2K_GEMV, W.Q3K_GEMV]


@pytest.mark.parametrize("cfg", GEMV_CFGS, ids=[c.name for c in GEMV_CFGS])
def test_gemv_gemm_workload(kq, cfg):
    import torch

    say(f"workload {cfg.name}: encoding (GPU and oracle)")
    wq, ob = _encoded(kq, cfg.codec, cfg.seed, cfg.n, cfg.k, cfg.dist)
    x = W.gemv_activations(cfg)
    out_t = torch.float32 if cfg.out_dtype == "f32" else torch.float16
    y = _nan((cfg.m, cfg.n), out_t)
    say(f"workload {cfg.name}: kernel")
    if cfg.m <= 8:
        kq.kq_qmv(cfg.codec, wq, cfg.n, cfg.k, dev(x), y)
    else:
        kq.kq_qmm(cfg.codec, wq, cfg.n, cfg.k, dev(x), y)
    got = host(y).astype(np.float64)
    say(f"workload {cfg.name}: oracle over all {cfg.n} columns")
    ref = F.qmatmul(cfg.codec, ob, cfg.k, x)
    err = assert_close_rows(got, ref, what=cfg.name)
    say(f"workload {cfg.name}: max row-normalized error {err:.2e} over {got.size} outputs")

    if cfg.m == 1:
        say(f"workload {cfg.name}: dequantize, every row")
        step = 8192
        out = torch.empty((step, cfg.k), dtype=torch.float32, device="cuda")
        for a in range(0, cfg.n, step):
            b = min(cfg.n, a + step)
            kq.kq_dequantize(cfg.codec, wq[a:b], cfg.k, out[: b - a])
            want = F.dequantize(cfg.codec, ob[a:b], cfg.k)
            assert np.array_equal(host(out[: b - a]).view(np.uint32), want.view(np.uint32)), (cfg.name, a)
    del wq, y
    torch.cuda.empty_cache()


def test_moe_seg_workload(kq):
    import torch

    cfg = W.MOE_SEG_Q4K
    rows_w = cfg.n_experts * cfg.n
    say(f"workload {cfg.name}: encoding (GPU and oracle)")
    wq, ob = _encoded(kq, cfg.codec, cfg.seed, rows_w, cfg.k)
    rb = ob.shape[1]
    ob3 = ob.reshape(cfg.n_experts, cfg.n, rb)
    r = W.routing(cfg.seed, cfg.tokens, cfg.top_k, cfg.n_experts)
    x = W.activations(cfg.seed, cfg.tokens, cfg.k)[r.token_of_row]
    rows = x.shape[0]
    cap = kq.kq_expert_tile_map_capacity(rows, cfg.n_experts)
    map_ = torch.empty((cap, 3), dtype=torch.int32, device="cuda")
    counts = torch.empty((1,), dtype=torch.int32, device="cuda")
    say(f"workload {cfg.name}: tile map + seg")
    kq.kq_expert_tile_map(u32(r.sorted_ids), cfg.n_experts, map_, counts)
    y = _nan((rows, cfg.n), torch.float16)
    kq.kq_gather_qmm_seg(cfg.codec, wq, cfg.n_experts, cfg.n, cfg.k, dev(x), map_, counts, y)
    count = int(host(counts)[0])
    tiles, ref_count = matmul.expert_tile_map(r.sorted_ids, cfg.n_experts)
    assert count == ref_count == 92
    assert np.array_equal(host(map_)[:count].view(np.uint32), tiles)
    say(f"workload {cfg.name}: oracle over all {cfg.n} columns")
    ref = F.gather_qmm_seg(cfg.codec, ob3, cfg.k, x, tiles)
    got = host(y).astype(np.float64)
    err = assert_close_rows(got, ref, what=cfg.name)
    say(f"workload {cfg.name}: max row-normalized error {err:.2e} over {got.size} outputs")

    # the sorted rows back to token order, weighted by routing scores
    scores = W.routing_scores(cfg.seed, cfg.tokens, cfg.top_k)
    inv = r.inv_order
    mixed = _nan((cfg.tokens, cfg.n), torch.float16)
    kq.kq_gather_mix(y, u32(inv), dev(scores), mixed)
    y_host = host(y).astype(np.float64)
    refm = matmul.gather_mix(y_host, inv, scores)
    terms = (np.abs(scores.astype(np.float64))[:, :, None] *
             np.abs(y_host[inv.astype(np.int64)]).reshape(cfg.tokens, cfg.top_k, cfg.n)).sum(axis=1)
    bound = cfg.top_k * 2.0 ** -23 * terms + 2.0 ** -11 * np.abs(refm) + 2.0 ** -24
    excess = np.abs(host(mixed).astype(np.float64) - refm) - bound
    assert np.all(excess <= 0), f"gather_mix max excess {excess.max():.3e}"
    say(f"workload MoE gather_mix ({cfg.tokens} tok x top-{cfg.top_k}, N={cfg.n}): within the f32-sum + f16 bound")

    # decode shape on the same experts: token 0's eight routed rows through
    # kq_gather_qmv, every column
    ids0 = r.ids[0].astype(np.uint32)
    xd = np.repeat(W.activations(cfg.seed, cfg.tokens, cfg.k)[:1], cfg.top_k, axis=0)
    yd = _nan((cfg.top_k, cfg.n), torch.float16)
    kq.kq_gather_qmv(cfg.codec, wq, cfg.n_experts, cfg.n, cfg.k, dev(xd), u32(ids0), yd)
    refd = matmul.gather_qmv(cfg.codec, ob3, cfg.k, xd, ids0)
    errd = assert_close_rows(host(yd).astype(np.float64), refd, what="MoE decode gather_qmv")
    say(f"workload MoE decode gather_qmv (token 0, top-{cfg.top_k}): max row-normalized error {errd:.2e}")

    # decode GLU gather: these experts as gate, an up stack drawn the same way
    # (seed + 100), token 0's slots, silu
    wu, obu = _encoded(kq, cfg.codec, cfg.seed + 100, rows_w, cfg.k)
    x0 = W.activations(cfg.seed, cfg.tokens, cfg.k)[:1]
    yg = _nan((cfg.top_k, cfg.n), torch.float16)
    kq.kq_moe_glu_gather(cfg.codec, wq, wu, cfg.n_experts, cfg.n, cfg.k, dev(x0), u32(ids0[None, :]), yg, "silu")
    refg = matmul.moe_glu_gather(cfg.codec, ob3, obu.reshape(cfg.n_experts, cfg.n, rb), cfg.k, x0,
                                 ids0[None, :], "silu")
    errg = assert_close_rows(host(yg).astype(np.float64), refg, what="MoE decode GLU gather")
    say(f"workload MoE decode GLU gather (token 0, top-{cfg.top_k}, silu): max row-normalized error {errg:.2e}")
    del wq, wu, y, yd, yg, mixed
    F.clear()
    torch.cuda.empty_cache()


def test_glu_prefill_workload(kq):
    # the GLU bench rows: q4_K gate (the GEMM workload's weights) and up (seed
    # + 100), 2048 x 14336 x 4096 and 16 x 14336 x 4096, float16 out, silu
    import torch

    c = W.Q4K_PREFILL_GEMM
    say("workload GLU prefill: encoding (GPU and oracle)")
    wg, og = _encoded(kq, c.codec, c.seed, c.n, c.k)
    wu, ou = _encoded(kq, c.codec, c.seed + 100, c.n, c.k)
    x = W.gemv_activations(c)
    y = _nan((c.m, c.n), torch.float16)
    say("workload GLU prefill: kernel")
    kq.kq_quantized_matmul_glu(c.codec, wg, wu, c.n, c.k, dev(x), y, "silu")
    say("workload GLU prefill: oracle over all columns")
    ref, g, u = F.glu(c.codec, og, ou, c.k, x, "silu", "f16")
    assert_glu_close(host(y), ref, g, u, "silu", True, what="GLU prefill")
    # the small-batch GLU row: the first 16 activation rows (the wide
    # matrix-core GEMV's two passes)
    y16 = _nan((16, c.n), torch.float16)
    say("workload GLU batch 16: kernel")
    kq.kq_quantized_matmul_glu(c.codec, wg, wu, c.n, c.k, dev(x[:16]), y16, "silu")
    ref16, g16, u16 = F.glu(c.codec, og, ou, c.k, x[:16], "silu", "f16")
    assert_glu_close(host(y16), ref16, g16, u16, "silu", True, what="GLU batch 16")
    del wg, wu, y, y16
    torch.cuda.empty_cache()


def test_residual_prefill_workload(kq):
    # the residual bench row: the q4_K down projection 4096 x 14336 (seed + 200)
    # over activations [2048, 14336] (seed + 200), residual [2048, 4096]
    # (seed + 201) updated in place, float16
    import torch

    c = W.Q4K_PREFILL_GEMM
    n, k = c.k, c.n
    say("workload residual prefill: encoding (GPU and oracle)")
    wd, od = _encoded(kq, c.codec, c.seed + 200, n, k)
    x = W.activations(c.seed + 200, c.m, k)
    res = W.activations(c.seed + 201, c.m, n)
    y = dev(res)
    say("workload residual prefill: kernel")
    kq.kq_quantized_matmul_residual(c.codec, wd, n, k, dev(x), y, y)
    say("workload residual prefill: oracle over all columns")
    ref = F.residual(c.codec, od, k, x, res)
    assert_close_rows(host(y).astype(np.float64), ref, what="residual prefill")
    del wd, y
    torch.cuda.empty_cache()


def test_small_prefill_workload(kq):
    # the small-prefill bench rows: the GEMM workload's q4_K 14336 x 4096 weight
    # with the first M of its activation rows through kq_quantized_matmul,
    # float16 out (16, 32 and 64 rows: the wide matrix-core GEMV on one, two
    # and four activation operands; 128: the GEMM)
    import torch

    c = W.Q4K_PREFILL_GEMM
    say("workload small prefill: encoding (GPU and oracle)")
    wq, ob = _encoded(kq, c.codec, c.seed, c.n, c.k)
    xa = W.gemv_activations(c)
    for m in (16, 32, 64, 128):
        x = xa[:m]
        y = _nan((m, c.n), torch.float16)
        say(f"workload small prefill: M={m}")
        kq.kq_quantized_matmul(c.codec, wq, c.n, c.k, dev(x), y)
        ref = F.qmatmul(c.codec, ob, c.k, x)
        assert_close_rows(host(y).astype(np.float64), ref, what=f"small prefill M={m}")
    del wq, y
    torch.cuda.empty_cache()
