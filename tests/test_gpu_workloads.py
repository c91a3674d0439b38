"""GPU parity at the workloads' full sizes (the five configurations, the other
codecs' rows and the fused epilogues' prefill rows), in the launch
configuration the benchmark times, checked on sampled outputs the oracle
computes one by one.

For each workload: the float32 weights are drawn (seeded, see
gguf_quant_matmul_amd/workloads.py), encoded on the GPU by kq_quantize, and the
GPU bytes of sampled rows must equal the oracle encoder's bytes for those rows.
The kernel runs over the whole tensor; sampled output columns (all activation
rows) are compared with the fp64 oracle; dequantize is compared bit for bit on
the sampled rows.
"""

import numpy as np
import pytest

from _gpu import assert_close_rows, assert_glu_close, dev, host, say, u32
from gguf_quant_matmul_amd import workloads as W
from oracle import codecs, encode, matmul

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kq():
    from gguf_quant_matmul_amd import kq as mod

    return mod


def _sample(n, count, seed):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(n, count - 2, replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(s))


GEMV_CFGS = [W.CFG1_Q4K_GEMV, *W.CFG2_GEMV, W.CFG3_Q6K_LMHEAD, W.CFG4_Q4K_GEMM,
             W.Q5K_GEMV, W.Q5K_GEMM, *W.LEGACY_GEMV, W.Q2K_GEMV, W.Q3K_GEMV]


@pytest.mark.parametrize("cfg", GEMV_CFGS, ids=[c.name for c in GEMV_CFGS])
def test_gemv_gemm_workload(kq, cfg):
    import torch

    say(f"workload {cfg.name}: drawing weights")
    wf = W.weight_rows(cfg.seed, cfg.n, cfg.k, cfg.dist)
    wdev = dev(wf)
    del wf
    rb = codecs.row_bytes(cfg.codec, cfg.k)
    wq = torch.empty((cfg.n, rb), dtype=torch.uint8, device="cuda")
    kq.kq_quantize(cfg.codec, wdev, wq)
    del wdev
    ns = _sample(cfg.n, 48, cfg.seed)
    wf_s = W.weight_rows(cfg.seed, cfg.n, cfg.k, cfg.dist, rows=ns)
    ref_bytes = encode.quantize(cfg.codec, wf_s)
    got_bytes = host(wq[torch.from_numpy(ns).cuda()])
    assert np.array_equal(got_bytes, ref_bytes), "kq_quantize bytes differ from the oracle encoder"

    x = W.gemv_activations(cfg)
    out_t = torch.float32 if cfg.out_dtype == "f32" else torch.float16
    y = torch.empty((cfg.m, cfg.n), dtype=out_t, device="cuda")
    say(f"workload {cfg.name}: kernel")
    if cfg.m <= 8:
        kq.kq_qmv(cfg.codec, wq, cfg.n, cfg.k, dev(x), y)
    else:
        kq.kq_qmm(cfg.codec, wq, cfg.n, cfg.k, dev(x), y)
    got = host(y)[:, ns].astype(np.float64)
    ref = matmul.qmatmul(cfg.codec, ref_bytes, cfg.k, x)
    err = assert_close_rows(got, ref, what=cfg.name)
    say(f"workload {cfg.name}: max row-normalized error {err:.2e}")

    if cfg.m == 1:
        say(f"workload {cfg.name}: dequantize")
        out = torch.empty((ns.size, cfg.k), dtype=torch.float32, device="cuda")
        kq.kq_dequantize(cfg.codec, wq[torch.from_numpy(ns).cuda()].contiguous(), cfg.k, out)
        assert np.array_equal(host(out).view(np.uint32), codecs.dequantize(cfg.codec, ref_bytes, cfg.k).view(np.uint32))
    del wq, y
    torch.cuda.empty_cache()


def test_moe_seg_workload(kq):
    import torch

    cfg = W.CFG5_MOE_SEG
    say(f"workload {cfg.name}: drawing weights")
    rows_w = cfg.n_experts * cfg.n
    wdev = dev(W.weight_rows(cfg.seed, rows_w, cfg.k))
    rb = codecs.row_bytes(cfg.codec, cfg.k)
    wq = torch.empty((rows_w, rb), dtype=torch.uint8, device="cuda")
    kq.kq_quantize(cfg.codec, wdev, wq)
    del wdev
    r = W.routing(cfg.seed, cfg.tokens, cfg.top_k, cfg.n_experts)
    x = W.activations(cfg.seed, cfg.tokens, cfg.k)[r.token_of_row]
    rows = x.shape[0]
    cap = kq.kq_expert_tile_map_capacity(rows, cfg.n_experts)
    map_ = torch.empty((cap, 3), dtype=torch.int32, device="cuda")
    counts = torch.empty((1,), dtype=torch.int32, device="cuda")
    say(f"workload {cfg.name}: tile map + seg")
    kq.kq_expert_tile_map(u32(r.sorted_ids), cfg.n_experts, map_, counts)
    y = torch.empty((rows, cfg.n), dtype=torch.float16, device="cuda")
    kq.kq_gather_qmm_seg(cfg.codec, wq, cfg.n_experts, cfg.n, cfg.k, dev(x), map_, counts, y)
    count = int(host(counts)[0])
    tiles, ref_count = matmul.expert_tile_map(r.sorted_ids, cfg.n_experts)
    assert count == ref_count == 92
    assert np.array_equal(host(map_)[:count].view(np.uint32), tiles)

    ns = _sample(cfg.n, 24, cfg.seed)
    widx = (np.arange(cfg.n_experts)[:, None] * cfg.n + ns[None, :]).reshape(-1)
    wf_s = W.weight_rows(cfg.seed, rows_w, cfg.k, rows=widx)
    ref_bytes = encode.quantize(cfg.codec, wf_s)
    assert np.array_equal(host(wq[torch.from_numpy(widx).cuda()]), ref_bytes)
    ref = matmul.gather_qmm_seg(cfg.codec, ref_bytes.reshape(cfg.n_experts, ns.size, rb), cfg.k, x, tiles)
    got = host(y)[:, ns].astype(np.float64)
    err = assert_close_rows(got, ref, what=cfg.name)
    say(f"workload {cfg.name}: max row-normalized error {err:.2e}")

    # the sorted rows back to token order, weighted by routing scores
    scores = W.routing_scores(cfg.seed, cfg.tokens, cfg.top_k)
    inv = r.inv_order
    mixed = torch.empty((cfg.tokens, cfg.n), dtype=torch.float16, device="cuda")
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
    # kq_gather_qmv, checked on the sampled columns
    ids0 = r.ids[0].astype(np.uint32)
    xd = np.repeat(W.activations(cfg.seed, cfg.tokens, cfg.k)[:1], cfg.top_k, axis=0)
    yd = torch.empty((cfg.top_k, cfg.n), dtype=torch.float16, device="cuda")
    kq.kq_gather_qmv(cfg.codec, wq, cfg.n_experts, cfg.n, cfg.k, dev(xd), u32(ids0), yd)
    refd = matmul.gather_qmv(cfg.codec, ref_bytes.reshape(cfg.n_experts, ns.size, rb), cfg.k, xd, ids0)
    errd = assert_close_rows(host(yd)[:, ns].astype(np.float64), refd, what="MoE decode gather_qmv")
    say(f"workload MoE decode gather_qmv (token 0, top-{cfg.top_k}): max row-normalized error {errd:.2e}")

    # decode GLU gather: these experts as gate, an up stack drawn the same way
    # (seed + 100), token 0's slots, silu
    wudev = dev(W.weight_rows(cfg.seed + 100, rows_w, cfg.k))
    wu = torch.empty((rows_w, rb), dtype=torch.uint8, device="cuda")
    kq.kq_quantize(cfg.codec, wudev, wu)
    del wudev
    x0 = W.activations(cfg.seed, cfg.tokens, cfg.k)[:1]
    yg = torch.empty((cfg.top_k, cfg.n), dtype=torch.float16, device="cuda")
    kq.kq_moe_glu_gather(cfg.codec, wq, wu, cfg.n_experts, cfg.n, cfg.k, dev(x0), u32(ids0[None, :]), yg, "silu")
    up_bytes = encode.quantize(cfg.codec, W.weight_rows(cfg.seed + 100, rows_w, cfg.k, rows=widx))
    assert np.array_equal(host(wu[torch.from_numpy(widx).cuda()]), up_bytes)
    refg = matmul.moe_glu_gather(cfg.codec, ref_bytes.reshape(cfg.n_experts, ns.size, rb),
                                 up_bytes.reshape(cfg.n_experts, ns.size, rb), cfg.k, x0, ids0[None, :], "silu")
    errg = assert_close_rows(host(yg)[:, ns].astype(np.float64), refg, what="MoE decode GLU gather")
    say(f"workload MoE decode GLU gather (token 0, top-{cfg.top_k}, silu): max row-normalized error {errg:.2e}")
    del wq, wu, y, yd, yg, mixed
    torch.cuda.empty_cache()


def _gpu_encode(kq, codec, seed, n, k, dist="normal"):
    import torch

    wdev = dev(W.weight_rows(seed, n, k, dist))
    wq = torch.empty((n, codecs.row_bytes(codec, k)), dtype=torch.uint8, device="cuda")
    kq.kq_quantize(codec, wdev, wq)
    del wdev
    return wq


def test_glu_prefill_workload(kq):
    # the GLU bench rows: q4_K gate (the GEMM workload's weights) and up (seed
    # + 100), 2048 x 14336 x 4096 and 16 x 14336 x 4096, float16 out, silu
    import torch

    c = W.CFG4_Q4K_GEMM
    say("workload GLU prefill: weights")
    wg = _gpu_encode(kq, c.codec, c.seed, c.n, c.k)
    wu = _gpu_encode(kq, c.codec, c.seed + 100, c.n, c.k)
    x = W.gemv_activations(c)
    y = torch.empty((c.m, c.n), dtype=torch.float16, device="cuda")
    say("workload GLU prefill: kernel")
    kq.kq_quantized_matmul_glu(c.codec, wg, wu, c.n, c.k, dev(x), y, "silu")
    ns = _sample(c.n, 32, 11)
    g_rows = encode.quantize(c.codec, W.weight_rows(c.seed, c.n, c.k, rows=ns))
    u_rows = encode.quantize(c.codec, W.weight_rows(c.seed + 100, c.n, c.k, rows=ns))
    assert np.array_equal(host(wg[torch.from_numpy(ns).cuda()]), g_rows)
    ref = matmul.quantized_matmul_glu(c.codec, g_rows, u_rows, c.k, x, "silu", "f16")
    g, u = matmul.qmatmul(c.codec, g_rows, c.k, x), matmul.qmatmul(c.codec, u_rows, c.k, x)
    assert_glu_close(host(y)[:, ns], ref, g, u, "silu", True, what="GLU prefill")
    # the small-batch GLU row: the first 16 activation rows (the wide
    # matrix-core GEMV's two passes)
    y16 = torch.empty((16, c.n), dtype=torch.float16, device="cuda")
    say("workload GLU batch 16: kernel")
    kq.kq_quantized_matmul_glu(c.codec, wg, wu, c.n, c.k, dev(x[:16]), y16, "silu")
    ref16 = matmul.quantized_matmul_glu(c.codec, g_rows, u_rows, c.k, x[:16], "silu", "f16")
    assert_glu_close(host(y16)[:, ns], ref16, g[:16], u[:16], "silu", True, what="GLU batch 16")
    del wg, wu, y, y16
    torch.cuda.empty_cache()


def test_residual_prefill_workload(kq):
    # the residual bench row: the q4_K down projection 4096 x 14336 (seed + 200)
    # over activations [2048, 14336] (seed + 200), residual [2048, 4096]
    # (seed + 201) updated in place, float16
    import torch

    c = W.CFG4_Q4K_GEMM
    n, k = c.k, c.n
    say("workload residual prefill: weights")
    wd = _gpu_encode(kq, c.codec, c.seed + 200, n, k)
    x = W.activations(c.seed + 200, c.m, k)
    res = W.activations(c.seed + 201, c.m, n)
    y = dev(res)
    say("workload residual prefill: kernel")
    kq.kq_quantized_matmul_residual(c.codec, wd, n, k, dev(x), y, y)
    ns = _sample(n, 32, 12)
    w_rows = encode.quantize(c.codec, W.weight_rows(c.seed + 200, n, k, rows=ns))
    ref = matmul.quantized_matmul_residual(c.codec, w_rows, k, x, res[:, ns])
    assert_close_rows(host(y)[:, ns].astype(np.float64), ref, what="residual prefill")
    del wd, y
    torch.cuda.empty_cache()


def test_small_prefill_workload(kq):
    # the small-prefill bench rows: the GEMM workload's q4_K 14336 x 4096 weight
    # with the first M of its activation rows through kq_quantized_matmul,
    # float16 out (16, 32 and 64 rows: the wide matrix-core GEMV on one, two
    # and four activation operands; 128: the GEMM)
    import torch

    c = W.CFG4_Q4K_GEMM
    say("workload small prefill: weights")
    wq = _gpu_encode(kq, c.codec, c.seed, c.n, c.k)
    ns = _sample(c.n, 32, 13)
    w_rows = encode.quantize(c.codec, W.weight_rows(c.seed, c.n, c.k, rows=ns))
    assert np.array_equal(host(wq[torch.from_numpy(ns).cuda()]), w_rows)
    xa = W.gemv_activations(c)
    for m in (16, 32, 64, 128):
        x = xa[:m]
        y = torch.empty((m, c.n), dtype=torch.float16, device="cuda")
        say(f"workload small prefill: M={m}")
        kq.kq_quantized_matmul(c.codec, wq, c.n, c.k, dev(x), y)
        ref = matmul.qmatmul(c.codec, w_rows, c.k, x)
        assert_close_rows(host(y)[:, ns].astype(np.float64), ref, what=f"small prefill M={m}")
    del wq, y
    torch.cuda.empty_cache()
