#!/usr/bin/env python3
"""Benchmark of the kq hot path on one MI355X: q4_K decode GEMV (kq_qmv) and
q4_K prefill GEMM (kq_qmm), plus every other row of the path measured once.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-rows] [--no-cpu]
    python bench.py --counters      # eager launches for rocprofv3 --pmc passes

One step = 64 back-to-back q4_K GEMVs (4096 x 4096, one activation row,
float32 out), each over its own weight copy (604 MB in all, so no copy is in
the 256 MB Infinity Cache when it is read), then one q4_K GEMM (M=2048,
N=14336, K=4096, float16 out).  Each is a HIP graph replayed on torch's
current stream; HIP events on that stream bracket each replay.

Prints ONE JSON line.  ``value`` is the GEMV's algorithmic HBM rate (wire
bytes + activations + outputs per launch / mean launch duration).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "q4_K qmv GB/s (% of HBM peak); q4_K qmm TFLOP/s (% of f16 MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16 MFMA, published
COLD_BYTES = 512 << 20         # rotate weight copies until this much is touched (> 256 MB MALL)
COPY_REF_BYTES = 256 << 20     # the elementwise copy that scales the HBM byte counters

# HBM bytes per launch from rocprofv3 counter passes over ``bench.py --counters``
# (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's reading for a
# copy of COPY_REF_BYTES).  A figure is reported only while the digest of the
# kernel's sources still matches the one the counters were taken on.
TRAFFIC = {
    "qmv": {"sources": ("kq_qmv.hip", "kq_qmv_impl.h", "kq_units.h", "kq_decode.h", "kq_internal.h"), "digest": "25b2875065d079cf",
            "bytes": 9587117},
    "qmm": {"sources": ("kq_qmm.hip", "kq_qmm_impl.h", "kq_internal.h", "kq_decode.h"), "digest": "fa8872933f2ea1fc", "bytes": 357213926},
}


def source_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gguf_quant_matmul_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic(kernel):
    t = TRAFFIC[kernel]
    if t["bytes"] is None or t["digest"] != source_digest(t["sources"]):
        return None
    return t["bytes"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--no-rows", action="store_true", help="skip the per-row measurements")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--counters", action="store_true",
                   help="no timing: eager launches of the copy reference, the 64 cold GEMVs and 2 GEMMs, "
                        "for rocprofv3 --pmc passes")
    p.add_argument("--digests", action="store_true", help="print the kernels' source digests and exit")
    return p.parse_args()


def capture(torch, fn):
    """A HIP graph of the launches fn() makes on the capture stream (no memsets inside)."""
    fn()  # eager run first (also warms the code objects)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# Untimed replays before any timing, in milliseconds of GPU work: the first
# ~25 ms of a heavy burst that follows host work run up to 45% slower while
# the device's clock and power control settles (per-replay traces of the
# lm-head GEMV dip from 80 to 118 us per launch and recover over ~35
# replays), so a timed window that starts cold measures the transient, not
# the kernel.
SETTLE_MS = 100.0


def settle(torch, graphs, min_ms=SETTLE_MS):
    """Replay the graphs in turn until at least min_ms of wall time has passed."""
    t0 = time.perf_counter()
    n = 0
    while n < 2 or (time.perf_counter() - t0) * 1e3 < min_ms:
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        n += 1


def time_graph(torch, g, launches, reps):
    """Mean milliseconds per launch over `reps` replays, HIP events around each
    replay, after the settle replays."""
    settle(torch, [g])
    evs = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        evs.append((s, e))
    torch.cuda.synchronize()
    return float(np.mean([s.elapsed_time(e) for s, e in evs])) / launches


def gpu_weights(torch, kq, codec, seed, n, k, dist):
    from gguf_quant_matmul_amd import workloads as W

    wf = torch.from_numpy(W.weight_rows(seed, n, k, dist)).cuda()
    wq = torch.empty((n, kq.kq_row_bytes(codec, k)), dtype=torch.uint8, device="cuda")
    kq.kq_quantize(codec, wf, wq)
    del wf
    return wq


def plain_read(torch, kq, ws, nl, groups=(256, 512, 1024, 2048, 4096, 8192)):
    """The plain-read reference: kq_stream_read over the same rotated weight
    copies, in the same graph-replay protocol as the GEMV it stands beside;
    the fastest of a few grid sizes."""
    nc, nb = len(ws), ws[0].numel()
    out = torch.empty((4 * max(groups),), dtype=torch.int32, device="cuda")
    best = None
    for gsz in groups:
        g = capture(torch, lambda: [kq.kq_stream_read(ws[i % nc], out[:4 * gsz]) for i in range(nl)])
        ms = time_graph(torch, g, nl, 5)
        if best is None or ms < best[0]:
            best = (ms, gsz)
    ms, gsz = best
    return {"row": "plain_read", "workload": f"plain read of {nb} B, {nc} rotating copies", "us": round(ms * 1e3, 2),
            "GB/s": round(nb / ms / 1e6, 1), "hbm_frac": round(nb / ms / 1e6 / HBM_PEAK_GBS, 3), "groups": gsz,
            "copies": nc}


def copies_for(nbytes):
    return max(1, min(64, math.ceil(COLD_BYTES / nbytes)))


def measure_rows(torch, kq):
    """Each remaining row of the path once, cold where the data would fit the MALL."""
    from gguf_quant_matmul_amd import workloads as W

    rows = []

    def gemv_row(cfg, reps=None, read_ref=False):
        wq = gpu_weights(torch, kq, cfg.codec, cfg.seed, cfg.n, cfg.k, cfg.dist)
        nb = wq.numel()
        nc = copies_for(nb)
        ws = [wq] + [wq.clone() for _ in range(nc - 1)]
        x = torch.from_numpy(W.gemv_activations(cfg)).cuda()
        y = torch.empty((cfg.m, cfg.n), dtype=torch.float32, device="cuda")
        nl = reps or max(nc, 8)
        g = capture(torch, lambda: [kq.kq_qmv(cfg.codec, ws[i % nc], cfg.n, cfg.k, x, y) for i in range(nl)])
        ms = time_graph(torch, g, nl, 5)
        alg = nb + x.numel() * 2 + y.numel() * 4
        gbs = alg / ms / 1e6
        row = {"row": "kq_qmv", "workload": cfg.name, "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
               "hbm_frac": round(gbs / HBM_PEAK_GBS, 3), "alg_bytes": alg, "copies": nc}
        if read_ref:
            rd = plain_read(torch, kq, ws, nl)
            row["read_us"] = rd["us"]
            row["of_read"] = round(rd["us"] / row["us"], 3)
            rows.append(dict(rd, workload=f"{rd['workload']} ({cfg.name} weights)"))
        rows.append(row)
        del ws, wq
        torch.cuda.empty_cache()

    for cfg in W.Q8_0_Q4_0_GEMVS:
        gemv_row(cfg, read_ref=cfg.m == 1)
    gemv_row(W.Q6K_LMHEAD_GEMV, reps=8, read_ref=True)

    # MoE: tile map + expert-segment GEMM
    cfg = W.MOE_SEG_Q4K
    wq = gpu_weights(torch, kq, cfg.codec, cfg.seed, cfg.n_experts * cfg.n, cfg.k, "normal")
    nc = copies_for(wq.numel())
    ws = [wq] + [wq.clone() for _ in range(nc - 1)]
    r = W.routing(cfg.seed, cfg.tokens, cfg.top_k, cfg.n_experts)
    x = torch.from_numpy(W.activations(cfg.seed, cfg.tokens, cfg.k)[r.token_of_row]).cuda()
    ids = torch.from_numpy(r.sorted_ids.view(np.int32)).cuda()
    cap = kq.kq_expert_tile_map_capacity(ids.numel(), cfg.n_experts)
    map_ = torch.empty((cap, 3), dtype=torch.int32, device="cuda")
    counts = torch.empty((1,), dtype=torch.int32, device="cuda")
    y = torch.empty((x.shape[0], cfg.n), dtype=torch.float16, device="cuda")
    nl = max(nc, 6)
    gm = capture(torch, lambda: [kq.kq_expert_tile_map(ids, cfg.n_experts, map_, counts) for _ in range(nl)])
    gs = capture(torch, lambda: [kq.kq_gather_qmm_seg(cfg.codec, ws[i % nc], cfg.n_experts, cfg.n, cfg.k, x, map_,
                                                      counts, y) for i in range(nl)])
    ms_map, ms_seg = time_graph(torch, gm, nl, 5), time_graph(torch, gs, nl, 5)
    alg = wq.numel() + x.numel() * 2 + y.numel() * 2
    flop = 2 * x.shape[0] * cfg.n * cfg.k
    rows.append({"row": "kq_expert_tile_map", "workload": cfg.name, "us": round(ms_map * 1e3, 2)})
    # the sorted rows back to token order, score-weighted (sorted-prefill MoE epilogue)
    inv = torch.from_numpy(r.inv_order.view(np.int32)).cuda()
    scores = torch.from_numpy(W.routing_scores(cfg.seed, cfg.tokens, cfg.top_k)).cuda()
    mixed = torch.empty((cfg.tokens, cfg.n), dtype=torch.float16, device="cuda")
    ymix = [torch.randn_like(y) for _ in range(copies_for(y.numel() * 2))]
    nmix = max(len(ymix), 16)
    gmx = capture(torch, lambda: [kq.kq_gather_mix(ymix[i % len(ymix)], inv, scores, mixed) for i in range(nmix)])
    ms_mix = time_graph(torch, gmx, nmix, 5)
    alg_mix = y.numel() * 2 + mixed.numel() * 2 + inv.numel() * 4 + scores.numel() * 4
    rows.append({"row": "kq_gather_mix", "workload": f"MoE unsort + score mix {cfg.tokens} tok x top-{cfg.top_k}, "
                 f"N={cfg.n} f16", "us": round(ms_mix * 1e3, 2), "GB/s": round(alg_mix / ms_mix / 1e6, 1),
                 "hbm_frac": round(alg_mix / ms_mix / 1e6 / HBM_PEAK_GBS, 3), "alg_bytes": alg_mix,
                 "copies": len(ymix)})
    del ymix
    rows.append({"row": "kq_gather_qmm_seg", "workload": cfg.name, "us": round(ms_seg * 1e3, 2),
                 "GB/s": round(alg / ms_seg / 1e6, 1), "hbm_frac": round(alg / ms_seg / 1e6 / HBM_PEAK_GBS, 3),
                 "TFLOP/s": round(flop / ms_seg / 1e9, 1),
                 "mfma_frac": round(flop / ms_seg / 1e9 / MFMA_F16_PEAK_TFLOPS, 3), "alg_bytes": alg, "copies": nc})
    # MoE decode: one token's top-8 routed rows through kq_gather_qmv on the same
    # expert weights; launch i takes token i's experts and weight copy i % nc
    nl = max(nc, 16)
    dec_ids = torch.from_numpy(np.ascontiguousarray(r.ids[:nl].astype(np.uint32)).view(np.int32)).cuda()
    xtok = W.activations(cfg.seed, nl, cfg.k)
    xd = [torch.from_numpy(np.repeat(xtok[i:i + 1], cfg.top_k, axis=0)).cuda() for i in range(nl)]
    yd = torch.empty((cfg.top_k, cfg.n), dtype=torch.float16, device="cuda")
    gd = capture(torch, lambda: [kq.kq_gather_qmv(cfg.codec, ws[i % nc], cfg.n_experts, cfg.n, cfg.k, xd[i],
                                                  dec_ids[i], yd) for i in range(nl)])
    ms_dec = time_graph(torch, gd, nl, 5)
    alg_dec = cfg.top_k * cfg.n * wq.shape[1] + cfg.top_k * cfg.k * 2 + cfg.top_k * cfg.n * 2
    rows.append({"row": "kq_gather_qmv", "workload": f"MoE decode gather_qmv 1 tok top-{cfg.top_k} of "
                 f"{cfg.n_experts} experts, {cfg.n}x{cfg.k} {cfg.codec}", "us": round(ms_dec * 1e3, 2),
                 "GB/s": round(alg_dec / ms_dec / 1e6, 1), "hbm_frac": round(alg_dec / ms_dec / 1e6 / HBM_PEAK_GBS, 3),
                 "alg_bytes": alg_dec, "copies": nc})
    # MoE decode GLU: the same token's slots through kq_moe_glu_gather, these
    # experts as gate and an up stack drawn the same way (seed + 100); launch i
    # takes token i's experts and copy i % nc of both stacks
    del xd
    wu = gpu_weights(torch, kq, cfg.codec, cfg.seed + 100, cfg.n_experts * cfg.n, cfg.k, "normal")
    wus = [wu] + [wu.clone() for _ in range(nc - 1)]
    xg = [torch.from_numpy(np.ascontiguousarray(xtok[i:i + 1])).cuda() for i in range(nl)]
    gids = dec_ids.view(nl, 1, cfg.top_k)
    gg = capture(torch, lambda: [kq.kq_moe_glu_gather(cfg.codec, ws[i % nc], wus[i % nc], cfg.n_experts, cfg.n,
                                                      cfg.k, xg[i], gids[i], yd, "silu") for i in range(nl)])
    ms_glu = time_graph(torch, gg, nl, 5)
    alg_glu = 2 * cfg.top_k * cfg.n * wq.shape[1] + cfg.k * 2 + cfg.top_k * cfg.n * 2
    rows.append({"row": "kq_moe_glu_gather", "workload": f"MoE decode GLU gather (silu) 1 tok top-{cfg.top_k} of "
                 f"{cfg.n_experts} experts, gate+up {cfg.n}x{cfg.k} {cfg.codec}", "us": round(ms_glu * 1e3, 2),
                 "GB/s": round(alg_glu / ms_glu / 1e6, 1), "hbm_frac": round(alg_glu / ms_glu / 1e6 / HBM_PEAK_GBS, 3),
                 "alg_bytes": alg_glu, "copies": nc})
    del ws, wq, wus, wu, xg
    torch.cuda.empty_cache()

    # dequantize (q4_K 4096 x 4096 -> float16)
    c1 = W.Q4K_DECODE_GEMV
    wq = gpu_weights(torch, kq, c1.codec, c1.seed, c1.n, c1.k, c1.dist)
    out = torch.empty((c1.n, c1.k), dtype=torch.float16, device="cuda")
    nc = copies_for(wq.numel() + out.numel() * 2)
    ws = [wq] + [wq.clone() for _ in range(nc - 1)]
    g = capture(torch, lambda: [kq.kq_dequantize(c1.codec, ws[i], c1.k, out) for i in range(nc)])
    ms = time_graph(torch, g, nc, 5)
    alg = wq.numel() + out.numel() * 2
    rows.append({"row": "kq_dequantize", "workload": "q4_K 4096x4096 -> f16", "us": round(ms * 1e3, 2),
                 "GB/s": round(alg / ms / 1e6, 1), "hbm_frac": round(alg / ms / 1e6 / HBM_PEAK_GBS, 3),
                 "alg_bytes": alg})
    del ws, wq, out
    torch.cuda.empty_cache()
    rows += epilogue_rows(torch, kq)
    rows += codec_rows(torch, kq)
    rows += bf16_rows(torch, kq)
    return rows


def bf16_rows(torch, kq):
    """bfloat16 activations on the q4_K decode GEMV (float32 out), the prefill
    GEMM and the MoE segment GEMM (bfloat16 out), same protocol as the float16
    rows."""
    from gguf_quant_matmul_amd import workloads as W

    out = []
    c1, c4, c5 = W.Q4K_DECODE_GEMV, W.Q4K_PREFILL_GEMM, W.MOE_SEG_Q4K
    w1 = gpu_weights(torch, kq, c1.codec, c1.seed, c1.n, c1.k, c1.dist)
    nc = copies_for(w1.numel())
    ws = [w1] + [w1.clone() for _ in range(nc - 1)]
    x = torch.from_numpy(W.activations_bf16(c1.seed, c1.m, c1.k)).cuda().to(torch.bfloat16)
    y = torch.empty((c1.m, c1.n), dtype=torch.float32, device="cuda")
    g = capture(torch, lambda: [kq.kq_qmv(c1.codec, ws[i], c1.n, c1.k, x, y) for i in range(nc)])
    ms = time_graph(torch, g, nc, 5)
    alg = w1.numel() + x.numel() * 2 + y.numel() * 4
    out.append({"row": "kq_qmv_bf16", "workload": f"{c1.name} M=1, bf16 x, f32 out", "us": round(ms * 1e3, 2),
                "GB/s": round(alg / ms / 1e6, 1), "hbm_frac": round(alg / ms / 1e6 / HBM_PEAK_GBS, 3),
                "alg_bytes": alg, "copies": nc})
    del ws, w1
    w4 = gpu_weights(torch, kq, c4.codec, c4.seed, c4.n, c4.k, c4.dist)
    x4 = torch.from_numpy(W.activations_bf16(c4.seed, c4.m, c4.k)).cuda().to(torch.bfloat16)
    y4 = torch.empty((c4.m, c4.n), dtype=torch.bfloat16, device="cuda")
    g = capture(torch, lambda: kq.kq_qmm(c4.codec, w4, c4.n, c4.k, x4, y4))
    ms = time_graph(torch, g, 1, 5)
    flop = 2 * c4.m * c4.n * c4.k
    out.append({"row": "kq_qmm_bf16", "workload": f"{c4.name}, bf16 x, bf16 out", "us": round(ms * 1e3, 2),
                "TFLOP/s": round(flop / ms / 1e9, 1), "mfma_frac": round(flop / ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 3)})
    del w4, x4, y4
    w5 = gpu_weights(torch, kq, c5.codec, c5.seed, c5.n_experts * c5.n, c5.k, "normal")
    nc = copies_for(w5.numel())
    ws = [w5] + [w5.clone() for _ in range(nc - 1)]
    r = W.routing(c5.seed, c5.tokens, c5.top_k, c5.n_experts)
    x5 = torch.from_numpy(W.activations_bf16(c5.seed, c5.tokens, c5.k)[r.token_of_row]).cuda().to(torch.bfloat16)
    ids = torch.from_numpy(r.sorted_ids.view(np.int32)).cuda()
    cap = kq.kq_expert_tile_map_capacity(ids.numel(), c5.n_experts)
    map_ = torch.empty((cap, 3), dtype=torch.int32, device="cuda")
    counts = torch.empty((1,), dtype=torch.int32, device="cuda")
    kq.kq_expert_tile_map(ids, c5.n_experts, map_, counts)
    y5 = torch.empty((x5.shape[0], c5.n), dtype=torch.bfloat16, device="cuda")
    nl = max(nc, 6)
    g = capture(torch, lambda: [kq.kq_gather_qmm_seg(c5.codec, ws[i % nc], c5.n_experts, c5.n, c5.k, x5, map_,
                                                     counts, y5) for i in range(nl)])
    ms = time_graph(torch, g, nl, 5)
    alg = w5.numel() + x5.numel() * 2 + y5.numel() * 2
    flop = 2 * x5.shape[0] * c5.n * c5.k
    out.append({"row": "kq_gather_qmm_seg_bf16", "workload": f"{c5.name}, bf16 x, bf16 out",
                "us": round(ms * 1e3, 2), "GB/s": round(alg / ms / 1e6, 1),
                "hbm_frac": round(alg / ms / 1e6 / HBM_PEAK_GBS, 3), "TFLOP/s": round(flop / ms / 1e9, 1),
                "mfma_frac": round(flop / ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 3), "alg_bytes": alg, "copies": nc})
    del ws, w5
    torch.cuda.empty_cache()
    return out


def cold_gemv_row(torch, kq, cfg):
    """One GEMV workload over rotated weight copies; returns (row, weights)."""
    from gguf_quant_matmul_amd import workloads as W

    wq = gpu_weights(torch, kq, cfg.codec, cfg.seed, cfg.n, cfg.k, cfg.dist)
    nb = wq.numel()
    nc = copies_for(nb)
    ws = [wq] + [wq.clone() for _ in range(nc - 1)]
    x = torch.from_numpy(W.gemv_activations(cfg)).cuda()
    y = torch.empty((cfg.m, cfg.n), dtype=torch.float32, device="cuda")
    nl = max(nc, 8)
    g = capture(torch, lambda: [kq.kq_qmv(cfg.codec, ws[i % nc], cfg.n, cfg.k, x, y) for i in range(nl)])
    ms = time_graph(torch, g, nl, 5)
    alg = nb + x.numel() * 2 + y.numel() * 4
    del ws
    return {"row": "kq_qmv", "workload": cfg.name, "us": round(ms * 1e3, 2), "GB/s": round(alg / ms / 1e6, 1),
            "hbm_frac": round(alg / ms / 1e6 / HBM_PEAK_GBS, 3), "alg_bytes": alg, "copies": nc}, wq


def codec_rows(torch, kq):
    """q5_K on the decode GEMV, prefill GEMM and MoE segment shapes; the legacy
    32-value codecs, q2_K and q3_K on the 14336x4096 GEMV; small prefill
    batches (M = 16, 64, 128) on the q4_K GEMM weight."""
    from gguf_quant_matmul_amd import workloads as W

    rows = []
    for cfg in W.LEGACY_GEMV + (W.Q2K_GEMV, W.Q3K_GEMV):
        r, _ = cold_gemv_row(torch, kq, cfg)
        rows.append(r)
    r, wq = cold_gemv_row(torch, kq, W.Q5K_GEMV)
    rows.append(r)
    # small prefill batches on the q4_K 14336 x 4096 weight (kq_quantized_matmul
    # routes M <= 16 to the GEMV, M <= 64 to the wide matrix-core GEMV, larger M
    # to the GEMM), weight copies rotated
    c4 = W.Q4K_PREFILL_GEMM
    w4 = gpu_weights(torch, kq, c4.codec, c4.seed, c4.n, c4.k, c4.dist)
    nc = copies_for(w4.numel())
    w4s = [w4] + [w4.clone() for _ in range(nc - 1)]
    xa = torch.from_numpy(W.gemv_activations(c4)).cuda()
    for m in (16, 32, 64, 128):
        ym = torch.empty((m, c4.n), dtype=torch.float16, device="cuda")
        xm = xa[:m]
        g = capture(torch, lambda: [kq.kq_quantized_matmul(c4.codec, w4s[i % nc], c4.n, c4.k, xm, ym) for i in range(nc)])
        ms = time_graph(torch, g, nc, 5)
        flop = 2 * m * c4.n * c4.k
        alg = w4.numel() + xm.numel() * 2 + ym.numel() * 2
        rows.append({"row": "kq_quantized_matmul", "workload": f"q4_K small prefill {m}x{c4.n}x{c4.k}, f16 out",
                     "us": round(ms * 1e3, 2), "GB/s": round(alg / ms / 1e6, 1),
                     "hbm_frac": round(alg / ms / 1e6 / HBM_PEAK_GBS, 3), "TFLOP/s": round(flop / ms / 1e9, 1),
                     "alg_bytes": alg, "copies": nc})
    del w4s, w4
    cfg = W.Q5K_GEMM
    xm = torch.from_numpy(W.gemv_activations(cfg)).cuda()
    ym = torch.empty((cfg.m, cfg.n), dtype=torch.float16, device="cuda")
    g = capture(torch, lambda: [kq.kq_qmm(cfg.codec, wq, cfg.n, cfg.k, xm, ym) for _ in range(3)])
    ms = time_graph(torch, g, 3, 5)
    flop = 2 * cfg.m * cfg.n * cfg.k
    rows.append({"row": "kq_qmm", "workload": cfg.name, "us": round(ms * 1e3, 2),
                 "TFLOP/s": round(flop / ms / 1e9, 1), "mfma_frac": round(flop / ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 3)})
    del wq, xm, ym
    # the MoE segment workload with q5_K experts
    c5 = W.MOE_SEG_Q4K
    we = gpu_weights(torch, kq, "q5_k", c5.seed, c5.n_experts * c5.n, c5.k, "normal")
    nc = copies_for(we.numel())
    wes = [we] + [we.clone() for _ in range(nc - 1)]
    r = W.routing(c5.seed, c5.tokens, c5.top_k, c5.n_experts)
    xs = torch.from_numpy(W.activations(c5.seed, c5.tokens, c5.k)[r.token_of_row]).cuda()
    ids = torch.from_numpy(r.sorted_ids.view(np.int32)).cuda()
    cap = kq.kq_expert_tile_map_capacity(ids.numel(), c5.n_experts)
    map_ = torch.empty((cap, 3), dtype=torch.int32, device="cuda")
    counts = torch.empty((1,), dtype=torch.int32, device="cuda")
    kq.kq_expert_tile_map(ids, c5.n_experts, map_, counts)
    ys = torch.empty((xs.shape[0], c5.n), dtype=torch.float16, device="cuda")
    nl = max(nc, 6)
    gs = capture(torch, lambda: [kq.kq_gather_qmm_seg("q5_k", wes[i % nc], c5.n_experts, c5.n, c5.k, xs, map_,
                                                      counts, ys) for i in range(nl)])
    ms = time_graph(torch, gs, nl, 5)
    alg = we.numel() + xs.numel() * 2 + ys.numel() * 2
    flop = 2 * xs.shape[0] * c5.n * c5.k
    rows.append({"row": "kq_gather_qmm_seg", "workload": c5.name.replace("MoE", "q5_K MoE"),
                 "us": round(ms * 1e3, 2), "GB/s": round(alg / ms / 1e6, 1),
                 "hbm_frac": round(alg / ms / 1e6 / HBM_PEAK_GBS, 3), "TFLOP/s": round(flop / ms / 1e9, 1),
                 "mfma_frac": round(flop / ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 3), "alg_bytes": alg, "copies": nc})
    del wes, we
    torch.cuda.empty_cache()
    return rows


def epilogue_rows(torch, kq):
    """The fused epilogues on a transformer block's shapes (Llama-3-8B FFN: gate/up 14336x4096, down 4096x14336),
    prefill (2048 rows, float16 out) and decode (one row, float32 out), each beside the plain matmul of the same
    weight so the epilogue's cost shows."""
    from gguf_quant_matmul_amd import workloads as W

    rows = []
    c4 = W.Q4K_PREFILL_GEMM
    m_pf, k_ffn, n_ffn = c4.m, c4.k, c4.n

    def row(name, workload, fused, plain, nl, flop, alg, extra=None):
        gf, gp = capture(torch, lambda: [fused(i) for i in range(nl)]), capture(torch, lambda: [plain(i) for i in range(nl)])
        ms_f, ms_p = time_graph(torch, gf, nl, 5), time_graph(torch, gp, nl, 5)
        r = {"row": name, "workload": workload, "us": round(ms_f * 1e3, 2), "us_plain_matmul": round(ms_p * 1e3, 2),
             "GB/s": round(alg / ms_f / 1e6, 1), "hbm_frac": round(alg / ms_f / 1e6 / HBM_PEAK_GBS, 3), "alg_bytes": alg}
        if flop:
            r["TFLOP/s"] = round(flop / ms_f / 1e9, 1)
            r["mfma_frac"] = round(flop / ms_f / 1e9 / MFMA_F16_PEAK_TFLOPS, 3)
        rows.append(r)

    # GLU: gate = the q4_K prefill weight, up drawn the same way (seed + 100)
    wg = gpu_weights(torch, kq, c4.codec, c4.seed, n_ffn, k_ffn, c4.dist)
    wu = gpu_weights(torch, kq, c4.codec, c4.seed + 100, n_ffn, k_ffn, c4.dist)
    nb = wg.numel()
    xp = torch.from_numpy(W.gemv_activations(c4)).cuda()
    yp = torch.empty((m_pf, n_ffn), dtype=torch.float16, device="cuda")
    row("kq_quantized_matmul_glu", f"q4_K GLU (silu) prefill {m_pf}x{n_ffn}x{k_ffn}, gate+up, f16 out",
        lambda i: kq.kq_quantized_matmul_glu(c4.codec, wg, wu, n_ffn, k_ffn, xp, yp, "silu"),
        lambda i: kq.kq_quantized_matmul(c4.codec, wg, n_ffn, k_ffn, xp, yp), 3,
        2 * 2 * m_pf * n_ffn * k_ffn, 2 * nb + xp.numel() * 2 + yp.numel() * 2)
    # decode: rotate weight copies so each launch reads from HBM
    nc = copies_for(2 * nb)
    wgs, wus = [wg] + [wg.clone() for _ in range(nc - 1)], [wu] + [wu.clone() for _ in range(nc - 1)]
    x1 = xp[:1].clone()
    y1 = torch.empty((1, n_ffn), dtype=torch.float32, device="cuda")
    nl = max(nc, 8)
    row("kq_quantized_matmul_glu", f"q4_K GLU (silu) decode 1x{n_ffn}x{k_ffn}, gate+up, f32 out",
        lambda i: kq.kq_quantized_matmul_glu(c4.codec, wgs[i % nc], wus[i % nc], n_ffn, k_ffn, x1, y1, "silu"),
        lambda i: kq.kq_quantized_matmul(c4.codec, wgs[i % nc], n_ffn, k_ffn, x1, y1), nl,
        0, 2 * nb + k_ffn * 2 + n_ffn * 4)
    # a small decode batch: the two passes of the wide matrix-core GEMV
    x16 = xp[:16].clone()
    y16 = torch.empty((16, n_ffn), dtype=torch.float16, device="cuda")
    row("kq_quantized_matmul_glu", f"q4_K GLU (silu) batch 16x{n_ffn}x{k_ffn}, gate+up, f16 out",
        lambda i: kq.kq_quantized_matmul_glu(c4.codec, wgs[i % nc], wus[i % nc], n_ffn, k_ffn, x16, y16, "silu"),
        lambda i: kq.kq_quantized_matmul(c4.codec, wgs[i % nc], n_ffn, k_ffn, x16, y16), nl,
        2 * 2 * 16 * n_ffn * k_ffn, 2 * nb + x16.numel() * 2 + y16.numel() * 2)
    del wgs, wus, wg, wu, yp
    torch.cuda.empty_cache()

    # residual: the down projection 4096x14336 with the residual stream updated in place
    wd = gpu_weights(torch, kq, c4.codec, c4.seed + 200, k_ffn, n_ffn, c4.dist)
    nb = wd.numel()
    xd = torch.from_numpy(W.activations(c4.seed + 200, m_pf, n_ffn)).cuda()
    res = torch.from_numpy(W.activations(c4.seed + 201, m_pf, k_ffn)).cuda()
    row("kq_quantized_matmul_residual", f"q4_K down proj + residual prefill {m_pf}x{k_ffn}x{n_ffn}, f16 in place",
        lambda i: kq.kq_quantized_matmul_residual(c4.codec, wd, k_ffn, n_ffn, xd, res, res),
        lambda i: kq.kq_quantized_matmul(c4.codec, wd, k_ffn, n_ffn, xd, res), 3,
        2 * m_pf * k_ffn * n_ffn, nb + xd.numel() * 2 + 2 * res.numel() * 2)
    nc = copies_for(nb)
    wds = [wd] + [wd.clone() for _ in range(nc - 1)]
    x1 = xd[:1].clone()
    r1 = torch.zeros((1, k_ffn), dtype=torch.float32, device="cuda")
    nl = max(nc, 8)
    row("kq_quantized_matmul_residual", f"q4_K down proj + residual decode 1x{k_ffn}x{n_ffn}, f32 in place",
        lambda i: kq.kq_quantized_matmul_residual(c4.codec, wds[i % nc], k_ffn, n_ffn, x1, r1, r1),
        lambda i: kq.kq_quantized_matmul(c4.codec, wds[i % nc], k_ffn, n_ffn, x1, r1), nl,
        0, nb + n_ffn * 2 + 2 * k_ffn * 4)
    del wds, wd, xd, res
    torch.cuda.empty_cache()

    # bias: q8_0 14336x4096, one row
    c2 = W.Q8_0_Q4_0_GEMVS[0]
    wq = gpu_weights(torch, kq, c2.codec, c2.seed, c2.n, c2.k, c2.dist)
    nb = wq.numel()
    nc = copies_for(nb)
    ws = [wq] + [wq.clone() for _ in range(nc - 1)]
    x1 = torch.from_numpy(W.gemv_activations(c2)).cuda()
    bias = torch.from_numpy(np.random.default_rng(c2.seed).standard_normal(c2.n).astype(np.float32)).cuda()
    y1 = torch.empty((1, c2.n), dtype=torch.float32, device="cuda")
    nl = max(nc, 8)
    row("kq_quantized_matmul_qmv_bias", f"q8_0 GEMV + bias 1x{c2.n}x{c2.k}, f32 out",
        lambda i: kq.kq_quantized_matmul_qmv_bias(c2.codec, ws[i % nc], c2.n, c2.k, x1, bias, y1),
        lambda i: kq.kq_quantized_matmul(c2.codec, ws[i % nc], c2.n, c2.k, x1, y1), nl,
        0, nb + c2.k * 2 + 2 * c2.n * 4)
    del ws, wq
    torch.cuda.empty_cache()
    return rows


def counters_pass(torch, kq, w1s, x1, y1, w4, x4, y4):
    """Eager launches for hardware-counter passes.  First a plain elementwise
    copy (torch.neg) of COPY_REF_BYTES four times: it reads and writes exactly
    that many bytes, which calibrates FETCH_SIZE and WRITE_SIZE.  Then the
    timed workloads as the timed region runs them (one GEMV per cold weight
    copy, two GEMMs), and after them two launches each of the q8_0 and q4_0
    GEMVs at M = 8, one q6_K lm-head GEMV and two MoE tile maps and segment
    GEMMs, so one pass covers every HBM- and MFMA-bound row."""
    from gguf_quant_matmul_amd import workloads as W

    c1, c4 = W.Q4K_DECODE_GEMV, W.Q4K_PREFILL_GEMM
    src = torch.ones(COPY_REF_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    for w in w1s:
        kq.kq_qmv(c1.codec, w, c1.n, c1.k, x1, y1)
    for _ in range(2):
        kq.kq_qmm(c4.codec, w4, c4.n, c4.k, x4, y4)
    torch.cuda.synchronize()
    launched = {"copy": 4, "qmv q4_K 4096x4096 M=1": len(w1s), "qmm q4_K 2048x14336x4096": 2}

    for cfg in W.Q8_0_Q4_0_GEMVS:
        if cfg.m != 8:
            continue
        w = gpu_weights(torch, kq, cfg.codec, cfg.seed, cfg.n, cfg.k, cfg.dist)
        x = torch.from_numpy(W.gemv_activations(cfg)).cuda()
        y = torch.empty((cfg.m, cfg.n), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        for _ in range(2):
            kq.kq_qmv(cfg.codec, w, cfg.n, cfg.k, x, y)
        torch.cuda.synchronize()
        launched[f"qmv {cfg.codec} {cfg.n}x{cfg.k} M=8"] = 2
        del w
    c3 = W.Q6K_LMHEAD_GEMV
    w = gpu_weights(torch, kq, c3.codec, c3.seed, c3.n, c3.k, c3.dist)
    x = torch.from_numpy(W.gemv_activations(c3)).cuda()
    y = torch.empty((c3.m, c3.n), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    kq.kq_qmv(c3.codec, w, c3.n, c3.k, x, y)
    torch.cuda.synchronize()
    launched["qmv q6_K 128256x4096 M=1"] = 1
    del w
    torch.cuda.empty_cache()

    c5 = W.MOE_SEG_Q4K
    w = gpu_weights(torch, kq, c5.codec, c5.seed, c5.n_experts * c5.n, c5.k, "normal")
    r = W.routing(c5.seed, c5.tokens, c5.top_k, c5.n_experts)
    x = torch.from_numpy(W.activations(c5.seed, c5.tokens, c5.k)[r.token_of_row]).cuda()
    ids = torch.from_numpy(r.sorted_ids.view(np.int32)).cuda()
    cap = kq.kq_expert_tile_map_capacity(ids.numel(), c5.n_experts)
    map_ = torch.empty((cap, 3), dtype=torch.int32, device="cuda")
    counts = torch.empty((1,), dtype=torch.int32, device="cuda")
    y = torch.empty((x.shape[0], c5.n), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    for _ in range(2):
        kq.kq_expert_tile_map(ids, c5.n_experts, map_, counts)
        kq.kq_gather_qmm_seg(c5.codec, w, c5.n_experts, c5.n, c5.k, x, map_, counts, y)
    torch.cuda.synchronize()
    launched["tile map + seg q4_K MoE 512 tok top-8"] = 2
    return {"mode": "counters", "copy_ref_bytes": COPY_REF_BYTES, "launches": launched}


def cpu_baseline():
    """The oracle as it stands, timed on this host on a bounded sample of each of
    the five workloads: NumPy decode (single-threaded) and the float64 matmul
    (BLAS threads) timed separately, the lm-head in a 1024-row chunk of N."""
    from gguf_quant_matmul_amd import workloads as W
    from oracle import codecs, encode, matmul

    try:
        from threadpoolctl import threadpool_info

        blas = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        blas = 1

    def timed(fn, budget=1.5):
        reps, t0 = 0, time.perf_counter()
        while reps < 2 or time.perf_counter() - t0 < budget:
            r = fn()
            reps += 1
        return (time.perf_counter() - t0) / reps, r

    def one(name, codec, seed, n_full, k, dist, rows, x, flop_rate, unit):
        wq = encode.quantize(codec, W.weight_rows(seed, n_full, k, dist, rows=np.arange(rows)))
        t_dec, wd = timed(lambda: codecs.dequantize(codec, wq, k, np.float32))
        t_mm, _ = timed(lambda: matmul.matmul_f64(x, wd))
        tot = t_dec + t_mm
        if flop_rate:
            val = 2 * x.shape[0] * rows * k / tot / 1e12
        else:
            val = (wq.nbytes + x.size * 2 + x.shape[0] * rows * 4) / tot / 1e9
        return {"workload": name, "sample": f"{rows} of {n_full} weight rows x {x.shape[0]} activation rows",
                "decode_ms": round(t_dec * 1e3, 2), "matmul_ms": round(t_mm * 1e3, 2),
                "value": round(val, 5 if flop_rate else 3), "unit": unit}

    c1, c3, c4, c5 = W.Q4K_DECODE_GEMV, W.Q6K_LMHEAD_GEMV, W.Q4K_PREFILL_GEMM, W.MOE_SEG_Q4K
    cfgs = [one(c1.name, c1.codec, c1.seed, c1.n, c1.k, c1.dist, 1024, W.gemv_activations(c1), False, "GB/s")]
    for c in W.Q8_0_Q4_0_GEMVS:
        if c.m in (1, 8):
            cfgs.append(one(c.name, c.codec, c.seed, c.n, c.k, c.dist, 1024, W.gemv_activations(c), False, "GB/s"))
    cfgs.append(one(c3.name, c3.codec, c3.seed, c3.n, c3.k, c3.dist, 1024, W.gemv_activations(c3), False, "GB/s"))
    cfgs.append(one(c4.name, c4.codec, c4.seed, c4.n, c4.k, c4.dist, 128, W.gemv_activations(c4), True, "TFLOP/s"))
    # MoE segment GEMM: the first expert's first 256 weight rows times its routed rows
    r = W.routing(c5.seed, c5.tokens, c5.top_k, c5.n_experts)
    xs = W.activations(c5.seed, c5.tokens, c5.k)[r.token_of_row][r.sorted_ids == 0]
    cfgs.append(one(c5.name, c5.codec, c5.seed, c5.n_experts * c5.n, c5.k, "normal", 256, xs, True, "TFLOP/s"))
    head = cfgs[0]
    return {
        "value": head["value"], "unit": "GB/s", "cores": int(max(blas, 1)), "kind": "oracle",
        "sample": f"q4_K GEMV on 1024 of 4096 weight rows (K=4096, M=1): NumPy decode {head['decode_ms']} ms "
                  f"(single-threaded) + float64 matmul {head['matmul_ms']} ms (BLAS, {blas} threads)",
        "configs": cfgs,
        "host_cpus": os.cpu_count(),
    }


def main():
    args = parse()
    if args.digests:
        print(json.dumps({k: source_digest(v["sources"]) for k, v in TRAFFIC.items()}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the kq path is a single-GPU kernel library "
              "(its multi-GPU sharding is a design note, not built).", file=sys.stderr)
        sys.exit(2)

    import torch

    from gguf_quant_matmul_amd import kq
    from gguf_quant_matmul_amd import workloads as W

    assert torch.cuda.is_available(), "needs a GPU"
    dev_name = torch.cuda.get_device_properties(0).name
    log(f"device: {dev_name}")

    c1, c4 = W.Q4K_DECODE_GEMV, W.Q4K_PREFILL_GEMM
    log("preparing inputs (weights drawn on the host, encoded on the GPU by kq_quantize)")
    w1 = gpu_weights(torch, kq, c1.codec, c1.seed, c1.n, c1.k, c1.dist)
    n_cold = 64
    w1s = [w1] + [w1.clone() for _ in range(n_cold - 1)]
    x1 = torch.from_numpy(W.gemv_activations(c1)).cuda()
    y1 = torch.empty((1, c1.n), dtype=torch.float32, device="cuda")
    w4 = gpu_weights(torch, kq, c4.codec, c4.seed, c4.n, c4.k, c4.dist)
    x4 = torch.from_numpy(W.gemv_activations(c4)).cuda()
    y4 = torch.empty((c4.m, c4.n), dtype=torch.float16, device="cuda")

    alg1 = w1.numel() + x1.numel() * 2 + y1.numel() * 4           # 9,461,760 B
    flop4 = 2 * c4.m * c4.n * c4.k                                 # 240,518,168,576
    alg4 = w4.numel() + x4.numel() * 2 + y4.numel() * 2
    if args.counters:
        print(json.dumps(counters_pass(torch, kq, w1s, x1, y1, w4, x4, y4)), flush=True)
        return

    # One step: the 64 cold GEMVs (one HIP graph) and one GEMM (one HIP graph).
    g1 = capture(torch, lambda: [kq.kq_qmv(c1.codec, w1s[i], c1.n, c1.k, x1, y1) for i in range(n_cold)])
    g4 = capture(torch, lambda: kq.kq_qmm(c4.codec, w4, c4.n, c4.k, x4, y4))
    settle(torch, [g1, g4])  # device clocks to their steady state; then the W warmup steps
    for _ in range(args.warmup):
        g1.replay()
        g4.replay()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        g1.replay()
        ev[i][1].record()
        g4.replay()
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per1 = np.array([a.elapsed_time(b) for a, b, _ in ev]) / n_cold  # per-launch ms, one value per step
    per4 = np.array([b.elapsed_time(c) for _, b, c in ev])
    ms1, ms4 = float(per1.mean()), float(per4.mean())
    stream_ms = ms1

    gbs = alg1 / ms1 / 1e6
    tflops = flop4 / ms4 / 1e9
    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; weights drawn on the host, q4_K-encoded on the GPU)",
        "config": {
            "workload": "q4_K decode GEMV N=4096 K=4096 M=1 f32-out, cold (64 rotating weight copies); "
                        "q4_K prefill GEMM M=2048 N=14336 K=4096 f16-out",
            "global_batch": 1,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic("qmv"),
            "kernel": "kq_qmv q4_K (qmv_stage_kernel<q4_K, M=1>)", "alg_bytes_per_launch": alg1,
            "mean_launch_us": round(ms1 * 1e3, 3),
            "median_launch_us": round(float(np.median(per1)) * 1e3, 3),
            "p90_launch_us": round(float(np.percentile(per1, 90)) * 1e3, 3),
        },
        "qmm": {
            "value": round(tflops, 1), "unit": "TFLOP/s", "mean_launch_us": round(ms4 * 1e3, 2),
            "median_launch_us": round(float(np.median(per4)) * 1e3, 2),
            "p90_launch_us": round(float(np.percentile(per4, 90)) * 1e3, 2),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic("qmm"),
                         "kernel": "kq_qmm q4_K (qmm_kernel<q4_K, 256, 224>)", "alg_flop_per_launch": flop4,
                         "alg_bytes_per_launch": alg4},
        },
        "timing": "HIP graphs: one replay = 64 GEMVs over distinct cold weight copies (back to back on one "
                  "stream), one replay = one GEMM; 100 ms of untimed settle replays (device clocks to steady "
                  "state), then the warmup steps; HIP events around each replay; per-launch time = replay "
                  "time / launches (includes the GPU-side gap between consecutive kernels); mean, median and "
                  "p90 over the timed steps",
        "device": dev_name,
    }
    # the plain-read ceiling of the GEMV's weight stream, same protocol
    rd = plain_read(torch, kq, w1s, n_cold)
    out["roofline"]["read_ceiling"] = {"us": rd["us"], "GB/s": rd["GB/s"], "groups": rd["groups"],
                                       "gemv_over_read": round(ms1 * 1e3 / rd["us"], 3)}
    # the launch floor of that protocol: the same graph of back-to-back launches
    # of a near-empty kernel (one workgroup reading 16 bytes)
    tiny = torch.zeros((16,), dtype=torch.uint8, device="cuda")
    tout = torch.empty((4,), dtype=torch.int32, device="cuda")
    gl = capture(torch, lambda: [kq.kq_stream_read(tiny, tout) for _ in range(n_cold)])
    out["roofline"]["launch_floor_us"] = round(time_graph(torch, gl, n_cold, 5) * 1e3, 2)
    del gl, tiny, tout
    del w1s, w1, w4, x4, y4
    torch.cuda.empty_cache()
    if not args.no_rows:
        log("measuring the other rows")
        out["rows"] = [dict(rd, workload=f"{rd['workload']} (the q4_K decode GEMV's weights)")] + measure_rows(torch, kq)
    if not args.no_cpu:
        log("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
