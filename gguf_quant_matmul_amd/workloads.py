"""Seeded synthetic inputs for the five workloads (CPU, NumPy).

This module holds no arithmetic of the method: it draws float weights,
float16 activations and MoE routing, nothing else.  Both the tests (which feed
the oracle) and the benchmark (which feeds the HIP path) take their inputs
from here.

Recipe (each tensor from its own counter-keyed NumPy stream, so draw order
never matters):
  * weights: row chunks of 256 rows; chunk c of tensor seed s comes from
    ``numpy.random.default_rng([s, 0, c])``; N(0, 0.02) or Student-t(5)*0.02,
    float32.  A row's values can be regenerated alone (its chunk only).
  * activations: ``default_rng([s, 1])``, N(0, 1) float32, rounded to float16
    (RNE).
  * routing: ``default_rng([s, 2])``; per token ``rng.choice(E, top_k,
    replace=False)``; the (token, slot) pairs are ordered by a STABLE sort on
    expert id, so ties keep (token, slot) order.
  * routing scores: ``default_rng([s, 3])``, Exponential(1) per (token, slot),
    each token's normalized to sum 1 (like top-k softmax weights), float32.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
from dataclasses import dataclass

import numpy as np

ROW_CHUNK = 256


def weight_rows(seed: int, n: int, k: int, dist: str = "normal", rows=None) -> np.ndarray:
    """Float32 weights [n, k] (or only ``rows``, an iterable of row indices)."""
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows, dtype=np.int64)
    if dist not in ("normal", "t5"):
        raise ValueError(dist)
    out = np.empty((rows.size, k), dtype=np.float32)
    chunks = np.unique(rows // ROW_CHUNK)
    contiguous = rows.size == n and np.array_equal(rows, np.arange(n))

    def one(c):
        lo = int(c) * ROW_CHUNK
        cnt = min(ROW_CHUNK, n - lo)
        rng = np.random.default_rng([seed, 0, int(c)])
        if dist == "normal":
            blk = rng.standard_normal((cnt, k), dtype=np.float32) * np.float32(0.02)
        else:
            blk = (rng.standard_t(5, (cnt, k)) * 0.02).astype(np.float32)
        if contiguous:
            out[lo:lo + cnt] = blk
        else:
            sel = np.nonzero(rows // ROW_CHUNK == c)[0]
            out[sel] = blk[rows[sel] - lo]

    # chunks are independent streams: draw them on a few threads
    workers = min(16, os.cpu_count() or 1, len(chunks))
    if workers > 1:
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, chunks))
    else:
        for c in chunks:
            one(c)
    return out


def activations(seed: int, m: int, k: int) -> np.ndarray:
    """Float16 activations [m, k]: N(0,1) float32 rounded to float16."""
    rng = np.random.default_rng([seed, 1])
    return rng.standard_normal((m, k), dtype=np.float32).astype(np.float16)


def to_bf16(a: np.ndarray) -> np.ndarray:
    """Finite float32 values rounded to the nearest bfloat16 (ties to even),
    returned as float32 holding bfloat16 values (NumPy has no bfloat16)."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def activations_bf16(seed: int, m: int, k: int) -> np.ndarray:
    """Bfloat16 activations [m, k] (as float32 values): the same N(0,1) draw
    as ``activations``, rounded to bfloat16."""
    rng = np.random.default_rng([seed, 1])
    return to_bf16(rng.standard_normal((m, k), dtype=np.float32))


@dataclass
class Routing:
    tokens: int
    top_k: int
    n_experts: int
    ids: np.ndarray          # [tokens, top_k] expert id per (token, slot)
    order: np.ndarray        # [tokens*top_k] flat (token*top_k + slot) of each sorted row
    sorted_ids: np.ndarray   # [tokens*top_k] uint32 expert id of each sorted row

    @property
    def token_of_row(self) -> np.ndarray:
        return self.order // self.top_k

    @property
    def inv_order(self) -> np.ndarray:
        """[tokens*top_k] uint32: the sorted row of each flat (token*top_k + slot)."""
        inv = np.empty(self.order.size, dtype=np.uint32)
        inv[self.order] = np.arange(self.order.size, dtype=np.uint32)
        return inv


def routing_scores(seed: int, tokens: int, top_k: int) -> np.ndarray:
    """[tokens, top_k] float32 routing weights: positive, each token's summing to 1."""
    rng = np.random.default_rng([seed, 3])
    s = rng.exponential(1.0, (tokens, top_k))
    return (s / s.sum(axis=1, keepdims=True)).astype(np.float32)


def routing(seed: int, tokens: int, top_k: int, n_experts: int) -> Routing:
    rng = np.random.default_rng([seed, 2])
    ids = np.stack([rng.choice(n_experts, top_k, replace=False) for _ in range(tokens)]).astype(np.int64)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    return Routing(tokens, top_k, n_experts, ids, order, flat[order].astype(np.uint32))


# ---------------------------------------------------------------------------
# The five workloads (shapes and distributions as stated for each).
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class GemvConfig:
    name: str
    codec: str
    n: int
    k: int
    m: int
    seed: int
    dist: str
    out_dtype: str  # "f32" or "f16"


Q4K_DECODE_GEMV = GemvConfig("q4_K decode GEMV 4096x4096", "q4_k", 4096, 4096, 1, 0, "normal", "f32")
Q8_0_Q4_0_GEMVS = tuple(
    GemvConfig(f"{c} GEMV 14336x4096 M={m}", c, 14336, 4096, m, 1, "normal", "f32")
    for c in ("q8_0", "q4_0") for m in (1, 2, 4, 8)
)
Q6K_LMHEAD_GEMV = GemvConfig("q6_K lm-head GEMV 128256x4096", "q6_k", 128256, 4096, 1, 2, "t5", "f32")
Q4K_PREFILL_GEMM = GemvConfig("q4_K prefill GEMM 2048x14336x4096", "q4_k", 14336, 4096, 2048, 3, "normal", "f16")


# q5_K on the q4_K decode and prefill shapes (a widening of the codec set; seed 5)
Q5K_GEMV = GemvConfig("q5_K GEMV 14336x4096 M=1", "q5_k", 14336, 4096, 1, 5, "normal", "f32")
Q5K_GEMM = GemvConfig("q5_K prefill GEMM 2048x14336x4096", "q5_k", 14336, 4096, 2048, 5, "normal", "f16")
# q2_K and q3_K on the same GEMV shape (seeds 7, 8)
Q2K_GEMV = GemvConfig("q2_K GEMV 14336x4096 M=1", "q2_k", 14336, 4096, 1, 7, "normal", "f32")
Q3K_GEMV = GemvConfig("q3_K GEMV 14336x4096 M=1", "q3_k", 14336, 4096, 1, 8, "normal", "f32")
# the legacy 32-value codecs on the q8_0 / q4_0 GEMV shape (seed 6)
LEGACY_GEMV = tuple(GemvConfig(f"{c} GEMV 14336x4096 M=1", c, 14336, 4096, 1, 6, "normal", "f32")
                    for c in ("q4_1", "q5_0", "q5_1"))


@dataclass(frozen=True)
class MoeConfig:
    name: str
    codec: str
    n_experts: int
    n: int
    k: int
    tokens: int
    top_k: int
    seed: int
    out_dtype: str


MOE_SEG_Q4K = MoeConfig("MoE gather_qmm_seg 512 tok top-8 of 64 experts, 1536x4096", "q4_k", 64, 1536, 4096, 512, 8, 4, "f16")


def gemv_activations(cfg: GemvConfig) -> np.ndarray:
    """x for a GEMV/GEMM workload.  The q8_0/q4_0 workload draws [8, K] once and uses the first M rows."""
    if cfg.seed == 1:
        return activations(cfg.seed, 8, cfg.k)[: cfg.m]
    return activations(cfg.seed, cfg.m, cfg.k)
