"""Oracle references at full workload sizes, computed in row chunks on a thread pool.

The oracle functions are plain NumPy; here they only run on slices of the
weight rows (the output columns), so a whole [M, N] reference of a
full-size workload takes seconds rather than minutes.  Nothing here changes
the oracle's arithmetic: every chunk is one call of the oracle function on
its rows, and the chunks are concatenated in order.  BLAS is held to one
thread inside the pool so the workers do not oversubscribe the host.
"""

from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
from threadpoolctl import threadpool_limits

from gguf_quant_matmul_amd import workloads as W
from oracle import codecs, encode, matmul

CHUNK = 1024
WORKERS = max(1, min(16, os.cpu_count() or 1))

_BYTES: dict = {}
_CACHE_LIMIT = 2 << 30  # bytes of cached wire bytes kept before the cache starts over


def _remember(key, value):
    if sum(v.nbytes for v in _BYTES.values()) + value.nbytes > _CACHE_LIMIT:
        _BYTES.clear()
    _BYTES[key] = value
    return value


def pmap_rows(fn, n, chunk=CHUNK):
    """[fn(a, b) for consecutive row ranges [a, b) of [0, n)], run on the pool."""
    starts = list(range(0, n, chunk))
    with threadpool_limits(1), cf.ThreadPoolExecutor(WORKERS) as ex:
        return list(ex.map(lambda a: fn(a, min(n, a + chunk)), starts))


def oracle_bytes(codec: str, seed: int, n: int, k: int, dist: str = "normal") -> np.ndarray:
    """The oracle encoder's wire bytes [n, row_bytes] of a workload's seeded weights (cached)."""
    key = (codec, seed, n, k, dist)
    if key not in _BYTES:
        parts = pmap_rows(lambda a, b: encode.quantize(codec, W.weight_rows(seed, n, k, dist, rows=np.arange(a, b))), n)
        return _remember(key, np.concatenate(parts))
    return _BYTES[key]


def random_bytes(codec: str, n: int, k: int, seed: int, scale: float = 0.02) -> np.ndarray:
    """Oracle-encoded N(0, scale) weights [n, row_bytes] from one seeded draw (cached)."""
    key = ("rand", codec, n, k, seed, scale)
    if key not in _BYTES:
        w = (np.random.default_rng(seed).standard_normal((n, k)) * scale).astype(np.float32)
        return _remember(key, np.concatenate(pmap_rows(lambda a, b: encode.quantize(codec, w[a:b]), n)))
    return _BYTES[key]


def clear() -> None:
    _BYTES.clear()


def qmatmul(codec: str, w: np.ndarray, k: int, x: np.ndarray) -> np.ndarray:
    """matmul.qmatmul over all of w's rows: [M, N] float64."""
    return np.concatenate(pmap_rows(lambda a, b: matmul.qmatmul(codec, w[a:b], k, x), w.shape[0]), axis=1)


def dequantize(codec: str, w: np.ndarray, k: int, dtype=np.float32) -> np.ndarray:
    return np.concatenate(pmap_rows(lambda a, b: codecs.dequantize(codec, w[a:b], k, dtype), w.shape[0]))


def residual(codec, w, k, x, res, gate=None):
    """matmul.quantized_matmul_residual over all output columns."""
    def one(a, b):
        g = None if gate is None else gate[..., a:b]
        return matmul.quantized_matmul_residual(codec, w[a:b], k, x, res[:, a:b], g)
    return np.concatenate(pmap_rows(one, w.shape[0]), axis=1)


def glu(codec, wg, wu, k, x, act, out):
    """matmul.quantized_matmul_glu plus the gate and up products, over all output columns."""
    def one(a, b):
        return (matmul.quantized_matmul_glu(codec, wg[a:b], wu[a:b], k, x, act, out),
                matmul.qmatmul(codec, wg[a:b], k, x), matmul.qmatmul(codec, wu[a:b], k, x))
    parts = pmap_rows(one, wg.shape[0])
    return tuple(np.concatenate([p[i] for p in parts], axis=1) for i in range(3))


def gather_qmm_seg(codec, w, k, x, tiles):
    """matmul.gather_qmm_seg over all output columns; w [E, N, row_bytes]."""
    return np.concatenate(pmap_rows(lambda a, b: matmul.gather_qmm_seg(codec, w[:, a:b], k, x, tiles), w.shape[1]),
                          axis=1)
