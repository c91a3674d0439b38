"""Oracle: quantized matmul, expert tile map and expert-sorted gather (CPU, NumPy).

Test infrastructure only (see ``oracle/__init__``).

Definitions followed
  * mlx-kquant ``bindings.cpp`` page, ``quantized_matmul`` docstring: the
    result is ``x @ dequant(w)`` with ``w`` laid out [N, K] (transpose=True);
    nuvec-core ``quantized.rs`` page, ``quantized_matmul``: ``x`` times the
    transposed dequantized weight.  Here: ``y[m, n] = sum_k x[m, k] * W[n, k]``
    with W the exact dequantized values, accumulated in float64.  Both
    operands are exact in float64 (x is fp16, W is an fp32 number), so the
    only error is float64 accumulation.
  * mlx-kquant ``bindings.cpp`` page, ``expert_tile_map`` docstring: from
    expert ids sorted ascending, tile each expert's segment into 64-row tiles
    (expert, row_start, num_rows); only the last tile of a segment may be
    partial; a count of valid tiles.  Tile order is unspecified there; this
    oracle emits expert-major, ascending row_start.
  * mlx-kquant ``bindings.cpp`` page, ``gather_qmv_kq`` docstring: one
    activation row per expert slot; row r times expert ``indices[r]``.
  * mlx-kquant ``bindings.cpp`` page, ``moe_glu_gather_kq`` docstring: the
    gate and up expert products of one token's activation row, combined by
    the GLU epilogue act(g) * u.  act 'silu': silu(g) * u; 'gelu' (its tanh
    approximation): gelu(g) * u; 'silu_limit': silu(min(g, limit)) *
    clip(u, -limit, limit).  silu(v) = v * sigmoid(v) = v / (1 + exp(-v));
    the tanh form of gelu is 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))
    (the standard tanh approximation; the page names it, not its formula).
    Output [T, R, N], slot (t, r) using expert indices[t, r].
  * mlx-kquant ``bindings.cpp`` page, ``gather_mix`` docstring: after a
    sorted-prefill MoE, out[t] = sum_s scores[t, s] * y[inv_order[t*k + s]]
    (unsort, score multiply and sum over slots).  Reading taken: a slot whose
    inv_order entry is not below the row count adds nothing.
  * mlx-kquant ``bindings.cpp`` page, ``gather_qmm_seg`` docstring: for each
    valid tile, rows [row_start, row_start+num_rows) of the expert-sorted x
    times expert ``e``'s dequantized weight, transposed; rows no tile covers
    are left unwritten.  hanzo-ml ``quantized/mod.rs`` page,
    ``moe_grouped_per_expert``: group routed rows by expert, one product per
    expert, scatter the rows back.  nuvec-core ``quantized.rs`` page,
    ``gather_qmm``: output batch i is x[lhs[i]] times dequantize(w)[rhs[i]]
    transposed.

  * mlx-kquant ``bindings.cpp`` page, ``quantized_matmul_residual``
    docstring: y = residual + gate * (x @ W^T), gate [N] or one row per batch
    (x's batch dims, then 1, then N), residual and gate in the output dtype,
    the fused store rounding once.  Reading taken: the M rows of x are
    ``gate_rows`` consecutive batches of M / gate_rows rows each.
  * same page, ``quantized_matmul_qmv_bias`` docstring: x @ W^T + bias for
    exactly one row of x (other row counts raise), bias of length N.
  * same page, ``quantized_matmul_glu`` docstring: y = act(x @ Wg^T) *
    (x @ Wu^T), act 'silu' or 'gelu_tanh'; the sums, the activation and the
    product in float32 (float64 here), the activation rounded once to y's
    dtype and the product once more; a float16 store keeps a finite value
    finite (clamped to the largest half of its sign), NaN and infinities
    pass.

Pins (tests/test_oracle_matmul.py): exact rational dot products (Python
``fractions``) on tiny shapes; one-hot x rows return weight columns exactly;
tile-map invariants by brute force plus a hand example; the gather equals a
per-row loop of the nuvec gather definition and reduces to qmm with one expert;
the gathered GEMV equals exact rational dot products per row and reduces to
qmm when every row names the same expert; the GLU gather's products equal the
gathered GEMV of each matrix, its activations match library routines
(``scipy.special.expit`` for the sigmoid, PyTorch's tanh-approximate gelu) at
the products, and 'silu_limit' with a limit above every |product| equals
'silu'.  The epilogues: a hand example of per-batch gate rows (constant gate
rows 1 and 2 on weight rows picked out by one-hot x), the no-gate case
reducing to the plain product, bias equal to a residual of repeated bias
rows, the float16 store's saturation on textbook values (65504 the largest
half, 65520 the first value that rounds to infinity), and the GLU with a
float32 output equal to the GLU gather's act(g) * u.
"""

from __future__ import annotations

import numpy as np

from .codecs import dequantize

TILE_ROWS = 64


def matmul_f64(x: np.ndarray, wdeq: np.ndarray) -> np.ndarray:
    """y = x @ wdeq.T in float64 (x [M, K], wdeq [N, K])."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(wdeq, dtype=np.float64).T


def qmatmul(codec: str, w: np.ndarray, k: int, x: np.ndarray) -> np.ndarray:
    """Reference for kq_qmv and kq_qmm: x [M, K] (fp16 values) times dequant(w) [N, K], transposed."""
    return matmul_f64(x, dequantize(codec, w, k, np.float32))


def expert_tile_map(sorted_ids: np.ndarray, n_experts: int):
    """Tiles (expert, row_start, num_rows) of <= 64 rows per expert segment.

    For each expert e with c_e > 0 rows starting at s_e, tiles
    (e, s_e + 64 t, min(64, c_e - 64 t)) for t < ceil(c_e / 64).  Ids outside
    [0, n_experts) get no tile.  Returns (tiles [T, 3] uint32, T).
    """
    ids = np.asarray(sorted_ids, dtype=np.int64)
    tiles = []
    for e in range(n_experts):
        rows = np.nonzero(ids == e)[0]
        if rows.size == 0:
            continue
        s, c = int(rows[0]), int(rows.size)
        for t in range(0, c, TILE_ROWS):
            tiles.append((e, s + t, min(TILE_ROWS, c - t)))
    arr = np.array(tiles, dtype=np.uint32).reshape(-1, 3)
    return arr, arr.shape[0]


def tile_map_capacity(rows: int, n_experts: int) -> int:
    """An upper bound on the tile count: ceil(rows/64) + min(n_experts, rows).

    sum_e ceil(c_e/64) <= sum_e (c_e/64 + 1) over the non-empty experts.
    """
    return -(-rows // TILE_ROWS) + min(n_experts, rows)


def gather_qmm_seg(codec: str, w: np.ndarray, k: int, x: np.ndarray, tiles: np.ndarray, fill=np.nan) -> np.ndarray:
    """Reference for kq_gather_qmm_seg: per tile, x rows times its expert's weight, transposed.

    w: [E, N, row_bytes]; x: [rows, K] expert-sorted; tiles: [T, 3].
    Rows no tile covers hold ``fill`` (they are unwritten by the contract).
    """
    n = w.shape[1]
    y = np.full((x.shape[0], n), fill, dtype=np.float64)
    for e, s, c in np.asarray(tiles, dtype=np.int64):
        y[s:s + c] = qmatmul(codec, w[e], k, x[s:s + c])
    return y


def gather_qmv(codec: str, w: np.ndarray, k: int, x: np.ndarray, ids: np.ndarray, fill=np.nan) -> np.ndarray:
    """Reference for kq_gather_qmv: row r is x[r] times expert ids[r]'s weight, transposed.

    mlx-kquant ``bindings.cpp`` page, ``gather_qmv_kq`` docstring: one
    activation row per expert slot, w laid out (n_experts, N, bytes_per_row),
    output row r uses expert indices[r].  w: [E, N, row_bytes]; x: [rows, K];
    ids: [rows].  Rows whose id is not below E hold ``fill`` (unwritten by the
    contract).
    """
    n_experts, n = w.shape[0], w.shape[1]
    ids = np.asarray(ids, dtype=np.int64)
    y = np.full((x.shape[0], n), fill, dtype=np.float64)
    for r, e in enumerate(ids):
        if 0 <= e < n_experts:
            y[r] = qmatmul(codec, w[e], k, x[r:r + 1])[0]
    return y


def glu_act(act: str, g: np.ndarray, u: np.ndarray, limit: float = 0.0) -> np.ndarray:
    """The GLU epilogue of ``moe_glu_gather_kq`` (its ``act`` argument), in float64."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):  # exp(-g) = inf for very negative g: silu(g) = -0
        return _glu_act(act, g, u, limit)


def _glu_act(act, g, u, limit):
    if act == "silu":
        return g / (1.0 + np.exp(-g)) * u
    if act == "gelu":
        return 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3))) * u
    if act == "silu_limit":
        if not limit > 0:
            raise ValueError("silu_limit needs limit > 0")
        gg = np.minimum(g, limit)
        return gg / (1.0 + np.exp(-gg)) * np.clip(u, -limit, limit)
    raise ValueError(f"unknown act {act!r}")


def moe_glu_gather(codec: str, gate_w: np.ndarray, up_w: np.ndarray, k: int, x: np.ndarray, ids: np.ndarray,
                   act: str = "silu", limit: float = 0.0, fill=np.nan) -> np.ndarray:
    """Reference for kq_moe_glu_gather: slot (t, r) is act(x[t] . gate[e], x[t] . up[e]) row by row.

    mlx-kquant ``bindings.cpp`` page, ``moe_glu_gather_kq`` docstring: x [T, K]
    (one activation row per token, shared by its slots), gate_w and up_w
    (n_experts, N, bytes_per_row), indices [T, R]; result [T, R, N].  Returned
    flattened to [T * R, N]; slots whose id is not below E hold ``fill``.
    """
    n_experts, n = gate_w.shape[0], gate_w.shape[1]
    ids = np.asarray(ids, dtype=np.int64).reshape(x.shape[0], -1)
    top_k = ids.shape[1]
    y = np.full((x.shape[0] * top_k, n), fill, dtype=np.float64)
    for t in range(x.shape[0]):
        for r in range(top_k):
            e = ids[t, r]
            if 0 <= e < n_experts:
                g = qmatmul(codec, gate_w[e], k, x[t:t + 1])[0]
                u = qmatmul(codec, up_w[e], k, x[t:t + 1])[0]
                y[t * top_k + r] = glu_act(act, g, u, limit)
    return y


def gather_mix(y: np.ndarray, inv_order: np.ndarray, scores: np.ndarray) -> np.ndarray:
    """Reference for kq_gather_mix: out[t] = sum_s scores[t, s] * y[inv_order[t * k + s]], in float64.

    mlx-kquant ``bindings.cpp`` page, ``gather_mix`` docstring.  y: [rows, N];
    inv_order: [T * k]; scores: [T, k].  Slots whose row is not below ``rows``
    add nothing.
    """
    y = np.asarray(y, dtype=np.float64)
    scores = np.asarray(scores, dtype=np.float64)
    tokens, top_k = scores.shape
    inv = np.asarray(inv_order, dtype=np.int64).reshape(tokens, top_k)
    out = np.zeros((tokens, y.shape[1]), dtype=np.float64)
    for t in range(tokens):
        for s in range(top_k):
            r = inv[t, s]
            if 0 <= r < y.shape[0]:
                out[t] += scores[t, s] * y[r]
    return out


def round_out(v: np.ndarray, out_dtype: str) -> np.ndarray:
    """v rounded to the output type, returned as float64: 'f32', or 'f16' with a
    finite value beyond the float16 range becoming the largest finite half of
    its sign (infinities and NaN pass), per the quantized_matmul_glu docstring."""
    v = np.asarray(v, dtype=np.float64)
    if out_dtype == "f32":
        return v.astype(np.float32).astype(np.float64)
    if out_dtype != "f16":
        raise ValueError(out_dtype)
    hmax = float(np.finfo(np.float16).max)
    sat = np.where(np.isfinite(v), np.clip(v, -hmax, hmax), v)
    return sat.astype(np.float16).astype(np.float64)


def quantized_matmul_residual(codec: str, w: np.ndarray, k: int, x: np.ndarray, residual: np.ndarray,
                              gate: np.ndarray | None = None) -> np.ndarray:
    """Reference for kq_quantized_matmul_residual: residual + gate * (x @ W^T) in float64.

    residual [M, N]; gate None, [N] or [G, N] with G dividing M: output row m
    takes gate row m // (M // G) (G consecutive batches of rows).
    """
    prod = qmatmul(codec, w, k, x)
    res = np.asarray(residual, dtype=np.float64).reshape(prod.shape)
    if gate is None:
        return res + prod
    g = np.asarray(gate, dtype=np.float64).reshape(-1, prod.shape[1])
    m, batches = prod.shape[0], g.shape[0]
    if batches == 0 or m % batches:
        raise ValueError(f"{batches} gate rows do not divide {m} rows")
    return res + g[np.arange(m) // (m // batches)] * prod


def quantized_matmul_qmv_bias(codec: str, w: np.ndarray, k: int, x: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """Reference for kq_quantized_matmul_qmv_bias: x @ W^T + bias, x exactly one row."""
    if x.shape[0] != 1:
        raise ValueError("the bias-fused matmul is decode-only: x must have exactly one row")
    return qmatmul(codec, w, k, x) + np.asarray(bias, dtype=np.float64)[None, :]


_GLU_NAMES = {"silu": "silu", "gelu_tanh": "gelu"}


def quantized_matmul_glu(codec: str, w_gate: np.ndarray, w_up: np.ndarray, k: int, x: np.ndarray,
                         act: str = "silu", out_dtype: str = "f32") -> np.ndarray:
    """Reference for kq_quantized_matmul_glu: round(round(act(x @ Wg^T)) * (x @ Wu^T)).

    The sums and the activation in float64; the activation rounded to
    ``out_dtype`` ('f32' or 'f16', saturating), the product with the up sum
    rounded again.  Returns the rounded values as float64.
    """
    if act not in _GLU_NAMES:
        raise ValueError(f"act {act!r} is not 'silu' or 'gelu_tanh'")
    g = qmatmul(codec, w_gate, k, x)
    u = qmatmul(codec, w_up, k, x)
    a = round_out(glu_act(_GLU_NAMES[act], g, np.ones_like(g)), out_dtype)
    return round_out(a * u, out_dtype)
