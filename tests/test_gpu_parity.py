"""GPU parity: every libkq entry point against the oracle on seeded inputs.

Sizes span several tiles and a ragged tail; edge cases: odd K (generic
kernels), rows that are not 4-byte aligned (q6_K with an odd superblock count),
K longer than one LDS chunk, subnormal / negative / zero block scales, empty
tiles, ids outside the expert range.
"""

import zlib

import numpy as np
import pytest

import _full as F
from _gpu import TOL, assert_close_rows, assert_glu_close, dev, host, say, u32
from oracle import codecs, encode, matmul

pytestmark = pytest.mark.gpu

CODECS = ("q4_k", "q6_k", "q8_0", "q4_0", "q5_k", "q4_1", "q5_0", "q5_1", "q2_k", "q3_k")
SUPER = ("q4_k", "q5_k", "q6_k", "q2_k", "q3_k")  # 256-value superblocks


@pytest.fixture(scope="module")
def kq():
    from gguf_quant_matmul_amd import kq as mod

    return mod


def _torch():
    import torch

    return torch


def _weights(codec, n, k, seed, scale=0.02):
    # N(0, scale) float32 weights from one seeded draw, oracle-encoded in row
    # chunks on a thread pool (cached: several tests share the large shapes)
    return F.random_bytes(codec, n, k, seed, scale)


# K for the 8200-row shapes: a multiple of 256 (and 64) above the 16-row
# matrix-core GEMV's activation chunk for 5 and 8 rows (6400 and 4096 values),
# so its chunk loop runs more than once with the two-way K split that N >= 8161
# takes (the up/gate projections' and the lm-head's path)
K_WIDE = 6656


def _x(m, k, seed):
    return np.random.default_rng(seed + 1000).standard_normal((m, k)).astype(np.float16)


# ---------------------------------------------------------------------------
# dequantize: bit-exact
# ---------------------------------------------------------------------------

def _random_wire(codec, n, k, rng):
    """Random wire bytes with finite fp16 fields (exponent 31 replaced)."""
    rb = codecs.row_bytes(codec, k)
    w = rng.integers(0, 256, size=(n, rb), dtype=np.uint8)
    bb = codecs.block_bytes(codec)
    blk = w.reshape(n, -1, bb)
    offs = {"q8_0": [0], "q4_0": [0], "q4_k": [0, 2], "q5_k": [0, 2], "q6_k": [208], "q4_1": [0, 2], "q5_0": [0],
            "q5_1": [0, 2], "q2_k": [80, 82], "q3_k": [108]}[codec]
    for o in offs:
        hi = blk[..., o + 1]
        bad = (hi & 0x7C) == 0x7C
        blk[..., o + 1] = np.where(bad, hi & 0xBF, hi)
    return blk.reshape(n, rb)


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("out_dtype", ["f32", "f16"])
@pytest.mark.parametrize("kind", ["encoded", "random_bytes"])
def test_dequantize_bit_exact(kq, codec, out_dtype, kind):
    torch = _torch()
    rng = np.random.default_rng(zlib.crc32(repr((codec, kind)).encode()))
    k = 256 * 5 if codec in SUPER else 32 * 7
    n = 67
    w = _weights(codec, n, k, 1) if kind == "encoded" else _random_wire(codec, n, k, rng)
    dt = np.float32 if out_dtype == "f32" else np.float16
    say(f"dequantize {codec} {out_dtype} {kind} n={n} k={k}")
    out = torch.empty((n, k), dtype=torch.float32 if dt == np.float32 else torch.float16, device="cuda")
    kq.kq_dequantize(codec, dev(w), k, out)
    got = host(out)
    ref = codecs.dequantize(codec, w, k, dt)
    ui = np.uint32 if dt == np.float32 else np.uint16
    assert np.array_equal(got.view(ui), ref.view(ui)), f"{codec}: {np.sum(got.view(ui) != ref.view(ui))} values differ"


def _q4k_double_rounding_blocks(count=12):
    """q4_K blocks whose value d*sc*q - dmin*m rounds differently to float16
    directly and via float32: the float16 output must be RNE of the float32."""
    rng = np.random.default_rng(2024)
    blocks = []
    while len(blocks) < count:
        d, dm = int(rng.integers(0x0400, 0x7800)), int(rng.integers(0x0400, 0x7800))
        sc, m, q = int(rng.integers(1, 64)), int(rng.integers(1, 64)), int(rng.integers(0, 16))
        D, DM = float(np.uint16(d).view(np.float16)), float(np.uint16(dm).view(np.float16))
        exact = D * sc * q - DM * m
        with np.errstate(over="ignore"):
            via32, direct = np.float16(np.float32(exact)), np.float16(exact)
        if via32 == direct or not np.isfinite(via32):
            continue
        b = np.zeros(144, np.uint8)
        b[0], b[1], b[2], b[3] = d & 255, d >> 8, dm & 255, dm >> 8
        b[4], b[8] = sc, m            # sub-block 0: sc_0 = s[0] & 63, m_0 = s[4] & 63
        b[16:48] = q                  # low nibbles of qs[0..31]: values 0..31 of sub-block 0
        blocks.append((b, via32))
    return blocks


def test_dequantize_f16_rounds_via_f32(kq):
    torch = _torch()
    cases = _q4k_double_rounding_blocks()
    w = np.stack([b for b, _ in cases])
    out = torch.empty((len(cases), 256), dtype=torch.float16, device="cuda")
    kq.kq_dequantize("q4_k", dev(w), 256, out)
    got = host(out)
    ref = codecs.dequantize("q4_k", w, 256, np.float16)
    for i, (_, via32) in enumerate(cases):
        assert ref[i, 0] == via32
        assert got[i, 0] == via32, (i, got[i, 0], via32)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("name", ["q4_k_block.txt", "q6_k_block.txt", "q8_0_block.txt", "q4_0_block.txt",
                                  "q5_k_block.txt", "q4_1_block.txt", "q5_0_block.txt", "q5_1_block.txt",
                                  "q2_k_block.txt", "q3_k_block.txt"])
def test_dequantize_golden_blocks(kq, name):
    from test_oracle_codecs import _load_golden

    torch = _torch()
    codec, blk, values = _load_golden(name)
    k = codecs.block_values(codec)
    w = np.tile(blk, (3, 1))  # 3 rows (row starts 2-byte aligned for q6_K)
    for tdt, ndt in ((torch.float32, np.float32), (torch.float16, np.float16)):
        out = torch.empty((3, k), dtype=tdt, device="cuda")
        kq.kq_dequantize(codec, dev(w), k, out)
        got = host(out)
        for v, expect in values:
            for r in range(3):
                assert float(got[r, v]) == expect and np.signbit(got[r, v]) == np.signbit(expect), (name, r, v)
        ref = codecs.dequantize(codec, w, k, ndt)
        ui = np.uint32 if ndt == np.float32 else np.uint16
        assert np.array_equal(got.view(ui), ref.view(ui))


# ---------------------------------------------------------------------------
# qmv / qmm: tolerance vs fp64 oracle
# ---------------------------------------------------------------------------

def _shapes_qmv(codec):
    # (8300, 1024): one or two rows take the streaming GEMV (N >= 8192, K <= 4096), 8300 rows a ragged last block
    # (8200, 768): three superblocks, so q3_K and q6_K rows start 2 bytes off a dword on every other row
    # (4102, 2048): rows a multiple of 16 bytes for every codec, so one row takes the LDS-staged GEMV, 4102
    # rows a ragged last block of four
    if codec in SUPER:
        return [(37, 512), (300, 256 * 17), (8200, K_WIDE), (8300, 1024), (8200, 768),   # 17 superblocks: q6_K rows only 2-byte aligned
                (4102, 2048)]
    return [(37, 96), (300, 4160), (45, 2048 + 32), (8200, K_WIDE), (8300, 1024),  # 96 and 2080: odd block counts -> generic kernel
            (4102, 2048)]


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 12, 16])
def test_qmv_parity(kq, codec, m):
    torch = _torch()
    for n, k in _shapes_qmv(codec):
        w = _weights(codec, n, k, 7 + n)
        x = _x(m, k, n)
        say(f"qmv {codec} m={m} n={n} k={k}")
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        kq.kq_qmv(codec, dev(w), n, k, dev(x), y)
        ref = F.qmatmul(codec, w, k, x)
        assert_close_rows(host(y), ref, what=f"qmv {codec} m={m} n={n} k={k}")
        # float16 output
        y16 = torch.full((m, n), float("nan"), dtype=torch.float16, device="cuda")
        kq.kq_qmv(codec, dev(w), n, k, dev(x), y16)
        assert_close_rows(host(y16), ref, what=f"qmv f16 {codec} m={m}")


@pytest.mark.parametrize("codec", CODECS)
def test_qmm_parity(kq, codec):
    torch = _torch()
    shapes = [(1, 37, 512), (130, 200, 512), (257, 131, 256 * 9 if codec in SUPER else 64 * 9)]
    if codec not in SUPER:
        shapes.append((70, 40, 96))  # odd block count -> generic kernel
    for m, n, k in shapes:
        w = _weights(codec, n, k, 11 + m)
        x = _x(m, k, m + n)
        ref = matmul.qmatmul(codec, w, k, x)
        for tdt in (torch.float16, torch.float32):
            say(f"qmm {codec} m={m} n={n} k={k} {tdt}")
            y = torch.empty((m, n), dtype=tdt, device="cuda")
            kq.kq_qmm(codec, dev(w), n, k, dev(x), y)
            assert_close_rows(host(y).astype(np.float64), ref, what=f"qmm {codec} m={m} n={n} k={k}")


# ---------------------------------------------------------------------------
# fused epilogues: residual / gate, bias, GLU product
# ---------------------------------------------------------------------------

def _epi_shapes(codec):
    kk = 256 * 9 if codec in SUPER else 64 * 9
    shapes = [(1, 37, kk), (3, 300, kk), (4, 45, kk), (8, 45, kk), (130, 200, kk), (260, 131, kk)]
    # 3..64 rows: the 16-row matrix-core GEMV up to 8 rows, then the wide one
    # (one, two, four A operands)
    shapes += [(12, 70, kk), (24, 90, kk), (40, 45, kk), (64, 33, kk), (40, 8200, kk)]
    # 3 and 8 rows on N >= 8161: the 16-row kernel's two-way K split, with
    # two activation chunks at 8 rows
    shapes += [(3, 8200, K_WIDE), (8, 8200, K_WIDE)]
    if codec not in SUPER:
        shapes += [(4, 45, 2048 + 32), (70, 40, 96)]  # odd block counts: generic kernels
    return shapes


@pytest.mark.parametrize("codec", CODECS)
def test_quantized_matmul_residual_parity(kq, codec):
    # y = residual + gate * p on the dot2 GEMV (M <= 2, or odd block counts),
    # matrix-core GEMVs (M <= 64) and GEMM bodies; gate
    # absent, one row, or one row per batch of consecutive rows; in place
    # (residual is y) and out of place
    torch = _torch()
    for m, n, k in _epi_shapes(codec):
        w = _weights(codec, n, k, 13 + m)
        x = _x(m, k, 2 * m + n)
        rng = np.random.default_rng(m * 1000 + n)
        batches = [b for b in (2, 4) if m % b == 0][:1]
        gates = [None, rng.uniform(-2, 2, n)] + [rng.uniform(-2, 2, (b, n)) for b in batches]
        for tdt, ndt in ((torch.float32, np.float32), (torch.float16, np.float16)):
            res = rng.standard_normal((m, n)).astype(ndt)
            for gi, gate in enumerate(gates):
                g = None if gate is None else gate.astype(ndt)
                ref = F.residual(codec, w, k, x, res, g)
                say(f"residual {codec} m={m} n={n} k={k} gate={gi} {tdt}")
                y = torch.full((m, n), float("nan"), dtype=tdt, device="cuda")
                kq.kq_quantized_matmul_residual(codec, dev(w), n, k, dev(x), dev(res), y,
                                                None if g is None else dev(g))
                e = assert_close_rows(host(y).astype(np.float64), ref, what=f"residual {codec} m={m} gate={gi}")
                say(f"  worst row error {e:.2e}")
            say(f"residual in place {codec} m={m} n={n} k={k} {tdt}")
            y = dev(res)
            kq.kq_quantized_matmul_residual(codec, dev(w), n, k, dev(x), y, y, dev(gates[1].astype(ndt)))
            ref = F.residual(codec, w, k, x, res, gates[1].astype(ndt))
            assert_close_rows(host(y).astype(np.float64), ref, what=f"residual in place {codec} m={m}")


@pytest.mark.parametrize("codec", CODECS)
def test_quantized_matmul_qmv_bias_parity(kq, codec):
    torch = _torch()
    for n, k in _shapes_qmv(codec) + [(130000, 256 if codec in SUPER else 64)]:
        w = _weights(codec, n, k, 17 + n)
        x = _x(1, k, n + 3)
        bias = np.random.default_rng(n).standard_normal(n)
        for tdt, ndt in ((torch.float32, np.float32), (torch.float16, np.float16)):
            b = bias.astype(ndt)
            say(f"qmv_bias {codec} n={n} k={k} {tdt}")
            y = torch.full((1, n), float("nan"), dtype=tdt, device="cuda")
            kq.kq_quantized_matmul_qmv_bias(codec, dev(w), n, k, dev(x), dev(b), y)
            ref = matmul.quantized_matmul_qmv_bias(codec, w, k, x, b)
            e = assert_close_rows(host(y).astype(np.float64), ref, what=f"qmv_bias {codec} n={n} k={k}")
            say(f"  worst row error {e:.2e}")


@pytest.mark.parametrize("codec", CODECS)
def test_quantized_matmul_glu_parity(kq, codec):
    # act(x Wg^T) * (x Wu^T): one GEMV pass for M <= 3, two wide matrix-core
    # GEMV passes up to 64 rows (K a multiple of 64; one, two or four A
    # operands, K split four ways for narrow N and two ways for N = 8200),
    # two GEMM passes above; the activation rounded to y's type before the
    # product.  Gate and up are row slices of one [2N, row_bytes] weight.
    torch = _torch()
    kk = 256 * 5 if codec in SUPER else 64 * 5
    shapes = [(1, 48, kk), (2, 304, kk), (3, 96, kk), (5, 48, kk), (8, 112, kk), (20, 80, kk), (48, 40, kk),
              (16, 8200, kk), (130, 208, kk), (257, 96, kk)]
    # the two passes of 4 and 8 rows on N >= 8161 (two-way K split, two
    # activation chunks at 8 rows)
    shapes += [(4, 8200, K_WIDE), (8, 8200, K_WIDE)]
    if codec not in SUPER:
        shapes += [(2, 48, 96), (70, 48, 96)]
    for m, n, k in shapes:
        wcat = _weights(codec, 2 * n, k, 23 + m, scale=0.05)
        wg, wu = wcat[:n], wcat[n:]
        x = _x(m, k, m + 5 * n)
        dcat = dev(wcat)
        rb = wcat.shape[1]
        g, u = F.qmatmul(codec, wg, k, x), F.qmatmul(codec, wu, k, x)
        assert (n * rb) % 16 == 0
        for act in ("silu", "gelu_tanh"):
            for tdt, odt in ((torch.float32, "f32"), (torch.float16, "f16")):
                say(f"glu {codec} m={m} n={n} k={k} {act} {odt}")
                y = torch.full((m, n), float("nan"), dtype=tdt, device="cuda")
                kq.kq_quantized_matmul_glu(codec, dcat[:n], dcat[n:], n, k, dev(x), y, act)
                ref = F.glu(codec, wg, wu, k, x, act, odt)[0]
                assert_glu_close(host(y), ref, g, u, act, odt == "f16", what=f"glu {codec} m={m} {act} {odt}")


@pytest.mark.parametrize("m", [2, 40, 130])
def test_quantized_matmul_glu_f16_saturates(kq, m):
    # products beyond the float16 range store the largest finite half of
    # their sign, on the one-pass GEMV (M = 2) and the wide GEMV's two passes
    # (M = 40), and on the GEMM's (M = 130)
    torch = _torch()
    n, k = 64, 256
    w = _weights("q8_0", 2 * n, k, 31, scale=25.0)
    x = _x(m, k, 77)
    ref = matmul.quantized_matmul_glu("q8_0", w[:n], w[n:], k, x, "silu", "f16")
    say(f"glu saturation m={m}")
    y = torch.empty((m, n), dtype=torch.float16, device="cuda")
    d = dev(w)
    kq.kq_quantized_matmul_glu("q8_0", d[:n], d[n:], n, k, dev(x), y, "silu")
    got = host(y).astype(np.float64)
    assert np.all(np.isfinite(got))
    # products clearly past the float16 range (1% beyond the rounding
    # boundary 65520) must store exactly the largest half of their sign
    g, u = matmul.qmatmul("q8_0", w[:n], k, x), matmul.qmatmul("q8_0", w[n:], k, x)
    prod = matmul.round_out(g / (1.0 + np.exp(-g)), "f16") * u
    far = np.abs(prod) >= 1.01 * 65520.0
    assert far.sum() > 10
    assert np.array_equal(got[far], np.sign(prod[far]) * 65504.0)
    # elsewhere the usual bar, scaled by each row's largest product before the
    # clamp: the clamp shrinks the row maximum, not the products' own error
    # (the GEMM's float16 weights put an error of about 2^-12 of the weights'
    # scale on each sum, and a cancelled gate sum times a large up sum keeps it)
    scale = np.abs(prod).max(axis=1, keepdims=True)
    assert np.all(np.abs(got - ref) <= TOL * scale), float((np.abs(got - ref) / scale).max())


def test_quantized_matmul_routes_by_m(kq):
    torch = _torch()
    n, k = 64, 512
    w = _weights("q4_k", n, k, 3)
    for m in (1, 8, 9, 16, 17, 40):
        x = _x(m, k, m)
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        kq.kq_quantized_matmul("q4_k", dev(w), n, k, dev(x), y)
        assert_close_rows(host(y), matmul.qmatmul("q4_k", w, k, x), what=f"quantized_matmul m={m}")


@pytest.mark.parametrize("n", (72, 8200))
@pytest.mark.parametrize("codec", CODECS)
def test_quantized_matmul_small_prefill_wide_gemv(kq, codec, n):
    # 9..64 rows with K a multiple of 64 take the wide matrix-core GEMV: one
    # 16-row activation operand up to 16 rows, two up to 32, four up to 64;
    # for a matrix with few rows (N = 72) K is split four ways per row group
    # instead of two (N = 8200).  Both N leave a partial last workgroup; K
    # spans several activation chunks (1024 values, or 512 for four operands
    # split two ways) and ends in a short one.
    torch = _torch()
    k = 1280 if codec in SUPER else 1344
    w = _weights(codec, n, k, 31)
    wd = dev(w)
    for m in (9, 16, 17, 31, 32, 33, 50, 64):
        x = _x(m, k, 40 + m)
        want = matmul.qmatmul(codec, w, k, x)
        for dt in (torch.float32, torch.float16):
            y = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
            say(f"{codec} quantized_matmul m={m} n={n} k={k} {dt}")
            kq.kq_quantized_matmul(codec, wd, n, k, dev(x), y)
            got = host(y).astype(np.float64)
            assert np.isfinite(got).all(), f"{codec} m={m}: unwritten outputs"
            assert_close_rows(got, want, what=f"{codec} quantized_matmul m={m} {dt}")


def test_qmm_row_independence_and_determinism(kq):
    torch = _torch()
    m, n, k = 200, 96, 1024
    w = dev(_weights("q4_k", n, k, 5))
    x = _x(m, k, 1)
    y1 = torch.empty((m, n), dtype=torch.float16, device="cuda")
    y2 = torch.empty_like(y1)
    kq.kq_qmm("q4_k", w, n, k, dev(x), y1)
    kq.kq_qmm("q4_k", w, n, k, dev(x), y2)
    assert torch.equal(y1, y2), "run-to-run determinism"
    sub = np.array([0, 5, 77, 128, 199])
    ys = torch.empty((sub.size, n), dtype=torch.float16, device="cuda")
    kq.kq_qmm("q4_k", w, n, k, dev(x[sub]), ys)
    assert np.array_equal(host(ys).view(np.uint16), host(y1)[sub].view(np.uint16)), "row independence"


def test_qmv_row_bits_do_not_depend_on_other_rows(kq):
    torch = _torch()
    n, k, m = 200, 1024, 4
    w = dev(_weights("q6_k", n, k, 9))
    x = _x(m, k, 2)
    x2 = x.copy()
    x2[1:] = _x(m - 1, k, 3)
    ya = torch.empty((m, n), dtype=torch.float32, device="cuda")
    yb = torch.empty_like(ya)
    kq.kq_qmv("q6_k", w, n, k, dev(x), ya)
    kq.kq_qmv("q6_k", w, n, k, dev(x2), yb)
    assert torch.equal(ya[0], yb[0])


# ---------------------------------------------------------------------------
# expert tile map and expert-sorted gather GEMM
# ---------------------------------------------------------------------------

def _tile_map_gpu(kq, ids, e):
    torch = _torch()
    cap = kq.kq_expert_tile_map_capacity(ids.size, e)
    map_ = torch.full((max(cap, 1), 3), -1, dtype=torch.int32, device="cuda")
    counts = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    kq.kq_expert_tile_map(u32(ids) if ids.size else torch.empty(0, dtype=torch.int32, device="cuda"), e,
                          map_[:cap] if cap else map_, counts, status)
    return map_, counts, int(host(counts)[0]), int(host(status)[0]), cap


@pytest.mark.parametrize("seed", range(6))
def test_tile_map_matches_oracle(kq, seed):
    rng = np.random.default_rng(seed)
    e = int(rng.integers(1, 300))
    rows = int(rng.integers(0, 5000))
    ids = np.sort(rng.integers(0, e, rows)).astype(np.uint32) if seed % 2 else \
        np.sort(rng.zipf(1.3, rows) % e).astype(np.uint32)
    say(f"tile map e={e} rows={rows}")
    map_, _, count, status, cap = _tile_map_gpu(kq, ids, e)
    tiles, ref_count = matmul.expert_tile_map(ids, e)
    assert count == ref_count and status == 0
    got = host(map_)[:count].view(np.uint32)
    assert np.array_equal(got, tiles)  # both expert-major
    # slots past the count are untouched
    assert np.all(host(map_)[count:cap] == -1)


def test_tile_map_workload_and_status_flags(kq):
    from gguf_quant_matmul_amd import workloads

    r = workloads.routing(4, 512, 8, 64)
    map_, _, count, status, _ = _tile_map_gpu(kq, r.sorted_ids, 64)
    assert count == 92 and status == 0
    # ids past the expert range: no tile, status bit 1
    ids = np.array([0, 0, 1, 7, 7], np.uint32)
    _, _, count, status, _ = _tile_map_gpu(kq, ids, 4)
    assert count == 2 and status == 2
    # unsorted ids: status bit 0
    ids = np.array([3, 1, 2, 2, 0], np.uint32)
    _, _, _, status, _ = _tile_map_gpu(kq, ids, 4)
    assert status & 1
    # no rows
    _, _, count, status, _ = _tile_map_gpu(kq, np.zeros(0, np.uint32), 4)
    assert count == 0 and status == 0


@pytest.mark.parametrize("codec", CODECS)
def test_gather_qmm_seg_parity(kq, codec):
    # K in one 512-value chunk or a partial one; K over several chunks with a
    # ragged last chunk and N over two 192-row blocks with a ragged tail
    torch = _torch()
    rng = np.random.default_rng(17)
    kq_ = codec in SUPER
    shapes = [(6, 96, 512 if kq_ else 320), (3, 200, 1280 if kq_ else 1344)]
    if kq_:  # several 512-value windows of the exact-operand q4_K kernel, a ragged 128-row block
        shapes.append((4, 200, 2048))
    for e, n, k in shapes:
        ids = np.sort(np.concatenate([rng.integers(0, e - 1, 190), [e - 1] * 3, [e + 2] * 4])).astype(np.uint32)
        rows = ids.size
        wf = (rng.standard_normal((e, n, k)) * 0.02).astype(np.float32)
        w = encode.quantize(codec, wf)
        x = _x(rows, k, 5)
        map_, counts, count, status, cap = _tile_map_gpu(kq, ids, e)
        assert status == 2
        tiles = host(map_)[:count].view(np.uint32)
        ref = matmul.gather_qmm_seg(codec, w, k, x, tiles)
        covered = ids < e
        for tdt in (torch.float16, torch.float32):
            say(f"seg {codec} e={e} n={n} k={k} rows={rows} {tdt}")
            y = torch.full((rows, n), float("nan"), dtype=tdt, device="cuda")
            kq.kq_gather_qmm_seg(codec, dev(w), e, n, k, dev(x), map_[:cap], counts, y)
            got = host(y).astype(np.float64)
            assert np.all(np.isnan(got[~covered])), "uncovered rows must stay unwritten"
            assert_close_rows(got[covered], ref[covered], what=f"seg {codec} n={n} k={k}")


@pytest.mark.parametrize("scale", [2.0 ** -14, 2.0 ** 9])
def test_gather_seg_q4k_activation_range(kq, scale):
    # the q4_K segment kernel forms sub-block sums of x for the min term:
    # activations far below and far above 1 (sums near 2^-10 and near 2^16)
    # keep the row bar
    torch = _torch()
    rng = np.random.default_rng(29)
    e, n, k = 3, 136, 1024
    ids = np.sort(rng.integers(0, e, 150)).astype(np.uint32)
    rows = ids.size
    w = encode.quantize("q4_k", (rng.standard_normal((e, n, k)) * 0.02).astype(np.float32))
    x = (np.random.default_rng(31).standard_normal((rows, k)) * scale).astype(np.float16)
    map_, counts, count, status, cap = _tile_map_gpu(kq, ids, e)
    tiles = host(map_)[:count].view(np.uint32)
    ref = matmul.gather_qmm_seg("q4_k", w, k, x, tiles)
    say(f"seg q4_k activation scale {scale}")
    y = torch.full((rows, n), float("nan"), dtype=torch.float32, device="cuda")
    kq.kq_gather_qmm_seg("q4_k", dev(w), e, n, k, dev(x), map_[:cap], counts, y)
    assert_close_rows(host(y).astype(np.float64), ref, what=f"seg q4_k x scale {scale}")


@pytest.mark.parametrize("codec", ["q4_k", "q4_0", "q8_0", "q5_k", "q4_1", "q5_0", "q5_1", "q2_k", "q3_k"])
def test_gather_seg_tile_boundaries(kq, codec):
    # expert rows 96 (a full tile and a 32-row tail), 97 (a 33-row tail),
    # 133 (two full tiles and a 5-row tail), 64 (one full tile), 20 and one
    # out-of-range id block: full, partial and single-group tiles of one
    # expert back to back in one map; N with a ragged last column block
    torch = _torch()
    rng = np.random.default_rng(23)
    e, n, k = 5, 400, 512
    sizes = [96, 97, 133, 64, 20]
    ids = np.concatenate([np.full(c, i, np.uint32) for i, c in enumerate(sizes)] + [np.full(3, e + 1, np.uint32)])
    rows = ids.size
    w = encode.quantize(codec, (rng.standard_normal((e, n, k)) * 0.02).astype(np.float32))
    x = _x(rows, k, 6)
    map_, counts, count, status, cap = _tile_map_gpu(kq, ids, e)
    tiles = host(map_)[:count].view(np.uint32)
    assert [int(t[2]) for t in tiles] == [64, 32, 64, 33, 64, 64, 5, 64, 20]
    ref = matmul.gather_qmm_seg(codec, w, k, x, tiles)
    covered = ids < e
    for tdt in (torch.float16, torch.float32):
        say(f"seg tile boundaries {codec} {tdt}")
        y = torch.full((rows, n), float("nan"), dtype=tdt, device="cuda")
        kq.kq_gather_qmm_seg(codec, dev(w), e, n, k, dev(x), map_[:cap], counts, y)
        got = host(y).astype(np.float64)
        assert np.all(np.isnan(got[~covered])), "uncovered rows must stay unwritten"
        assert_close_rows(got[covered], ref[covered], what=f"seg tile boundaries {codec}")


@pytest.mark.parametrize("n", [200, 50])
def test_gather_seg_q4k_merged_tails(kq, n):
    # the q4_K segment kernel works a full tile and a following tail of at most
    # 16 rows of the same expert as one 80-row tile.  Expert rows 80 (64 + 16,
    # merged), 65 (64 + 1, merged), 81 (64 + 17, not merged), 144 (64 + 64 +
    # 16: the second full tile takes the tail), 16 and 64; N = 200 leaves the
    # last 64-row weight block ragged, N = 50 leaves the tails' blocks empty.
    # The same map with its entries reversed merges nothing (a tail then
    # precedes its full tile) and must give the same bits.
    torch = _torch()
    rng = np.random.default_rng(37)
    e, k = 6, 1024
    sizes = [80, 65, 81, 144, 16, 64]
    ids = np.concatenate([np.full(c, i, np.uint32) for i, c in enumerate(sizes)] + [np.full(2, e + 3, np.uint32)])
    rows = ids.size
    w = encode.quantize("q4_k", (rng.standard_normal((e, n, k)) * 0.02).astype(np.float32))
    x = _x(rows, k, 9)
    map_, counts, count, status, cap = _tile_map_gpu(kq, ids, e)
    tiles = host(map_)[:count].view(np.uint32)
    assert [int(t[2]) for t in tiles] == [64, 16, 64, 1, 64, 17, 64, 64, 16, 16, 64]
    ref = matmul.gather_qmm_seg("q4_k", w, k, x, tiles)
    covered = ids < e
    rev = torch.from_numpy(np.ascontiguousarray(host(map_)[:count][::-1])).cuda()
    for tdt in (torch.float16, torch.float32):
        say(f"seg q4_k merged tails n={n} {tdt}")
        y = torch.full((rows, n), float("nan"), dtype=tdt, device="cuda")
        kq.kq_gather_qmm_seg("q4_k", dev(w), e, n, k, dev(x), map_[:cap], counts, y)
        got = host(y).astype(np.float64)
        assert np.all(np.isnan(got[~covered])), "uncovered rows must stay unwritten"
        assert_close_rows(got[covered], ref[covered], what=f"seg q4_k merged tails n={n}")
        y2 = torch.full((rows, n), float("nan"), dtype=tdt, device="cuda")
        kq.kq_gather_qmm_seg("q4_k", dev(w), e, n, k, dev(x), rev, counts, y2)
        b1 = host(y).view(np.uint16 if tdt == torch.float16 else np.uint32)
        b2 = host(y2).view(np.uint16 if tdt == torch.float16 else np.uint32)
        assert np.array_equal(b1, b2), "merged and unmerged tiles must give the same bits"


@pytest.mark.parametrize("codec", CODECS)
def test_gather_qmv_parity(kq, codec):
    # one activation row per routed slot, ids in any order; an id past the
    # expert count leaves its row unwritten.  A 40000-row case takes the
    # 16-lanes-per-row layout, the small ones a whole wave per row.
    torch = _torch()
    rng = np.random.default_rng(19)
    cases = [(5, 100, 512, 9), (3, 33, 256, 4)]
    if codec == "q4_0":
        cases.append((2, 40000, 256, 3))
    for e, n, k, rows in cases:
        wf = (rng.standard_normal((e, n, k)) * 0.02).astype(np.float32)
        w = encode.quantize(codec, wf)
        x = _x(rows, k, 7 + n)
        ids = rng.integers(0, e, rows).astype(np.uint32)
        ids[1] = e + 3
        ref = matmul.gather_qmv(codec, w, k, x, ids)
        live = ids < e
        for tdt in (torch.float32, torch.float16):
            say(f"gather_qmv {codec} e={e} n={n} k={k} rows={rows} {tdt}")
            y = torch.full((rows, n), float("nan"), dtype=tdt, device="cuda")
            kq.kq_gather_qmv(codec, dev(w), e, n, k, dev(x), u32(ids), y)
            got = host(y).astype(np.float64)
            assert np.all(np.isnan(got[~live])), "rows with an out-of-range id must stay unwritten"
            assert_close_rows(got[live], ref[live], what=f"gather_qmv {codec} n={n} {tdt}")


@pytest.mark.parametrize("codec", CODECS)
def test_moe_glu_gather_parity(kq, codec):
    # gate and up of each routed slot with the GLU epilogue; one activation
    # row per token shared by its slots; an id past the expert count leaves
    # its slot unwritten.  The 40000-row case takes the 16-lanes-per-row
    # layout.
    torch = _torch()
    rng = np.random.default_rng(29)
    cases = [(5, 100, 512, 3, 4), (3, 33, 256, 2, 1)]
    if codec == "q4_k":
        cases.append((2, 40000, 256, 1, 2))
    for e, n, k, tokens, top_k in cases:
        gate = encode.quantize(codec, (rng.standard_normal((e, n, k)) * 0.05).astype(np.float32))
        up = encode.quantize(codec, (rng.standard_normal((e, n, k)) * 0.05).astype(np.float32))
        x = _x(tokens, k, 11 + n)
        ids = rng.integers(0, e, (tokens, top_k)).astype(np.uint32)
        ids.flat[-1] = e + 2
        live = ids.reshape(-1) < e
        for act, limit in (("silu", 0.0), ("gelu", 0.0), ("silu_limit", 0.4)):
            ref = matmul.moe_glu_gather(codec, gate, up, k, x, ids, act, limit)
            for tdt in (torch.float32, torch.float16):
                say(f"moe_glu_gather {codec} e={e} n={n} k={k} T={tokens} R={top_k} {act} {tdt}")
                y = torch.full((tokens * top_k, n), float("nan"), dtype=tdt, device="cuda")
                kq.kq_moe_glu_gather(codec, dev(gate), dev(up), e, n, k, dev(x), u32(ids), y, act, limit)
                got = host(y).astype(np.float64)
                assert np.all(np.isnan(got[~live])), "slots with an out-of-range id must stay unwritten"
                assert_close_rows(got[live], ref[live], what=f"moe_glu_gather {codec} n={n} {act} {tdt}")


def _mix_bound(y, inv, scores, f16):
    # float32 sum of top_k terms in order, then one rounding to the output type
    terms = np.abs(scores.astype(np.float64))[:, :, None] * np.abs(
        np.where((inv < y.shape[0])[:, None], y[np.minimum(inv, y.shape[0] - 1).astype(np.int64)], 0.0)
    ).reshape(scores.shape[0], scores.shape[1], -1)
    return scores.shape[1] * 2.0 ** -23 * terms.sum(axis=1)


def test_gather_mix_parity(kq):
    torch = _torch()
    rng = np.random.default_rng(31)
    for tokens, top_k, n in ((37, 5, 1028), (3, 1, 4), (70000, 2, 4)):
        rows = tokens * top_k
        inv = rng.permutation(rows).astype(np.uint32)
        inv[:: max(1, rows // 7)] = rows + 5  # some slots name no row
        scores = rng.standard_normal((tokens, top_k)).astype(np.float32)
        for f16 in (True, False):
            dt = np.float16 if f16 else np.float32
            y = rng.standard_normal((rows, n)).astype(dt)
            ref = matmul.gather_mix(y, inv, scores)
            say(f"gather_mix tokens={tokens} top_k={top_k} n={n} f16={f16}")
            out = torch.full((tokens, n), float("nan"), dtype=torch.float16 if f16 else torch.float32, device="cuda")
            kq.kq_gather_mix(dev(y), u32(inv), dev(scores), out)
            got = host(out).astype(np.float64)
            bound = _mix_bound(y.astype(np.float64), inv, scores, f16)
            if f16:
                bound = bound + 2.0 ** -11 * np.abs(ref) + 2.0 ** -24
            assert np.all(np.abs(got - ref) <= bound), f"gather_mix max excess {np.max(np.abs(got - ref) - bound):.3e}"


def test_gather_qmv_row_equals_qmv_bits(kq):
    # a routed row runs the same kernel as a one-row GEMV on its expert
    torch = _torch()
    rng = np.random.default_rng(20)
    e, n, k = 4, 64, 1024
    w = encode.quantize("q4_k", (rng.standard_normal((e, n, k)) * 0.02).astype(np.float32))
    x = _x(3, k, 9)
    ids = np.array([3, 0, 3], dtype=np.uint32)
    y = torch.empty((3, n), dtype=torch.float32, device="cuda")
    wd = dev(w)
    kq.kq_gather_qmv("q4_k", wd, e, n, k, dev(x), u32(ids), y)
    for r, ex in enumerate(ids):
        y1 = torch.empty((1, n), dtype=torch.float32, device="cuda")
        kq.kq_qmv("q4_k", wd[int(ex)], n, k, dev(x[r:r + 1]), y1)
        assert torch.equal(y[r:r + 1], y1)


def test_gather_seg_one_expert_equals_qmm_bits(kq):
    torch = _torch()
    n, k, rows = 100, 1024, 150
    w = _weights("q4_k", n, k, 21)
    x = dev(_x(rows, k, 8))
    ids = np.zeros(rows, np.uint32)
    map_, counts, count, _, cap = _tile_map_gpu(kq, ids, 1)
    assert count == 3
    ys = torch.empty((rows, n), dtype=torch.float16, device="cuda")
    kq.kq_gather_qmm_seg("q4_k", dev(w[None]), 1, n, k, x, map_[:cap], counts, ys)
    ref = matmul.qmatmul("q4_k", w, k, host(x))
    assert_close_rows(host(ys).astype(np.float64), ref, what="seg one expert")


def test_gather_seg_row_independence(kq):
    torch = _torch()
    rng = np.random.default_rng(3)
    e, n, k = 4, 64, 512
    w = dev(encode.quantize("q4_k", (rng.standard_normal((e, n, k)) * 0.02).astype(np.float32)))
    ids = np.sort(rng.integers(0, e, 200)).astype(np.uint32)
    x = _x(200, k, 4)
    map_, counts, _, _, cap = _tile_map_gpu(kq, ids, e)
    y = torch.empty((200, n), dtype=torch.float16, device="cuda")
    kq.kq_gather_qmm_seg("q4_k", w, e, n, k, dev(x), map_[:cap], counts, y)
    keep = np.sort(rng.choice(200, 60, replace=False))
    map2, counts2, _, _, cap2 = _tile_map_gpu(kq, ids[keep], e)
    y2 = torch.empty((60, n), dtype=torch.float16, device="cuda")
    kq.kq_gather_qmm_seg("q4_k", w, e, n, k, dev(x[keep]), map2[:cap2], counts2, y2)
    # rows land in different tiles (and tile positions) but each row's bits are the same
    assert np.array_equal(host(y2).view(np.uint16), host(y)[keep].view(np.uint16))


# ---------------------------------------------------------------------------
# encoder: bit-exact bytes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("dist", ["normal", "t5", "positive", "negative", "mixed"])
def test_quantize_bytes_match_oracle(kq, codec, dist):
    torch = _torch()
    rng = np.random.default_rng(zlib.crc32(repr((codec, dist)).encode()))
    n, k = 48, 1024
    if dist == "normal":
        w = rng.standard_normal((n, k)).astype(np.float32) * np.float32(0.02)
    elif dist == "t5":
        w = (rng.standard_t(5, (n, k)) * 0.02).astype(np.float32)
    elif dist == "positive":
        w = rng.uniform(0.001, 1, (n, k)).astype(np.float32)
    elif dist == "negative":
        w = -rng.uniform(0.001, 1, (n, k)).astype(np.float32)
    else:
        w = rng.standard_normal((n, k)).astype(np.float32)
        w[::3] *= np.float32(1e-6)
        w[1::5] = 0
        w[2, :300] = 0
    say(f"quantize {codec} {dist}")
    out = torch.empty((n, codecs.row_bytes(codec, k)), dtype=torch.uint8, device="cuda")
    kq.kq_quantize(codec, dev(w), out)
    got = host(out)
    ref = encode.quantize(codec, w)
    assert np.array_equal(got, ref), f"{np.sum(got != ref)} bytes differ"


@pytest.mark.parametrize("groups", [1, 7, 300])
def test_stream_read_xor(kq, groups):
    # the plain-read reference: group g XORs the 32-bit words of the g-th
    # contiguous share of ceil(n16 / groups) 16-byte pieces
    torch = _torch()
    rng = np.random.default_rng(groups)
    n16 = 10007
    src = rng.integers(0, 2 ** 32, size=n16 * 4, dtype=np.uint64).astype(np.uint32)
    out = torch.full((4 * groups,), -1, dtype=torch.int32, device="cuda")
    kq.kq_stream_read(dev(src.view(np.int32)), out)
    per = -(-n16 // groups)
    got = host(out).view(np.uint32).reshape(groups, 4)
    want = np.array([np.bitwise_xor.reduce(src[4 * g * per: 4 * min(n16, (g + 1) * per)]) if g * per < n16 else 0
                     for g in range(groups)], dtype=np.uint32)
    # each wave's word covers its lanes' pieces; the four of a group XOR to the share's XOR
    assert np.array_equal(np.bitwise_xor.reduce(got, axis=1), want)
