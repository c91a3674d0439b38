"""Pins for the oracle's encoder (reading R5: round to nearest against the stored parameters).

  * Brute force: for every value, decode the block with EVERY code of the
    codec and check the chosen code is a nearest grid point, ties to the
    lower code.
  * q8_0 closed form: |w - y| <= D/2 for every value (D the stored fp16 d).
  * Zero blocks encode to the zero-point code and decode to exact zeros.
  * Decoding then re-encoding a q8_0 / q4_0 tensor gives the same bytes.
"""

import zlib

import numpy as np
import pytest

from oracle import codecs, encode


def _all_codes_block(codec, blk, c):
    """A copy of the blocks with every code replaced by code c (packed per the layout reading)."""
    b = blk.copy()
    if codec == "q8_0":
        b[..., 2:34] = np.uint8(c & 255)
    elif codec == "q4_0":
        b[..., 2:18] = np.uint8(c | (c << 4))
    elif codec == "q4_k":
        b[..., 16:144] = np.uint8(c | (c << 4))
    elif codec in ("q4_1", "q5_0", "q5_1"):
        o = {"q4_1": 4, "q5_0": 6, "q5_1": 8}[codec]
        b[..., o:o + 16] = np.uint8((c & 15) | ((c & 15) << 4))
        if codec != "q4_1":
            b[..., o - 4:o] = np.uint8(255 * (c >> 4))
    elif codec == "q2_k":
        b[..., 16:80] = np.uint8(c * 0x55)
    elif codec == "q3_k":
        u = c + 4
        b[..., 0:32] = np.uint8(255 * (u >> 2))
        b[..., 32:96] = np.uint8((u & 3) * 0x55)
    elif codec == "q5_k":
        lo, h1 = c & 15, c >> 4
        b[..., 16:48] = np.uint8(255 * h1)
        b[..., 48:176] = np.uint8(lo | (lo << 4))
    elif codec == "q6_k":
        lo, h2 = c & 15, c >> 4
        b[..., 0:128] = np.uint8(lo | (lo << 4))
        b[..., 128:192] = np.uint8(h2 | (h2 << 2) | (h2 << 4) | (h2 << 6))
    return b


CODE_RANGE = {"q8_0": range(-128, 128), "q4_0": range(16), "q4_k": range(16), "q6_k": range(64),
              "q5_k": range(32), "q4_1": range(16), "q5_0": range(32), "q5_1": range(32),
              "q2_k": range(4), "q3_k": range(-4, 4)}


def _codes(codec, blk):
    if codec == "q8_0":
        return codecs.fields_q8_0(blk)[1].reshape(blk.shape[0], -1)
    if codec == "q4_0":
        return codecs.fields_q4_0(blk)[1].reshape(blk.shape[0], -1)
    if codec == "q4_k":
        return codecs.fields_q4_k(blk)[4].reshape(blk.shape[0], -1)
    if codec == "q5_k":
        return codecs.fields_q5_k(blk)[4].reshape(blk.shape[0], -1)
    if codec == "q2_k":
        return codecs.fields_q2_k(blk)[4].reshape(blk.shape[0], -1)
    if codec == "q3_k":
        return codecs.fields_q3_k(blk)[2].reshape(blk.shape[0], -1)
    if codec in ("q4_1", "q5_0", "q5_1"):
        return codecs.fields_legacy(codec, blk)[2].reshape(blk.shape[0], -1)
    return codecs.fields_q6_k(blk)[2].reshape(blk.shape[0], -1)


@pytest.mark.parametrize("codec", codecs.CODECS)
@pytest.mark.parametrize("dist", ["normal", "t5", "positive", "negative"])
def test_chosen_code_is_nearest_grid_point(codec, dist):
    rng = np.random.default_rng(zlib.crc32(repr((codec, dist)).encode()))
    k = codecs.block_values(codec)
    n = 6
    if dist == "normal":
        w = rng.standard_normal((n, k)).astype(np.float32) * np.float32(0.02)
    elif dist == "t5":
        w = (rng.standard_t(5, (n, k)) * 0.02).astype(np.float32)
    elif dist == "positive":
        w = rng.uniform(0.01, 1.0, (n, k)).astype(np.float32)
    else:
        w = -rng.uniform(0.01, 1.0, (n, k)).astype(np.float32)
    wq = encode.quantize(codec, w)
    blk = wq.reshape(n, 1, -1)
    chosen = _codes(codec, blk)
    grid = []
    codes = list(CODE_RANGE[codec])
    for c in codes:
        grid.append(codecs.dequantize(codec, _all_codes_block(codec, blk, c).reshape(n, -1), k).astype(np.float64))
    grid = np.stack(grid, axis=-1)  # [n, k, ncodes]
    err = np.abs(w.astype(np.float64)[..., None] - grid)
    best = np.array(codes)[np.argmin(err, axis=-1)]  # argmin takes the first = lowest code on ties
    assert np.array_equal(chosen, best)
    # and the decoded tensor is the grid point of the chosen code
    y = codecs.dequantize(codec, wq, k).astype(np.float64)
    assert np.array_equal(y, np.take_along_axis(grid, (chosen - codes[0])[..., None], -1)[..., 0])


def test_q8_0_error_bound_half_step():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((32, 512)).astype(np.float32) * np.float32(0.02)
    wq = encode.quantize("q8_0", w)
    y = codecs.dequantize("q8_0", wq, 512).astype(np.float64)
    d = codecs.fields_q8_0(wq.reshape(32, 16, 34))[0]  # [32, 16]
    D = np.repeat(d, 32, axis=1)
    assert np.all(np.abs(w - y) <= D / 2)


@pytest.mark.parametrize("codec", codecs.CODECS)
def test_zero_block(codec):
    k = codecs.block_values(codec)
    wq = encode.quantize(codec, np.zeros((2, k), np.float32))
    y = codecs.dequantize(codec, wq, k)
    assert np.all(y == 0) and not np.any(np.signbit(y))


@pytest.mark.parametrize("codec", ["q8_0", "q4_0"])
def test_decode_encode_fixed_point(codec):
    rng = np.random.default_rng(5)
    w = rng.standard_normal((8, 256)).astype(np.float32)
    wq = encode.quantize(codec, w)
    y = codecs.dequantize(codec, wq, 256)
    assert np.array_equal(encode.quantize(codec, y), wq)


@pytest.mark.parametrize("codec", codecs.CODECS)
def test_round_trip_error_small_relative_to_block(codec):
    rng = np.random.default_rng(9)
    k = 4 * codecs.block_values(codec)
    w = rng.standard_normal((16, k)).astype(np.float32) * np.float32(0.02)
    y = codecs.dequantize(codec, encode.quantize(codec, w), k)
    bits = codecs.GEOMETRY[codec][1]
    rel = np.sqrt(np.mean((w - y) ** 2)) / np.sqrt(np.mean(w ** 2))
    # uniform-noise rms of a b-bit grid spanning roughly +-3 sigma: ~ 6 / 2^b / sqrt(12)
    assert rel < 2.5 * 6 / 2 ** bits / np.sqrt(12)


# ---- hand-encoded blocks: the block-parameter rule (tests/golden/*_encode.txt) ----

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


def _load_encode_golden(name):
    """Parse a hand-encoded golden: inputs (sub-block patterns or single values) and expectations."""
    spec = {"subs": [], "w": [], "codes": []}
    with open(__import__("os").path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            val = val.split()
            if key == "codec":
                spec["codec"] = val[0]
            elif key == "sub":
                spec["subs"].append((int(val[0]), float(val[1]), float(val[2]), float(val[3])))
            elif key == "w":
                spec["w"].append((int(val[0]), float(val[1])))
            elif key == "code":
                spec["codes"].append((int(val[0]), int(val[1])))
            elif key in ("header", "bytes"):
                spec[key] = bytes.fromhex("".join(val))
            elif key in ("sc", "m"):
                spec[key] = [int(v) for v in val]
    return spec


def _golden_input(spec):
    codec = spec["codec"]
    if spec["subs"]:
        sub = {"q4_k": 32, "q6_k": 16}[codec]
        w = np.zeros(256, np.float64)
        for j, base, step, last in spec["subs"]:
            w[sub * j: sub * j + sub - 1] = base + step * np.arange(sub - 1)
            w[sub * j + sub - 1] = last
    else:
        n = len(spec["bytes"]) // codecs.block_bytes(codec) * codecs.block_values(codec)
        w = np.zeros(n, np.float64)
        for i, v in spec["w"]:
            w[i] = v
    w32 = w.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), w), "golden inputs must be exact in float32"
    return w32[None, :]


@pytest.mark.parametrize("name", ["q4_k_encode.txt", "q6_k_encode.txt", "q8_0_encode.txt", "q4_0_encode.txt"])
def test_golden_hand_encoded_blocks(name):
    spec = _load_encode_golden(name)
    codec = spec["codec"]
    w = _golden_input(spec)
    wq = encode.quantize(codec, w)[0]
    if "bytes" in spec:
        assert wq.tobytes().hex() == spec["bytes"].hex()
    if "header" in spec:
        if codec == "q4_k":  # d, dmin and the 12 packed scale bytes lead the block
            assert wq[:16].tobytes().hex() == spec["header"].hex()
        else:  # q6_K: d closes the block
            assert wq[208:210].tobytes().hex() == spec["header"].hex()
    blk = wq.reshape(1, 1, -1)
    if codec == "q4_k":
        _, _, sc, m, q = codecs.fields_q4_k(blk)
        assert sc.reshape(-1).tolist() == spec["sc"] and m.reshape(-1).tolist() == spec["m"]
        q = q.reshape(-1)
    elif codec == "q6_k":
        f = codecs.fields_q6_k(blk)
        assert f[1].reshape(-1).tolist() == spec["sc"]
        q = f[2].reshape(-1)
    else:
        q = _codes(codec, blk).reshape(-1)
    for v, expect in spec["codes"]:
        assert int(q[v]) == expect, (name, v, int(q[v]), expect)
