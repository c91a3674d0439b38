"""Pins for the oracle's codec geometry, field decode and dequantization.

Each test checks the oracle against something other than itself:
  * the byte totals of the mlx-kquant README "Codec reference" table;
  * NumPy's own binary16 conversion (a library routine) for every bit pattern;
  * hand-decoded superblocks (tests/golden/*.txt, derivations in the files);
  * codes packed by hand here from the layout reading, then decoded;
  * the MLX affine closed form (nuvec-core ``quantized.rs`` module comment:
    value = scale * code + bias with code in [0, 2^bits - 1]) as a second,
    independently written decoder over the same fields.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_codec_table_byte_totals():
    # mlx-kquant README, "Codec reference": q4_k 256/4/144, q6_k 256/6/210, q8_0 32/8/34, q4_0 32/4/18.
    assert codecs.GEOMETRY["q4_k"] == (256, 4, 144)
    assert codecs.GEOMETRY["q6_k"] == (256, 6, 210)
    assert codecs.GEOMETRY["q8_0"] == (32, 8, 34)
    assert codecs.GEOMETRY["q4_0"] == (32, 4, 18)
    assert codecs.GEOMETRY["q5_k"] == (256, 5, 176)  # the same table's q5_k row
    assert 2 + 2 + 12 + 32 + 128 == 176              # d, dmin, scales, qh, qs
    assert codecs.GEOMETRY["q4_1"] == (32, 4, 20) and 2 + 2 + 16 == 20          # d, m, qs
    assert codecs.GEOMETRY["q5_0"] == (32, 5, 22) and 2 + 4 + 16 == 22          # d, qh, qs
    assert codecs.GEOMETRY["q5_1"] == (32, 5, 24) and 2 + 2 + 4 + 16 == 24      # d, m, qh, qs
    assert codecs.GEOMETRY["q2_k"] == (256, 2, 84) and 16 + 64 + 2 + 2 == 84    # scales, qs, d, dmin
    assert codecs.GEOMETRY["q3_k"] == (256, 3, 110) and 32 + 64 + 12 + 2 == 110  # hmask, qs, scales, d
    # The layout reading must account for every byte of the block.
    assert 2 + 2 + 12 + 128 == 144          # d, dmin, scales, qs
    assert 128 + 64 + 16 + 2 == 210         # ql, qh, scales, d
    assert 2 + 32 == 34 and 2 + 16 == 18
    # Bytes per weight: 0.5625 for both q4_0 and q4_K (hanzo-ml quantized/mod.rs, cache_or_upload comment).
    assert 144 / 256 == 18 / 32 == 0.5625


def test_row_bytes_and_divisibility():
    assert codecs.row_bytes("q4_k", 4096) == 2304
    assert codecs.row_bytes("q6_k", 4096) == 3360
    assert codecs.row_bytes("q8_0", 4096) == 4352
    assert codecs.row_bytes("q4_0", 4096) == 2304
    with pytest.raises(ValueError):
        codecs.row_bytes("q4_k", 4000)
    with pytest.raises(ValueError):
        codecs.row_bytes("q8_0", 48)


def test_f16_decode_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    mine = codecs.f16_bits_to_f64(bits)
    lib = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    both_nan = np.isnan(mine) & np.isnan(lib)
    same = (mine == lib) & (np.signbit(mine) == np.signbit(lib))
    assert np.all(same | both_nan)
    assert np.isnan(mine).sum() == 2 * 1023
    assert codecs.f16_bits_to_f64(0x8000) == 0 and np.signbit(codecs.f16_bits_to_f64(0x8000))
    assert codecs.f16_bits_to_f64(0x0001) == 2.0 ** -24
    assert codecs.f16_bits_to_f64(0x7BFF) == 65504.0


def _load_golden(name):
    codec, raw, values = None, None, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line.startswith("codec:"):
                codec = line.split(":", 1)[1].strip()
            elif line.startswith("bytes:"):
                raw = bytes.fromhex(line.split(":", 1)[1])
            elif line.startswith("value:"):
                idx, val = line.split(":", 1)[1].split()
                values.append((int(idx), float.fromhex(val) if "0x" in val else float(val)))
    return codec, np.frombuffer(raw, dtype=np.uint8), values


@pytest.mark.parametrize("name", ["q4_k_block.txt", "q6_k_block.txt", "q8_0_block.txt", "q4_0_block.txt",
                                  "q5_k_block.txt", "q4_1_block.txt", "q5_0_block.txt", "q5_1_block.txt",
                                  "q2_k_block.txt", "q3_k_block.txt"])
@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_golden_hand_decoded_blocks(name, dtype):
    codec, blk, values = _load_golden(name)
    assert blk.size == codecs.block_bytes(codec)
    y = codecs.dequantize(codec, blk[None, :], codecs.block_values(codec), dtype)[0]
    assert y.dtype == dtype
    for v, expect in values:
        got = float(y[v])
        assert got == expect, (name, v, got, expect)
        assert np.signbit(got) == np.signbit(expect), (name, v, "sign of zero")


def _hand_pack(codec, rng, nblocks):
    """Pack random codes and parameters by hand from the layout reading; return (bytes, fields)."""
    if codec == "q8_0":
        q = rng.integers(-128, 128, size=(nblocks, 32))
        d = rng.integers(0, 0x7C00, size=nblocks) | (rng.integers(0, 2, size=nblocks) << 15)
        out = np.zeros((nblocks, 34), np.uint8)
        out[:, 0], out[:, 1] = d & 255, d >> 8
        out[:, 2:] = q & 255
        return out, dict(d=d, q=q)
    if codec == "q4_0":
        q = rng.integers(0, 16, size=(nblocks, 32))
        d = rng.integers(0, 0x7C00, size=nblocks)
        out = np.zeros((nblocks, 18), np.uint8)
        out[:, 0], out[:, 1] = d & 255, d >> 8
        for v in range(32):
            out[:, 2 + (v % 16)] |= (q[:, v] << (4 * (v // 16))).astype(np.uint8)
        return out, dict(d=d, q=q)
    if codec == "q4_k":
        q = rng.integers(0, 16, size=(nblocks, 256))
        sc = rng.integers(0, 64, size=(nblocks, 8))
        m = rng.integers(0, 64, size=(nblocks, 8))
        d = rng.integers(0, 0x7C00, size=nblocks)
        dm = rng.integers(0, 0x7C00, size=nblocks)
        out = np.zeros((nblocks, 144), np.uint8)
        out[:, 0], out[:, 1], out[:, 2], out[:, 3] = d & 255, d >> 8, dm & 255, dm >> 8
        # 6-bit pairs: low 6 bits of j<4 in bytes 0..7, j>=4 split 4+2 bits.
        for j in range(8):
            if j < 4:
                out[:, 4 + j] |= sc[:, j].astype(np.uint8)
                out[:, 8 + j] |= m[:, j].astype(np.uint8)
            else:
                out[:, 12 + (j - 4)] |= ((sc[:, j] & 15) | ((m[:, j] & 15) << 4)).astype(np.uint8)
                out[:, 4 + (j - 4)] |= ((sc[:, j] >> 4) << 6).astype(np.uint8)
                out[:, 8 + (j - 4)] |= ((m[:, j] >> 4) << 6).astype(np.uint8)
        for v in range(256):
            j, l = divmod(v, 32)
            out[:, 16 + 32 * (j // 2) + l] |= (q[:, v] << (4 * (j % 2))).astype(np.uint8)
        return out, dict(d=d, dm=dm, sc=sc, m=m, q=q)
    if codec in ("q4_1", "q5_0", "q5_1"):
        bits = 4 if codec == "q4_1" else 5
        q = rng.integers(0, 1 << bits, size=(nblocks, 32))
        d = rng.integers(0, 0x7C00, size=nblocks) | (rng.integers(0, 2, size=nblocks) << 15)
        mm = rng.integers(0, 0x7C00, size=nblocks) | (rng.integers(0, 2, size=nblocks) << 15)
        out = np.zeros((nblocks, codecs.block_bytes(codec)), np.uint8)
        out[:, 0], out[:, 1] = d & 255, d >> 8
        o = 2
        if codec != "q5_0":
            out[:, 2], out[:, 3] = mm & 255, mm >> 8
            o = 4
        if bits == 5:  # fifth bits: bit v of the little-endian uint32 at o
            for v in range(32):
                out[:, o + v // 8] |= ((q[:, v] >> 4) << (v % 8)).astype(np.uint8)
            o += 4
        for v in range(32):
            out[:, o + (v % 16)] |= ((q[:, v] & 15) << (4 * (v // 16))).astype(np.uint8)
        return out, dict(d=d, m=mm, q=q)
    if codec == "q3_k":
        q = rng.integers(-4, 4, size=(nblocks, 256))
        sc = rng.integers(-32, 32, size=(nblocks, 16))
        d = rng.integers(0, 0x7C00, size=nblocks) | (rng.integers(0, 2, size=nblocks) << 15)
        out = np.zeros((nblocks, 110), np.uint8)
        for v in range(256):
            h, r = divmod(v, 128)
            c, l = divmod(r, 32)
            u = q[:, v] + 4
            out[:, 32 + 32 * h + l] |= ((u & 3) << (2 * c)).astype(np.uint8)
            out[:, l] |= ((u >> 2) << (4 * h + c)).astype(np.uint8)
        st = sc + 32
        for j in range(16):
            out[:, 96 + (j % 8)] |= ((st[:, j] & 15) << (4 * (j // 8))).astype(np.uint8)
            out[:, 104 + (j % 4)] |= ((st[:, j] >> 4) << (2 * (j // 4))).astype(np.uint8)
        out[:, 108], out[:, 109] = d & 255, d >> 8
        return out, dict(d=d, sc=sc, q=q)
    if codec == "q2_k":
        q = rng.integers(0, 4, size=(nblocks, 256))
        sc = rng.integers(0, 16, size=(nblocks, 16))
        m = rng.integers(0, 16, size=(nblocks, 16))
        d = rng.integers(0, 0x7C00, size=nblocks)
        dm = rng.integers(0, 0x7C00, size=nblocks)
        out = np.zeros((nblocks, 84), np.uint8)
        out[:, 0:16] = (sc | (m << 4)).astype(np.uint8)
        for v in range(256):
            h, r = divmod(v, 128)
            c, l = divmod(r, 32)
            out[:, 16 + 32 * h + l] |= (q[:, v] << (2 * c)).astype(np.uint8)
        out[:, 80], out[:, 81], out[:, 82], out[:, 83] = d & 255, d >> 8, dm & 255, dm >> 8
        return out, dict(d=d, dm=dm, sc=sc, m=m, q=q)
    if codec == "q5_k":
        q = rng.integers(0, 32, size=(nblocks, 256))
        sc = rng.integers(0, 64, size=(nblocks, 8))
        m = rng.integers(0, 64, size=(nblocks, 8))
        d = rng.integers(0, 0x7C00, size=nblocks)
        dm = rng.integers(0, 0x7C00, size=nblocks)
        out = np.zeros((nblocks, 176), np.uint8)
        out[:, 0], out[:, 1], out[:, 2], out[:, 3] = d & 255, d >> 8, dm & 255, dm >> 8
        for j in range(8):  # the 6-bit scale/min packing of q4_K
            if j < 4:
                out[:, 4 + j] |= sc[:, j].astype(np.uint8)
                out[:, 8 + j] |= m[:, j].astype(np.uint8)
            else:
                out[:, 12 + (j - 4)] |= ((sc[:, j] & 15) | ((m[:, j] & 15) << 4)).astype(np.uint8)
                out[:, 4 + (j - 4)] |= ((sc[:, j] >> 4) << 6).astype(np.uint8)
                out[:, 8 + (j - 4)] |= ((m[:, j] >> 4) << 6).astype(np.uint8)
        for v in range(256):
            j, l = divmod(v, 32)
            out[:, 48 + 32 * (j // 2) + l] |= ((q[:, v] & 15) << (4 * (j % 2))).astype(np.uint8)
            out[:, 16 + l] |= ((q[:, v] >> 4) << j).astype(np.uint8)
        return out, dict(d=d, dm=dm, sc=sc, m=m, q=q)
    if codec == "q6_k":
        q = rng.integers(0, 64, size=(nblocks, 256))
        sc = rng.integers(-128, 128, size=(nblocks, 16))
        d = rng.integers(0, 0x7C00, size=nblocks) | (rng.integers(0, 2, size=nblocks) << 15)
        out = np.zeros((nblocks, 210), np.uint8)
        for v in range(256):
            h, r = divmod(v, 128)
            c, l = divmod(r, 32)
            shift = 0 if c < 2 else 4
            out[:, 64 * h + l + 32 * (c & 1)] |= ((q[:, v] & 15) << shift).astype(np.uint8)
            out[:, 128 + 32 * h + l] |= ((q[:, v] >> 4) << (2 * c)).astype(np.uint8)
        out[:, 192:208] = sc & 255
        out[:, 208], out[:, 209] = d & 255, d >> 8
        return out, dict(d=d, sc=sc, q=q)
    raise ValueError(codec)


def _round_to_f32(v: Fraction) -> float:
    """Round an exact dyadic rational to the nearest fp32 (ties to even), by integer arithmetic."""
    if v == 0:
        return 0.0
    sign = -1.0 if v < 0 else 1.0
    v = abs(v)
    num, den = v.numerator, v.denominator
    assert den & (den - 1) == 0, "dyadic"
    e = -(den.bit_length() - 1)
    n = num.bit_length()
    if n > 24:
        shift = n - 24
        keep, rem, half = num >> shift, num & ((1 << shift) - 1), 1 << (shift - 1)
        if rem > half or (rem == half and keep & 1):
            keep += 1
        num, e = keep, e + shift
    return sign * math.ldexp(num, e)


def _affine(codec, f):
    """MLX affine closed form over hand-packed fields: value = scale*code + bias, rounded once to fp32.

    Parameters per codec (the workload's formulas rewritten as affine groups):
      q8_0 : code q+128 (8 bits), scale d,      bias -128 d
      q4_0 : code q (4 bits),     scale d,      bias -8 d
      q4_K : code q (4 bits),     scale d*sc_j, bias -dmin*m_j   (groups of 32)
      q5_K : code q (5 bits),     scale d*sc_j, bias -dmin*m_j   (groups of 32)
      q2_K : code q (2 bits),     scale d*sc_j, bias -dmin*m_j   (groups of 16)
      q3_K : code q+4 (3 bits),   scale d*sc_j, bias -4 d*sc_j   (groups of 16)
      q4_1 : code q (4 bits),     scale d,      bias m
      q5_0 : code q (5 bits),     scale d,      bias -16 d
      q5_1 : code q (5 bits),     scale d,      bias m
      q6_K : code q (6 bits),     scale d*sc_j, bias -32 d*sc_j  (groups of 16)
    Evaluated in exact rational arithmetic, rounded to fp32 at the end.
    """
    half = lambda b: Fraction(float(np.array(b, dtype=np.uint16).view(np.float16)))  # noqa: E731
    rows = []
    for i in range(f["q"].shape[0]):
        if codec == "q8_0":
            d = half(f["d"][i])
            params = [(d, -128 * d, int(q) + 128) for q in f["q"][i]]
        elif codec == "q4_0":
            d = half(f["d"][i])
            params = [(d, -8 * d, int(q)) for q in f["q"][i]]
        elif codec in ("q4_1", "q5_1"):
            d, mm = half(f["d"][i]), half(f["m"][i])
            params = [(d, mm, int(q)) for q in f["q"][i]]
        elif codec == "q5_0":
            d = half(f["d"][i])
            params = [(d, -16 * d, int(q)) for q in f["q"][i]]
        elif codec == "q3_k":
            d = half(f["d"][i])
            params = [(d * int(f["sc"][i][v // 16]), -4 * d * int(f["sc"][i][v // 16]), int(f["q"][i][v]) + 4)
                      for v in range(256)]
        elif codec == "q2_k":
            d, dm = half(f["d"][i]), half(f["dm"][i])
            params = [(d * int(f["sc"][i][v // 16]), -dm * int(f["m"][i][v // 16]), int(f["q"][i][v])) for v in range(256)]
        elif codec in ("q4_k", "q5_k"):
            d, dm = half(f["d"][i]), half(f["dm"][i])
            params = [(d * int(f["sc"][i][v // 32]), -dm * int(f["m"][i][v // 32]), int(f["q"][i][v])) for v in range(256)]
        elif codec == "q6_k":
            d = half(f["d"][i])
            params = [(d * int(f["sc"][i][v // 16]), -32 * d * int(f["sc"][i][v // 16]), int(f["q"][i][v])) for v in range(256)]
        rows.append([_round_to_f32(s * c + b) for s, b, c in params])
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("codec", codecs.CODECS)
def test_hand_packed_codes_decode_to_affine_closed_form(codec):
    rng = np.random.default_rng(123)
    blocks, fields = _hand_pack(codec, rng, 24)
    k = codecs.block_values(codec)
    # fields decoded by the oracle match what was packed
    if codec == "q4_k":
        d, dmin, sc, m, q = codecs.fields_q4_k(blocks[:, None, :])
        assert np.array_equal(sc[:, 0], fields["sc"]) and np.array_equal(m[:, 0], fields["m"])
        assert np.array_equal(q[:, 0].reshape(24, 256), fields["q"])
    elif codec == "q5_k":
        d, dmin, sc, m, q = codecs.fields_q5_k(blocks[:, None, :])
        assert np.array_equal(sc[:, 0], fields["sc"]) and np.array_equal(m[:, 0], fields["m"])
        assert np.array_equal(q[:, 0].reshape(24, 256), fields["q"])
    elif codec == "q3_k":
        d, sc, q = codecs.fields_q3_k(blocks[:, None, :])
        assert np.array_equal(sc[:, 0], fields["sc"]) and np.array_equal(q[:, 0], fields["q"])
    elif codec == "q2_k":
        d, dmin, sc, m, q = codecs.fields_q2_k(blocks[:, None, :])
        assert np.array_equal(sc[:, 0], fields["sc"]) and np.array_equal(m[:, 0], fields["m"])
        assert np.array_equal(q[:, 0], fields["q"])
    elif codec in ("q4_1", "q5_0", "q5_1"):
        d, m, q = codecs.fields_legacy(codec, blocks[:, None, :])
        assert np.array_equal(q[:, 0], fields["q"])
    elif codec == "q6_k":
        d, scales, q = codecs.fields_q6_k(blocks[:, None, :])
        assert np.array_equal(scales[:, 0], fields["sc"]) and np.array_equal(q[:, 0], fields["q"])
    y = codecs.dequantize(codec, blocks, k, np.float32)
    ref = _affine(codec, fields)
    # Values agree exactly (the affine form may give +0 where the codec formula gives -0;
    # the sign of zero is pinned by the golden blocks instead).
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("codec", codecs.CODECS)
def test_f16_output_is_rne_of_f32(codec):
    rng = np.random.default_rng(7)
    blocks, _ = _hand_pack(codec, rng, 32)
    k = codecs.block_values(codec)
    y32 = codecs.dequantize(codec, blocks, k, np.float32)
    y16 = codecs.dequantize(codec, blocks, k, np.float16)
    with np.errstate(over="ignore"):
        ref = y32.astype(np.float16)
    assert np.array_equal(y16.view(np.uint16), ref.view(np.uint16))


def test_q4_k_single_rounding_matters():
    """q4_K's subtraction is the only rounding: a case where rounding d*sc*q first would differ."""
    # d = 2^10 (0x6400), sc = 63, q = 15 -> 967680; dmin = 2^-14 (0x0400), m = 1 -> 2^-14.
    blk = np.zeros((1, 144), np.uint8)
    blk[0, 0:2] = [0x00, 0x64]
    blk[0, 2:4] = [0x00, 0x04]
    blk[0, 4] = 63          # sc_0 = 63
    blk[0, 8] = 1           # m_0 = 1
    blk[0, 16] = 15         # v=0: low nibble 15
    y = codecs.dequantize("q4_k", blk, 256, np.float32)[0, 0]
    exact = 1024.0 * 63 * 15 - 2.0 ** -14
    assert float(y) == float(np.float32(exact))
    assert float(y) == 967680.0  # 2^-14 is below half an ulp of 967680 in fp32


def test_random_wire_bytes_finite_and_exact():
    """Random bytes (finite fp16 headers) decode without tripping the exactness checks."""
    rng = np.random.default_rng(11)
    for codec in codecs.CODECS:
        k = 2 * codecs.block_values(codec)
        w = rng.integers(0, 256, size=(8, codecs.row_bytes(codec, k)), dtype=np.uint8)
        y = codecs.dequantize(codec, w, k)
        assert y.shape == (8, k)
