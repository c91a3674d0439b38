"""Oracle: codec geometry, field decode and per-codec dequantization (CPU, NumPy).

Test infrastructure only (see ``oracle/__init__``). Shares no code with the
HIP path.

What the pages fix
  * mlx-kquant README, "Codec reference" table: q4_k is a 256-value
    superblock of 4-bit codes in 144 bytes; q6_k 256 values, 6 bits, 210
    bytes; q8_0 32 values, 8 bits, 34 bytes ("block scale"); q4_0 32 values,
    4 bits, 18 bytes ("block scale").
  * mlx-kquant ``bindings.cpp`` page, ``dequantize`` docstring: input is
    uint8 wire bytes whose last dim is a multiple of the codec's bytes per
    block; output float dtype defaults to float16.
  * the same table: q5_k is a 256-value superblock of 5-bit codes in 176
    bytes ("K-quant superblock"); q4_1 32 values, 4 bits, 20 bytes ("block
    scale + min"); q5_0 32 values, 5 bits, 22 bytes ("block scale"); q5_1 32
    values, 5 bits, 24 bytes ("block scale + min"); q2_k 256 values, 2 bits,
    84 bytes, and q3_k 256 values, 3 bits, 110 bytes ("K-quant superblock").  Their layouts are not on the pages and
    take reading R1 like the others.
  * The q4_K sub-block structure (8 sub-blocks of 32, 6-bit scale and min per
    sub-block, fp16 d and dmin) and the q6_K one (16 sub-blocks of 16, int8
    scales, fp16 d) are stated with the workloads.

Readings taken where the pages are silent
  R1  Byte layout inside a block: GGUF's (the README acknowledges ggml for the
      formats, the ``load_gguf`` docstring maps GGUF tensors zero-copy, and the
      CPU decoder is described as bit-exact against the ``gguf`` reference
      quantizer).  The offsets are written out in each ``_fields_*`` function.
  R2  fp16 fields are little-endian IEEE binary16, decoded exactly (subnormals
      honoured, the sign of zero kept, inf/NaN passed through).
  R3  Arithmetic: each value is the exact real number of the formula, rounded
      ONCE to fp32 (RNE).  For q8_0, q4_0, q5_0 and q6_K the exact value is
      already an fp32 number, as is q3_K's ``d*sc*q``.  For q2_K, q4_K and
      q5_K the only rounding is
      that of ``(d*sc)*q - (dmin*m)``; for q4_1 and q5_1 that of ``d*q + m`` (exact in
      float64: its bits span at most 2^-24 .. 2^21).
  R4  float16 output is RNE of the fp32 value (so q4_K -> f16 rounds twice, by
      definition).

Pins (tests/test_oracle_codecs.py): the binary16 decode against NumPy's own
float16 for all 65536 bit patterns; hand-decoded superblocks with literal
expected values (tests/golden/*.txt); the MLX affine closed form of the
nuvec-core ``quantized.rs`` module comment as a second decoder over the same
fields; the byte totals of the codec table.
"""

from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# Geometry: mlx-kquant README, "Codec reference" table.
# --------------------------------------------------------------------------

#: codec name -> (values per block, bits per code, bytes per block)
GEOMETRY = {
    "q4_k": (256, 4, 144),
    "q6_k": (256, 6, 210),
    "q8_0": (32, 8, 34),
    "q4_0": (32, 4, 18),
    "q5_k": (256, 5, 176),
    "q4_1": (32, 4, 20),
    "q5_0": (32, 5, 22),
    "q5_1": (32, 5, 24),
    "q2_k": (256, 2, 84),
    "q3_k": (256, 3, 110),
}

CODECS = tuple(GEOMETRY)


def block_values(codec: str) -> int:
    return GEOMETRY[codec][0]


def block_bytes(codec: str) -> int:
    return GEOMETRY[codec][2]


def row_bytes(codec: str, k: int) -> int:
    """Bytes of one weight row of K values (K a multiple of the block size)."""
    bv = block_values(codec)
    if k % bv:
        raise ValueError(f"K={k} is not a multiple of {bv} for {codec}")
    return (k // bv) * block_bytes(codec)


# --------------------------------------------------------------------------
# Field decode (reading R2)
# --------------------------------------------------------------------------


def f16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> exact float64 values, written out.

    sign s, exponent e (5 bits, bias 15), fraction f (10 bits):
      e == 0      : (-1)^s * 2^-14 * f/1024      (zero and subnormals)
      0 < e < 31  : (-1)^s * 2^(e-15) * (1 + f/1024)
      e == 31     : (-1)^s * inf if f == 0 else NaN
    """
    b = np.asarray(bits, dtype=np.uint32)
    s = (b >> 15) & 1
    e = ((b >> 10) & 31).astype(np.int64)
    f = (b & 1023).astype(np.float64)
    sign = np.where(s == 1, -1.0, 1.0)
    normal = sign * np.ldexp(1.0 + f / 1024.0, (e - 15).astype(np.int32))
    sub = sign * np.ldexp(f / 1024.0, -14)
    special = np.where(f == 0, sign * np.inf, np.nan)
    return np.where(e == 0, sub, np.where(e == 31, special, normal))


def le_u16(lo, hi) -> np.ndarray:
    """Two bytes, little-endian, as an unsigned 16-bit integer."""
    return np.asarray(lo, dtype=np.uint32) | (np.asarray(hi, dtype=np.uint32) << 8)


def as_int8(b) -> np.ndarray:
    """A byte read as a two's-complement int8."""
    v = np.asarray(b, dtype=np.int64)
    return np.where(v >= 128, v - 256, v)


def _blocks(w: np.ndarray, codec: str, k: int) -> np.ndarray:
    w = np.asarray(w)
    if w.dtype != np.uint8:
        raise TypeError("wire bytes must be uint8")
    rb = row_bytes(codec, k)
    if w.shape[-1] != rb:
        raise ValueError(f"last dim {w.shape[-1]} != row bytes {rb} for {codec} K={k}")
    n = int(np.prod(w.shape[:-1], dtype=np.int64))
    return w.reshape(n, k // block_values(codec), block_bytes(codec))


# --------------------------------------------------------------------------
# Per-codec field unpacking (reading R1: GGUF byte layout).
# Each returns integer codes and the per-group affine factors as exact
# float64 numbers; ``dequantize`` turns them into values.
# --------------------------------------------------------------------------


def fields_q8_0(blk: np.ndarray):
    """q8_0, 34 bytes: [0:2] d (fp16), [2:34] 32 int8 codes q.  value = d*q."""
    d = f16_bits_to_f64(le_u16(blk[..., 0], blk[..., 1]))  # [n, nb]
    q = as_int8(blk[..., 2:34])  # [n, nb, 32]
    return d, q


def fields_q4_0(blk: np.ndarray):
    """q4_0, 18 bytes: [0:2] d (fp16), [2:18] 16 bytes of nibbles.

    Value v < 16 is the low nibble of byte v; value v >= 16 the high nibble
    of byte v-16.  value = d*(q-8).
    """
    d = f16_bits_to_f64(le_u16(blk[..., 0], blk[..., 1]))
    qs = blk[..., 2:18].astype(np.int64)  # [n, nb, 16]
    q = np.concatenate([qs & 15, qs >> 4], axis=-1)  # [n, nb, 32]
    return d, q


def fields_legacy(codec: str, blk: np.ndarray):
    """q4_1 (20 B: d, m, qs[16]), q5_0 (22 B: d, qh[4], qs[16]), q5_1 (24 B:
    d, m, qh[4], qs[16]); d and m fp16, qh a little-endian uint32.

    Value v < 16 is the low nibble of qs[v], v >= 16 the high nibble of
    qs[v - 16]; for the 5-bit codecs bit v of qh is its fifth bit.
    value = d*q + m (q4_1, q5_1) or d*(q - 16) (q5_0).  Returns d, m (None
    for q5_0) and q [.., 32].
    """
    d = f16_bits_to_f64(le_u16(blk[..., 0], blk[..., 1]))
    m = f16_bits_to_f64(le_u16(blk[..., 2], blk[..., 3])) if codec in ("q4_1", "q5_1") else None
    o = {"q4_1": 4, "q5_0": 6, "q5_1": 8}[codec]
    qs = blk[..., o:o + 16].astype(np.int64)
    q = np.concatenate([qs & 15, qs >> 4], axis=-1)  # [.., 32]
    if codec != "q4_1":
        h = o - 4
        qh = sum(blk[..., h + i].astype(np.int64) << (8 * i) for i in range(4))
        q = q | (((qh[..., None] >> np.arange(32)) & 1) << 4)
    return d, m, q


def scale_min_q4_k(s: np.ndarray):
    """The 12 packed scale bytes of a q4_K superblock -> 8 (sc, m) pairs, 6-bit.

    j < 4 : sc = s[j] & 63,                           m = s[j+4] & 63
    j >= 4: sc = (s[j+4] & 15) | ((s[j-4] >> 6) << 4), m = (s[j+4] >> 4) | ((s[j] >> 6) << 4)
    """
    s = s.astype(np.int64)
    sc = np.empty(s.shape[:-1] + (8,), dtype=np.int64)
    m = np.empty_like(sc)
    for j in range(4):
        sc[..., j] = s[..., j] & 63
        m[..., j] = s[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j - 4] >> 6) << 4)
        m[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return sc, m


def fields_q4_k(blk: np.ndarray):
    """q4_K, 144 bytes: [0:2] d, [2:4] dmin (fp16), [4:16] packed scales, [16:144] qs.

    Value v lies in sub-block j = v // 32; its byte is qs[32*(j//2) + v%32],
    low nibble for even j, high nibble for odd j.
    value = (d*sc_j)*q - (dmin*m_j).
    """
    d = f16_bits_to_f64(le_u16(blk[..., 0], blk[..., 1]))
    dmin = f16_bits_to_f64(le_u16(blk[..., 2], blk[..., 3]))
    sc, m = scale_min_q4_k(blk[..., 4:16])
    qs = blk[..., 16:144].astype(np.int64)  # [n, nb, 128]
    q = np.empty(qs.shape[:-1] + (8, 32), dtype=np.int64)
    for j in range(8):
        byte = qs[..., 32 * (j // 2): 32 * (j // 2) + 32]
        q[..., j, :] = (byte & 15) if j % 2 == 0 else (byte >> 4)
    return d, dmin, sc, m, q  # q: [n, nb, 8, 32]


def fields_q5_k(blk: np.ndarray):
    """q5_K, 176 bytes: [0:2] d, [2:4] dmin (fp16), [4:16] packed scales (as
    q4_K), [16:48] qh, [48:176] qs.

    Value v lies in sub-block j = v // 32 at position l = v % 32: its low four
    bits are the nibble of qs[32*(j//2) + l] (low nibble for even j, high for
    odd j), its fifth bit is bit j of qh[l].
    value = (d*sc_j)*q - (dmin*m_j), q in 0..31.
    """
    d = f16_bits_to_f64(le_u16(blk[..., 0], blk[..., 1]))
    dmin = f16_bits_to_f64(le_u16(blk[..., 2], blk[..., 3]))
    sc, m = scale_min_q4_k(blk[..., 4:16])
    qh = blk[..., 16:48].astype(np.int64)  # [n, nb, 32]
    qs = blk[..., 48:176].astype(np.int64)  # [n, nb, 128]
    q = np.empty(qs.shape[:-1] + (8, 32), dtype=np.int64)
    for j in range(8):
        byte = qs[..., 32 * (j // 2): 32 * (j // 2) + 32]
        low4 = (byte & 15) if j % 2 == 0 else (byte >> 4)
        q[..., j, :] = low4 | (((qh >> j) & 1) << 4)
    return d, dmin, sc, m, q  # q: [n, nb, 8, 32]


def fields_q2_k(blk: np.ndarray):
    """q2_K, 84 bytes: [0:16] scales (sub-block j of 16 values: scale = low
    nibble of byte j, min = high nibble), [16:80] qs, [80:82] d, [82:84] dmin.

    Value v: h = v // 128, c = (v % 128) // 32, l = v % 32; its code is bits
    2c..2c+1 of qs[32h + l].  value = (d*sc_j)*q - (dmin*m_j), j = v // 16.
    """
    sc = (blk[..., 0:16] & 15).astype(np.int64)
    m = (blk[..., 0:16] >> 4).astype(np.int64)
    qs = blk[..., 16:80].astype(np.int64)
    d = f16_bits_to_f64(le_u16(blk[..., 80], blk[..., 81]))
    dmin = f16_bits_to_f64(le_u16(blk[..., 82], blk[..., 83]))
    q = np.empty(qs.shape[:-1] + (256,), dtype=np.int64)
    for v in range(256):
        h, r = divmod(v, 128)
        c, l = divmod(r, 32)
        q[..., v] = (qs[..., 32 * h + l] >> (2 * c)) & 3
    return d, dmin, sc, m, q  # sc, m: [.., 16]; q: [.., 256]


def scales_q3_k(s: np.ndarray) -> np.ndarray:
    """The 12 packed scale bytes of a q3_K superblock -> 16 signed scales.

    Scale j (6 bits, stored with +32): its low four bits are the low nibble of
    s[j] for j < 8 and the high nibble of s[j - 8] for j >= 8; its top two
    bits are bits 2(j // 4) .. 2(j // 4) + 1 of s[8 + j % 4].
    """
    s = s.astype(np.int64)
    out = np.empty(s.shape[:-1] + (16,), dtype=np.int64)
    for j in range(16):
        low4 = (s[..., j] & 15) if j < 8 else (s[..., j - 8] >> 4)
        high2 = (s[..., 8 + j % 4] >> (2 * (j // 4))) & 3
        out[..., j] = (low4 | (high2 << 4)) - 32
    return out


def fields_q3_k(blk: np.ndarray):
    """q3_K, 110 bytes: [0:32] hmask, [32:96] qs, [96:108] packed scales,
    [108:110] d.

    Value v: h = v // 128, c = (v % 128) // 32, l = v % 32; low two bits =
    bits 2c..2c+1 of qs[32h + l], high bit = bit 4h + c of hmask[l]; the code
    is low2 - 4 when the high bit is clear, low2 when it is set (-4..3).
    value = d*sc_j*q, j = v // 16.
    """
    hm = blk[..., 0:32].astype(np.int64)
    qs = blk[..., 32:96].astype(np.int64)
    sc = scales_q3_k(blk[..., 96:108])
    d = f16_bits_to_f64(le_u16(blk[..., 108], blk[..., 109]))
    q = np.empty(qs.shape[:-1] + (256,), dtype=np.int64)
    for v in range(256):
        h, r = divmod(v, 128)
        c, l = divmod(r, 32)
        low2 = (qs[..., 32 * h + l] >> (2 * c)) & 3
        hbit = (hm[..., l] >> (4 * h + c)) & 1
        q[..., v] = low2 - 4 * (1 - hbit)
    return d, sc, q  # sc [.., 16] signed; q [.., 256] in -4..3


def fields_q6_k(blk: np.ndarray):
    """q6_K, 210 bytes: [0:128] ql, [128:192] qh, [192:208] 16 int8 scales, [208:210] d.

    For value v: h = v//128, r = v%128, c = r//32, l = r%32.
      low4  = nibble of ql[64h + l + 32*(c&1)]: low nibble if c < 2 else high
      high2 = (qh[32h + l] >> 2c) & 3
      q     = low4 | high2 << 4             (0..63)
    value = (d*scales[v//16]) * (q - 32).
    """
    ql = blk[..., 0:128].astype(np.int64)
    qh = blk[..., 128:192].astype(np.int64)
    scales = as_int8(blk[..., 192:208])  # [n, nb, 16]
    d = f16_bits_to_f64(le_u16(blk[..., 208], blk[..., 209]))
    q = np.empty(ql.shape[:-1] + (256,), dtype=np.int64)
    for v in range(256):
        h, r = divmod(v, 128)
        c, l = divmod(r, 32)
        byte = ql[..., 64 * h + l + 32 * (c & 1)]
        low4 = (byte & 15) if c < 2 else (byte >> 4)
        high2 = (qh[..., 32 * h + l] >> (2 * c)) & 3
        q[..., v] = low4 | (high2 << 4)
    return d, scales, q


# --------------------------------------------------------------------------
# Dequantize (readings R3, R4)
# --------------------------------------------------------------------------


def _exact_f32(a64: np.ndarray) -> np.ndarray:
    """float64 -> float32 where the value must already be an fp32 number."""
    a32 = a64.astype(np.float32)
    ok = (a32.astype(np.float64) == a64) | np.isnan(a64)
    if not np.all(ok):
        raise AssertionError("value expected to be exact in fp32 is not")
    return a32


def dequantize(codec: str, w: np.ndarray, k: int, dtype=np.float32) -> np.ndarray:
    """Wire bytes [..., row_bytes] -> values [..., K] (float32, or float16 by RNE).

    mlx-kquant ``bindings.cpp`` page, ``dequantize`` docstring.  Each value is
    the exact formula value rounded once to fp32 (reading R3); float16 output
    is the RNE of that fp32 value (reading R4).
    """
    lead = np.asarray(w).shape[:-1]
    blk = _blocks(w, codec, k)
    n, nb = blk.shape[0], blk.shape[1]
    with np.errstate(invalid="ignore", over="ignore"):
        if codec == "q8_0":
            d, q = fields_q8_0(blk)
            y = _exact_f32(d[..., None] * q)
        elif codec == "q4_0":
            d, q = fields_q4_0(blk)
            y = _exact_f32(d[..., None] * (q - 8))
        elif codec == "q6_k":
            d, scales, q = fields_q6_k(blk)
            step = d[..., None] * scales  # [n, nb, 16], exact in float64
            y = _exact_f32(np.repeat(step, 16, axis=-1) * (q - 32))
        elif codec in ("q4_1", "q5_1"):
            d, m, q = fields_legacy(codec, blk)
            y = (d[..., None] * q + m[..., None]).astype(np.float32)  # exact in float64, one rounding
        elif codec == "q5_0":
            d, _, q = fields_legacy(codec, blk)
            y = _exact_f32(d[..., None] * (q - 16))
        elif codec == "q3_k":
            d, sc, q = fields_q3_k(blk)
            y = _exact_f32(np.repeat(d[..., None] * sc, 16, axis=-1) * q)
        elif codec == "q2_k":
            d, dmin, sc, m, q = fields_q2_k(blk)
            step = np.repeat(d[..., None] * sc, 16, axis=-1)  # [n, nb, 256]
            a = _exact_f32(step * q)
            b = _exact_f32(np.repeat(dmin[..., None] * m, 16, axis=-1))
            y = a - b  # float32 - float32: the single IEEE rounding
        elif codec in ("q4_k", "q5_k"):
            d, dmin, sc, m, q = fields_q4_k(blk) if codec == "q4_k" else fields_q5_k(blk)
            a = _exact_f32(d[..., None, None] * sc[..., None] * q)  # (d*sc)*q, exact
            b = _exact_f32(np.broadcast_to((dmin[..., None] * m)[..., None], a.shape))
            y = a - b  # float32 - float32: the single IEEE rounding
        else:
            raise ValueError(f"unknown codec {codec!r}")
    y = np.asarray(y, dtype=np.float32).reshape(n, nb * block_values(codec))
    if dtype == np.float16:
        with np.errstate(over="ignore"):
            y = y.astype(np.float16)  # RNE; beyond 65504 rounds to inf
    elif dtype != np.float32:
        raise ValueError("dtype must be float32 or float16")
    return y.reshape(lead + (k,))
