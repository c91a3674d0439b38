// kq_qmm_impl.h -- the quantized GEMM on gfx950 float16 matrix cores and its
// launchers, shared by the translation units that instantiate its store modes
// (kq_qmm.hip: the plain product and the kq_gather_qmm_seg dispatch;
// kq_qmm_res.hip: residual stores; kq_qmm_glu.hip, kq_qmm_glum.hip: the two
// GLU passes).  K that is not a whole number of 64-value units takes the
// plain kernel at the end of this file.
//
// mlx-kquant bindings.cpp page: quantized_matmul docstring (y = x @ dequant(w)
// transposed, w [N, K]); gather_qmm_seg docstring (expert-sorted rows walked
// tile by tile from a (expert, row_start, num_rows) map with <= 64 rows per
// tile, dead rows of a partial tile skipped, uncovered rows unwritten).
//
// Design.
//  * A workgroup of 8 waves (2 per SIMD, so one wave's decode overlaps the
//    other's matrix work) computes a BM x BN output tile, walking K 64 values
//    (one "unit") per step.  Each step stages the x tile (BM x 64 float16) and
//    DECODES the weight tile (BN rows x 64 values) from wire bytes into LDS as
//    float16; the waves then run v_mfma_f32_16x16x32_f16 with float32
//    accumulators.  LDS is double-buffered and the next step's wire bytes and
//    activations are loaded into registers before the current step's MFMAs,
//    so global latency hides behind matrix work; one barrier per step.
//  * Every decoded weight is rounded to float16 once, from its exact value
//    (q4_K: one float32 FMA, then RNE; q6_K: exact integer code*scale times
//    d; q8_0 / q4_0: d times the code), never through a rounded per-block
//    scale, which would put one correlated error on a whole sub-block.
//  * Within a 64-value step only the agreement of x and W on k matters to
//    the contraction: a q6_K unit's four 16-value segments are not
//    contiguous in K, so x is gathered with the same segment map.
//  * Tiles are ordered so that the workgroups on one XCD (blocks are dealt to
//    the 8 XCDs round-robin) share activation panels in that XCD's L2.
#pragma once

#include <type_traits>

#include "kq_decode.h"

namespace kq {
namespace {

constexpr int BK = 64;
// An LDS tile of R rows x BK values is two planes of R 64-byte rows: 16-byte
// chunk c (of eight per row) of row r sits in plane c & 1 at slot
// (c >> 1) ^ ((r >> 2) & 3) ^ (2 ((r >> 1) & 1)) of its plane row.  Measured
// on gfx950 (probes of lane address patterns, and variants of this kernel,
// against SQ_LDS_BANK_CONFLICT): 16-byte reads are served per 32-lane half
// over sixteen 16-byte bank slots (address / 16 mod 16), lanes 16 apart
// sharing a slot without conflict; 16-byte writes are served 8 lanes at a
// time over 128 bytes.  A fragment read has lane (r, g) take chunk 4 ks + g
// of row r (r < 16): lanes 16 apart read the two planes of one chunk pair, at
// one slot, and each 16-lane group covers all sixteen slots.  A weight store
// has lanes 2q, 2q + 1 write one chunk each of row q: any 8 lanes (4 rows)
// hit 8 distinct slots of 128 bytes.  Planes are 64 R bytes apart, a
// multiple of 256 for R a multiple of 4.
__device__ __forceinline__ int lds_off(int plane, int row, int c) {  // halves
  return (c & 1) * plane + row * 32 + 8 * ((c >> 1) ^ ((row >> 2) & 3) ^ (2 * ((row >> 1) & 1)));
}
struct LdsRow {  // one row of an LDS tile: base, halves per plane, row index
  half_t* tile;
  int plane, row;
};
__device__ __forceinline__ void st_chunk(const LdsRow& d, int c, u32x4 v) {
  *(u32x4*)(d.tile + lds_off(d.plane, d.row, c)) = v;
}
constexpr int NXCD = 8;

// Row offset of segment t (16 values) of unit u.
template <int C>
__device__ __forceinline__ int seg_off(int u, int t) {
  if (C == Q6_K) return 256 * (u >> 2) + 128 * ((u >> 1) & 1) + 32 * t + 16 * (u & 1);
  return 64 * u + 16 * t;
}

__device__ __forceinline__ half2_t h2(half_t a) { return half2_t{a, a}; }

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// 16 bytes at a 2-byte-aligned address: dwords from the dword-aligned address
// below it (never past the 16 bytes), shifted by sh = addr & 3 bytes.
struct Raw16 {
  u32x4 a;
  uint32_t b;
  __device__ __forceinline__ void load(const uint8_t* p, uint32_t sh) {
    const uint8_t* q = p - sh;
    a = ld_16B_a4(q);
    b = ld_u32(q + 16 - (sh ? 0 : 4));
  }
  __device__ __forceinline__ void get(uint32_t sh, uint32_t o[4]) const {
    o[0] = alignbyte(a.y, a.x, sh);
    o[1] = alignbyte(a.z, a.y, sh);
    o[2] = alignbyte(a.w, a.z, sh);
    o[3] = alignbyte(b, a.w, sh);
  }
};

// Half of unit u of one weight row: load() issues its global loads into
// registers, store() decodes them into 32 float16 values: segment t (16
// values) is LDS chunks 2t and 2t+1 of the row at dst (swizzle sw = row & 7).
template <int C> struct HalfUnit;

template <> struct HalfUnit<Q4_K> {
  // half hh: qs bytes 16hh..16hh+15 of sub-block pair P = u%4: positions
  // l in [16hh, 16hh+16) of sub-blocks 2P (low nibbles, segment hh) and 2P+1
  // (high nibbles, segment 2+hh).
  u32x4 h, q;
  __device__ __forceinline__ void load(const uint8_t* row, int u, int hh) {
    const uint8_t* blk = row + (u >> 2) * 144;
    h = ld_16B(blk);
    q = ld_16B(blk + 16 + 32 * (u & 3) + 16 * hh);
  }
  __device__ __forceinline__ void store(int u, int hh, const LdsRow& dst) const {
    const float d = f16_to_f32(h.x), dmin = f16_to_f32(h.x >> 16);
    uint32_t sc0, m0, sc1, m1;
    q4k_scale_min(h.y, h.z, h.w, 2 * (u & 3), sc0, m0);
    q4k_scale_min(h.y, h.z, h.w, 2 * (u & 3) + 1, sc1, m1);
    // Codes come as float16 (1024 + q) from one byte permute per pair; the
    // weight is fma((1024 + q), s, -(1024 s + dmin m)) in float32 (s and
    // dmin m exact, the constant rounded once in float32, about 2^-24 of
    // 1024 s) and rounded once to float16 (v_fma_mix).
    const float s0 = d * (float)sc0, c0 = -(1024.f * s0 + dmin * (float)m0);
    const float s1 = d * (float)sc1, c1 = -(1024.f * s1 + dmin * (float)m1);
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      slice8(qw[2 * i] & 0x0F0F0F0Fu, qw[2 * i + 1] & 0x0F0F0F0Fu, s0, c0, lo + 4 * i);
      slice8((qw[2 * i] >> 4) & 0x0F0F0F0Fu, (qw[2 * i + 1] >> 4) & 0x0F0F0F0Fu, s1, c1, hi + 4 * i);
    }
    st_chunk(dst, 2 * hh, u32x4{lo[0], lo[1], lo[2], lo[3]});
    st_chunk(dst, 2 * hh + 1, u32x4{lo[4], lo[5], lo[6], lo[7]});
    st_chunk(dst, 4 + 2 * hh, u32x4{hi[0], hi[1], hi[2], hi[3]});
    st_chunk(dst, 5 + 2 * hh, u32x4{hi[4], hi[5], hi[6], hi[7]});
  }
};

template <> struct HalfUnit<Q2_K> {
  // unit u' = u % 4 (half h = u' / 2, shifts c0 = 2 (u' % 2), c0 + 1); half
  // hh takes shift c0 + hh: segment 2hh (positions 0..15, sub-block 4u' +
  // 2hh) and 2hh + 1 (16..31, sub-block 4u' + 2hh + 1).
  u32x4 q0, q1;
  uint32_t sc, dd;
  __device__ __forceinline__ void load(const uint8_t* row, int u, int) {
    const uint8_t* blk = row + (u >> 2) * 84;
    const int up = u & 3;
    q0 = ld_16B_a4(blk + 16 + 32 * (up >> 1));
    q1 = ld_16B_a4(blk + 32 + 32 * (up >> 1));
    sc = ld_u32(blk + 4 * up);
    dd = ld_u32(blk + 80);
  }
  __device__ __forceinline__ void store(int u, int hh, const LdsRow& dst) const {
    const float d = f16_to_f32(dd), dmin = f16_to_f32(dd >> 16);
    const int shift = 2 * (2 * (u & 1) + hh);
    const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int g = 0; g < 2; ++g) {  // segment 2hh + g
      const uint32_t b = (sc >> (8 * (2 * hh + g))) & 0xFFu;
      const float s = d * (float)(b & 15u), c = -(1024.f * s + dmin * (float)(b >> 4));
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        slice8((qw[4 * g + 2 * i] >> shift) & 0x03030303u, (qw[4 * g + 2 * i + 1] >> shift) & 0x03030303u, s, c,
               o + 4 * i);
      st_chunk(dst, 4 * hh + 2 * g, u32x4{o[0], o[1], o[2], o[3]});
      st_chunk(dst, 4 * hh + 2 * g + 1, u32x4{o[4], o[5], o[6], o[7]});
    }
  }
};

template <> struct HalfUnit<Q3_K> {
  // unit u' = u % 4 (half h = u' / 2, shifts c0 = 2 (u' % 2), c0 + 1); half
  // hh takes positions l in [16hh, 16hh+16) at both shifts: sub-block 4u' +
  // hh (segment hh) and 4u' + 2 + hh (segment 2 + hh).  110-byte blocks are
  // 2-byte aligned; each span is read from the dword below it and stays in
  // the block (the scales from [92, 108)).
  Raw16 rq, rh, rs;
  uint32_t dbits, sh;
  __device__ __forceinline__ void load(const uint8_t* row, int u, int hh) {
    const uint8_t* blk = row + (u >> 2) * 110;
    sh = (uint32_t)((uintptr_t)blk & 3);
    rq.load(blk + 32 + 32 * ((u >> 1) & 1) + 16 * hh, sh);
    rh.load(blk + 16 * hh, sh);
    rs.load(blk + 92, sh);
    dbits = ld_u16(blk + 108);
  }
  __device__ __forceinline__ void store(int u, int hh, const LdsRow& dst) const {
    const int up = u & 3, h = up >> 1, c0 = 2 * (up & 1);
    uint32_t Q[4], H[4], S[4];
    rq.get(sh, Q); rh.get(sh, H); rs.get(sh, S);
    const float d = f16_to_f32(dbits);
    const uint32_t A = (up & 1) ? S[2] : S[1], B = S[3];
#pragma unroll
    for (int g = 0; g < 2; ++g) {  // shift c0 + g: sub-block 2g + hh, segment 2g + hh
      const float s = d * (float)q3k_scale(A, B, up, 2 * g + hh), c = -1028.f * s;
      const int c2 = c0 + g;
      uint32_t code[4], o[8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        code[i] = ((Q[i] >> (2 * c2)) & 0x03030303u) | (((H[i] >> (4 * h + c2)) & 0x01010101u) << 2);
#pragma unroll
      for (int i = 0; i < 2; ++i) slice8(code[2 * i], code[2 * i + 1], s, c, o + 4 * i);
      st_chunk(dst, 4 * g + 2 * hh, u32x4{o[0], o[1], o[2], o[3]});
      st_chunk(dst, 4 * g + 2 * hh + 1, u32x4{o[4], o[5], o[6], o[7]});
    }
  }
};

template <> struct HalfUnit<Q5_K> {
  // q4_K's half unit with 5-bit codes: the fifth bits of positions l in
  // [16hh, 16hh+16) are bits 2P (sub-block 2P) and 2P + 1 of qh[l].
  u32x4 h, q, e;
  __device__ __forceinline__ void load(const uint8_t* row, int u, int hh) {
    const uint8_t* blk = row + (u >> 2) * 176;
    h = ld_16B(blk);
    e = ld_16B(blk + 16 + 16 * hh);
    q = ld_16B(blk + 48 + 32 * (u & 3) + 16 * hh);
  }
  __device__ __forceinline__ void store(int u, int hh, const LdsRow& dst) const {
    const float d = f16_to_f32(h.x), dmin = f16_to_f32(h.x >> 16);
    uint32_t sc0, m0, sc1, m1;
    q4k_scale_min(h.y, h.z, h.w, 2 * (u & 3), sc0, m0);
    q4k_scale_min(h.y, h.z, h.w, 2 * (u & 3) + 1, sc1, m1);
    // as q4_K: fma((1024 + q), s, -(1024 s + dmin m)) rounded once to float16
    const float s0 = d * (float)sc0, c0 = -(1024.f * s0 + dmin * (float)m0);
    const float s1 = d * (float)sc1, c1 = -(1024.f * s1 + dmin * (float)m1);
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w}, qe[4] = {e.x, e.y, e.z, e.w};
    const int j0 = 2 * (u & 3);
    uint32_t l[4], t[4], lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qhs = qe[i] >> j0;
      l[i] = (qw[i] & 0x0F0F0F0Fu) | ((qhs << 4) & 0x10101010u);
      t[i] = ((qw[i] >> 4) & 0x0F0F0F0Fu) | ((qhs << 3) & 0x10101010u);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      slice8(l[2 * i], l[2 * i + 1], s0, c0, lo + 4 * i);
      slice8(t[2 * i], t[2 * i + 1], s1, c1, hi + 4 * i);
    }
    st_chunk(dst, 2 * hh, u32x4{lo[0], lo[1], lo[2], lo[3]});
    st_chunk(dst, 2 * hh + 1, u32x4{lo[4], lo[5], lo[6], lo[7]});
    st_chunk(dst, 4 + 2 * hh, u32x4{hi[0], hi[1], hi[2], hi[3]});
    st_chunk(dst, 5 + 2 * hh, u32x4{hi[4], hi[5], hi[6], hi[7]});
  }
};

template <> struct HalfUnit<Q6_K> {
  // unit u = (superblock s, h, half); half hh takes c = hh (low nibbles) and
  // c = hh + 2 (high nibbles) of ql[64h + 32hh + 16half + i].
  Raw16 rq, rh, rs;
  uint32_t dbits, sh;
  __device__ __forceinline__ void load(const uint8_t* row, int u, int hh) {
    const uint8_t* blk = row + (u >> 2) * 210;
    const int h = (u >> 1) & 1, half = u & 1;
    sh = (uint32_t)((uintptr_t)blk & 3);
    rq.load(blk + 64 * h + 32 * hh + 16 * half, sh);
    rh.load(blk + 128 + 32 * h + 16 * half, sh);
    rs.load(blk + 192, sh);
    dbits = ld_u16(blk + 208);
  }
  __device__ __forceinline__ void store(int u, int hh, const LdsRow& dst) const {
    const int h = (u >> 1) & 1, half = u & 1;
    uint32_t Q[4], H[4], S[4];
    rq.get(sh, Q);
    rh.get(sh, H);
    rs.get(sh, S);
    // scales[8h + 2c + half]: c = hh in dword 2h (byte half + 2hh), c = hh+2 in dword 2h+1
    const uint32_t slo = h ? S[2] : S[0], shi = h ? S[3] : S[1];
    const int bsh = 8 * (half + 2 * hh);
    // value = ((q - 32) * sc) * d: (q - 32) * sc is an integer of magnitude
    // <= 4096 (exact in float16 up to 2048), so each weight rounds by itself.
    const half2_t sa = h2((half_t)(float)(int)(int8_t)(slo >> bsh));
    const half2_t sb = h2((half_t)(float)(int)(int8_t)(shi >> bsh));
    const half2_t dd = h2(__builtin_bit_cast(half_t, (uint16_t)dbits));
    const half2_t k1056 = h2((half_t)1056.f);
    const int hs = 2 * hh;
    uint32_t a[8], b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ca = (Q[i] & 0x0F0F0F0Fu) | (((H[i] >> hs) << 4) & 0x30303030u);
      const uint32_t cb = ((Q[i] >> 4) & 0x0F0F0F0Fu) | (((H[i] >> (hs + 4)) << 4) & 0x30303030u);
      a[2 * i] = as_u32(((as_h2(pair01(ca)) - k1056) * sa) * dd);
      a[2 * i + 1] = as_u32(((as_h2(pair23(ca)) - k1056) * sa) * dd);
      b[2 * i] = as_u32(((as_h2(pair01(cb)) - k1056) * sb) * dd);
      b[2 * i + 1] = as_u32(((as_h2(pair23(cb)) - k1056) * sb) * dd);
    }
    st_chunk(dst, 2 * hh, u32x4{a[0], a[1], a[2], a[3]});
    st_chunk(dst, 2 * hh + 1, u32x4{a[4], a[5], a[6], a[7]});
    st_chunk(dst, 2 * hh + 4, u32x4{b[0], b[1], b[2], b[3]});
    st_chunk(dst, 2 * hh + 5, u32x4{b[4], b[5], b[6], b[7]});
  }
};

template <> struct HalfUnit<Q8_0> {
  // unit u = two blocks at 68u; half hh = block hh (34 bytes) -> segments 2hh, 2hh+1.
  // Nine dwords from the dword below the block cover it (sh = 0 or 2).
  u32x4 r0, r1;
  uint32_t r8, sh;
  __device__ __forceinline__ void load(const uint8_t* row, int u, int hh) {
    const uint8_t* p = row + 68 * u + 34 * hh;
    sh = (uint32_t)((uintptr_t)p & 3);
    const uint8_t* a = p - sh;
    r0 = ld_16B_a4(a);
    r1 = ld_16B_a4(a + 16);
    r8 = ld_u32(a + 32);
  }
  __device__ __forceinline__ void store(int, int hh, const LdsRow& dst) const {
    const uint32_t R[9] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w, r8};
    const half2_t d = h2(__builtin_bit_cast(half_t, (uint16_t)(sh ? (R[0] >> 16) : (R[0] & 0xFFFFu))));
    const half2_t k1152 = h2((half_t)1152.f);
    uint32_t o[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = (sh ? R[i + 1] : alignbyte(R[i + 1], R[i], 2)) ^ 0x80808080u;
      o[2 * i] = as_u32((as_h2(pair01(c)) - k1152) * d);  // exact code, one rounding
      o[2 * i + 1] = as_u32((as_h2(pair23(c)) - k1152) * d);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) st_chunk(dst, 4 * hh + i, u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]});
  }
};

template <> struct HalfUnit<Q4_0> {
  // unit u = two blocks at 36u; half hh = block hh (18 bytes): low nibbles are
  // values 0..15 (segment 2hh), high nibbles 16..31 (segment 2hh+1).
  u32x4 r0;
  uint32_t r4, sh;
  __device__ __forceinline__ void load(const uint8_t* row, int u, int hh) {
    const uint8_t* p = row + 36 * u + 18 * hh;
    sh = (uint32_t)((uintptr_t)p & 3);
    const uint8_t* a = p - sh;
    r0 = ld_16B_a4(a);
    r4 = ld_u32(a + 16);
  }
  __device__ __forceinline__ void store(int, int hh, const LdsRow& dst) const {
    const uint32_t R[5] = {r0.x, r0.y, r0.z, r0.w, r4};
    const half2_t d = h2(__builtin_bit_cast(half_t, (uint16_t)(sh ? (R[0] >> 16) : (R[0] & 0xFFFFu))));
    const half2_t k1032 = h2((half_t)1032.f);
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t q = sh ? R[i + 1] : alignbyte(R[i + 1], R[i], 2);
      const uint32_t l = q & 0x0F0F0F0Fu, t = (q >> 4) & 0x0F0F0F0Fu;
      lo[2 * i] = as_u32((as_h2(pair01(l)) - k1032) * d);
      lo[2 * i + 1] = as_u32((as_h2(pair23(l)) - k1032) * d);
      hi[2 * i] = as_u32((as_h2(pair01(t)) - k1032) * d);
      hi[2 * i + 1] = as_u32((as_h2(pair23(t)) - k1032) * d);
    }
    st_chunk(dst, 4 * hh, u32x4{lo[0], lo[1], lo[2], lo[3]});
    st_chunk(dst, 4 * hh + 1, u32x4{lo[4], lo[5], lo[6], lo[7]});
    st_chunk(dst, 4 * hh + 2, u32x4{hi[0], hi[1], hi[2], hi[3]});
    st_chunk(dst, 4 * hh + 3, u32x4{hi[4], hi[5], hi[6], hi[7]});
  }
};

// q4_1, q5_0, q5_1: half hh = block hh (low nibbles values 0..15, segment
// 2hh; high nibbles 16..31, segment 2hh+1).  The block's dwords are read from
// the dword-aligned address below it (q5_0's odd block sits 2 bytes past one:
// sh = 2); NWB dwords cover it without reading past the unit.
template <int C>
struct HalfUnitLeg {
  using L = Leg<C>;
  static constexpr int NWB = L::BB % 4 ? (L::BB + 2 + 3) / 4 : L::BB / 4;
  uint32_t R[NWB];
  uint32_t sh;
  __device__ __forceinline__ void load(const uint8_t* row, int u, int hh) {
    const uint8_t* p = row + 2 * L::BB * u + L::BB * hh;
    sh = L::BB % 4 ? (uint32_t)((uintptr_t)p & 3) : 0u;
    const uint8_t* a = p - sh;
#pragma unroll
    for (int i = 0; i < NWB; ++i) R[i] = ld_u32(a + 4 * i);
  }
  // the 4 bytes at block byte offset O (even)
  template <int O>
  __device__ __forceinline__ uint32_t at() const {
    if constexpr (L::BB % 4 == 0) {
      if constexpr (O % 4 == 0) return R[O / 4];
      else return alignbyte(R[O / 4 + 1], R[O / 4], 2);
    } else if constexpr (O % 4 == 0) {
      return sh ? alignbyte(R[O / 4 + 1], R[O / 4], 2) : R[O / 4];
    } else {
      return sh ? R[(O + 2) / 4] : alignbyte(R[O / 4 + 1], R[O / 4], 2);
    }
  }
  __device__ __forceinline__ void store(int, int hh, const LdsRow& dst) const {
    constexpr int qso = L::QS, qho = L::QH >= 0 ? L::QH : 0;
    const uint32_t w0 = at<0>();
    const uint32_t qh = L::QH >= 0 ? at<qho>() : 0u;
    const uint32_t q[4] = {at<qso>(), at<qso + 4>(), at<qso + 8>(), at<qso + 12>()};
    uint32_t lo[8], hi[8];
    if constexpr (L::MIN) {
      // fma((1024 + q), d, m - 1024 d) in float32, rounded once to float16
      const float d = f16_to_f32(w0), c = fmaf(-1024.f, d, f16_to_f32(w0 >> 16));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        slice8(leg_lo<C>(q[2 * i], qh, 2 * i), leg_lo<C>(q[2 * i + 1], qh, 2 * i + 1), d, c, lo + 4 * i);
        slice8(leg_hi<C>(q[2 * i], qh, 2 * i), leg_hi<C>(q[2 * i + 1], qh, 2 * i + 1), d, c, hi + 4 * i);
      }
    } else {
      // (1024 + q - 1024 - ZP) is the exact code; times d, one rounding
      const half2_t d = h2(__builtin_bit_cast(half_t, (uint16_t)(w0 & 0xFFFFu)));
      const half2_t k = h2((half_t)(1024.f + L::ZP));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t l = leg_lo<C>(q[i], qh, i), t = leg_hi<C>(q[i], qh, i);
        lo[2 * i] = as_u32((as_h2(pair01(l)) - k) * d);
        lo[2 * i + 1] = as_u32((as_h2(pair23(l)) - k) * d);
        hi[2 * i] = as_u32((as_h2(pair01(t)) - k) * d);
        hi[2 * i + 1] = as_u32((as_h2(pair23(t)) - k) * d);
      }
    }
    st_chunk(dst, 4 * hh, u32x4{lo[0], lo[1], lo[2], lo[3]});
    st_chunk(dst, 4 * hh + 1, u32x4{lo[4], lo[5], lo[6], lo[7]});
    st_chunk(dst, 4 * hh + 2, u32x4{hi[0], hi[1], hi[2], hi[3]});
    st_chunk(dst, 4 * hh + 3, u32x4{hi[4], hi[5], hi[6], hi[7]});
  }
};
template <> struct HalfUnit<Q4_1> : HalfUnitLeg<Q4_1> {};
template <> struct HalfUnit<Q5_0> : HalfUnitLeg<Q5_0> {};
template <> struct HalfUnit<Q5_1> : HalfUnitLeg<Q5_1> {};

constexpr int QMM_THREADS = 512;

// Tile of the (tiles_m x nb, n fastest) grid run by this block: block b runs
// on XCD b % 8, and XCD x takes the contiguous tile range
// [x * per_xcd, (x+1) * per_xcd), so its workgroups share x panels in its L2.
__device__ __forceinline__ int xcd_tile(int per_xcd) {
  return (int)(blockIdx.x % NXCD) * per_xcd + (int)(blockIdx.x / NXCD);
}

constexpr int gcd_c(int a, int b) { return b ? gcd_c(b, a % b) : a; }
constexpr int lcm_c(int a, int b) { return a / gcd_c(a, b) * b; }

// PDA / PDB: prefetch distances in K-steps for activations and weights.  The
// loads for step s are issued at the start of step s - PD into register slot
// s % PD, stored (weights: decoded) to LDS buffer s % 2 during step s - 1, and
// consumed by the MFMAs of step s.  Activations come from L2 (their panel is
// shared by the tiles of one XCD) and need a shorter distance than weights.
//
// EP / ACT / epi: the output store (store_out: plain, the residual epilogue,
// or one of the two passes of the GLU product).
template <int C, int BM, int BN, int WM, int WN, int PDA, int PDB, bool F16, int EP = EP_PLAIN, int ACT = 0>
__global__ __launch_bounds__(QMM_THREADS) void qmm_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                          int64_t row_bytes, const half_t* __restrict__ x, int m_total,
                                                          int tiles_total, int per_xcd, void* __restrict__ y,
                                                          Epi epi) {
  static_assert(WM * WN == QMM_THREADS / 64, "8 waves");
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int TM = WTM / 16, TN = WTN / 16;  // 16x16 MFMA tiles per wave
  static_assert(TM >= 1 && TN >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
  static_assert(PDA >= 1 && PDB >= 1, "prefetch distance");
  constexpr int A_CHUNKS = BM * 8, A_PER_T = (A_CHUNKS + QMM_THREADS - 1) / QMM_THREADS;
  constexpr int B_HALVES = BN * 2, B_PER_T = (B_HALVES + QMM_THREADS - 1) / QMM_THREADS;
  constexpr int UNR = lcm_c(lcm_c(PDA, PDB), 2);
  __shared__ __attribute__((aligned(16))) half_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) half_t Bs[2][BN * BK];
  static_assert(BM % 4 == 0 && BN % 4 == 0, "planes 256-byte aligned");

  const int t = xcd_tile(per_xcd);
  if (t >= tiles_total) return;
  const int nb = (n + BN - 1) / BN;
  const int by = t / nb;
  const int n0 = (t - by * nb) * BN;
  const int m0 = by * BM;
  const int mrows = min(BM, m_total - m0);
  const uint8_t* wbase = w;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int wr0 = wm * WTM, wc0 = wn * WTN;
  // 16-row fragments of this wave that hold live rows (the rest skip their MFMAs)
  const int live_tm = min(TM, max(0, (mrows - wr0 + 15) / 16));

  float4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  u32x4 areg[PDA][A_PER_T];
  HalfUnit<C> braw[PDB][B_PER_T];

  // Activation chunks: 8 per tile row (4 segments x 2 halves of 8 values).
  // Chunk index c (thread + i x threads) takes row 8 (c >> 6) + 4 ((c >> 5) & 1)
  // + ((c & 15) >> 2) and chunk 2 (c & 3) + ((c >> 4) & 1): the 64 lanes of a
  // wave write 8 rows, and lanes 16 apart the two planes of one chunk pair.
  // Rows past the tile read a clamped valid row; their outputs are never
  // stored, so no predicate sits in the K loop.
  auto a_row = [](int c) { return 8 * (c >> 6) + 4 * ((c >> 5) & 1) + ((c & 15) >> 2); };
  auto a_part = [](int c) { return 2 * (c & 3) + ((c >> 4) & 1); };
  const half_t* xrow[A_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int c = min(tid + i * QMM_THREADS, A_CHUNKS - 1);
    xrow[i] = x + (int64_t)min(m0 + a_row(c), m_total - 1) * k + 8 * (a_part(c) & 1);
  }
  // Weight half-units: wave w decodes rows [w * RPW, (w+1) * RPW), two lanes
  // (halves) per row, so every wave has the same decode work.  Spare lanes
  // decode the wave's last row again but do not store it: several lanes
  // writing one LDS address serialize (SQ_LDS_BANK_CONFLICT).  Rows past N
  // read a clamped valid row (finite values, outputs never stored).
  constexpr int RPW = BN / 8;  // rows per wave
  static_assert(BN % 8 == 0 && 2 * RPW <= 64 && B_PER_T == 1, "one half-unit per lane");
  const int brow0 = wave * RPW + min(lane >> 1, RPW - 1);
  const uint8_t* const wrow0 = wbase + (int64_t)min(n0 + brow0, n - 1) * row_bytes;

  auto issue_a = [&](int slot, int u) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int part = a_part(tid + i * QMM_THREADS);
      areg[slot][i] = *(const u32x4*)(xrow[i] + seg_off<C>(u, part >> 1));
    }
  };
  auto issue_b = [&](int slot, int u) __attribute__((always_inline)) { braw[slot][0].load(wrow0, u, lane & 1); };
  auto stage = [&](int sa, int sb, int buf, int u) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int c = tid + i * QMM_THREADS;
      if (A_CHUNKS % QMM_THREADS == 0 || c < A_CHUNKS) {
        st_chunk(LdsRow{As[buf], BM * 32, a_row(c)}, a_part(c), areg[sa][i]);
      }
    }
    if (lane < 2 * RPW) braw[sb][0].store(u, lane & 1, LdsRow{Bs[buf], BN * 32, brow0});
  };
  // Fragment reads.  A step's first 32-wide K slice reads all its fragments
  // before its MFMAs, in the order the MFMAs consume them.  Every later slice's
  // fragments are read into the registers of the slice before, right after
  // their last use there: A fragment i once row group i's products have
  // issued, B fragment j once the last row group's product with it has.  So
  // that slice's LDS latency runs under the rest of the slice before, with
  // no extra registers.  Full tiles take a copy without the dead-fragment
  // test.
  const int fr = lane & 15, fc = lane >> 4;
  auto rd_a = [&](half8_t& d, int buf, int ks, int i) __attribute__((always_inline)) {
    d = *(const half8_t*)(As[buf] + lds_off(BM * 32, wr0 + 16 * i + fr, 4 * ks + fc));
  };
  auto rd_b = [&](half8_t& d, int buf, int ks, int j) __attribute__((always_inline)) {
    d = *(const half8_t*)(Bs[buf] + lds_off(BN * 32, wc0 + 16 * j + fr, 4 * ks + fc));
  };
  auto mfma_steps = [&](int buf, auto full) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full)::value;
    constexpr int NKS = BK / 32;
    half8_t a[TM], b[TN];
    rd_a(a[0], buf, 0, 0);
#pragma unroll
    for (int j = 0; j < TN; ++j) rd_b(b[j], buf, 0, j);
#pragma unroll
    for (int i = 1; i < TM; ++i) rd_a(a[i], buf, 0, i);
    asm volatile("" ::: "memory");  // keep every read above the MFMAs (the scheduler would sink them)
    static_for<NKS>([&](auto kc) __attribute__((always_inline)) {
      constexpr int ks = decltype(kc)::value;
      constexpr bool more = ks + 1 < NKS;
      static_for<TM>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const bool live = FULL || i < live_tm;
        static_for<TN>([&](auto jc) __attribute__((always_inline)) {
          constexpr int j = decltype(jc)::value;
          if (live) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
          if constexpr (more && i == TM - 1) {
            __builtin_amdgcn_sched_barrier(0);
            rd_b(b[j], buf, ks + 1, j);
            __builtin_amdgcn_sched_barrier(0);
          }
        });
        if constexpr (more) {
          __builtin_amdgcn_sched_barrier(0);
          rd_a(a[i], buf, ks + 1, i);
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    });
  };
  const bool full_rows = live_tm == TM;
  auto mfma_step = [&](int buf) __attribute__((always_inline)) {
    if (full_rows)
      mfma_steps(buf, std::true_type{});
    else
      mfma_steps(buf, std::false_type{});
  };

  // Waves w and w+4 share a SIMD: the first four stage the next step before
  // their MFMAs, the other four after, so one wave's decode runs while its
  // partner's MFMAs occupy the matrix unit.  The steady-state loop body has no
  // branches (step indices are clamped instead: a clamped extra load or stage
  // is harmless), so the compiler keeps PD steps of loads in flight.
  const int units = k / BK;
  const int last = units - 1;
#pragma unroll
  for (int s = 0; s < PDA; ++s) issue_a(s, min(s, last));
#pragma unroll
  for (int s = 0; s < PDB; ++s) issue_b(s, min(s, last));
  stage(0, 0, 0, 0);
  __syncthreads();
  const int units_main = units - units % UNR;
  auto kloop = [&](auto sf) __attribute__((always_inline)) {
    constexpr bool SF = decltype(sf)::value;
    for (int u0 = 0; u0 < units_main; u0 += UNR) {
#pragma unroll
      for (int du = 0; du < UNR; ++du) {
        const int u = u0 + du;
        issue_a(du % PDA, min(u + PDA, last));
        issue_b(du % PDB, min(u + PDB, last));
        if (SF) stage((du + 1) % PDA, (du + 1) % PDB, (du + 1) & 1, min(u + 1, last));
        mfma_step(du & 1);
        if (!SF) stage((du + 1) % PDA, (du + 1) % PDB, (du + 1) & 1, min(u + 1, last));
        __syncthreads();
      }
    }
    // leftover steps (units not a multiple of UNR): slot = du % PD still holds
    // because units_main is a multiple of both distances
#pragma unroll
    for (int du = 0; du < UNR; ++du) {
      const int u = units_main + du;
      if (u < units) {
        issue_a(du % PDA, min(u + PDA, last));
        issue_b(du % PDB, min(u + PDB, last));
        if (SF) stage((du + 1) % PDA, (du + 1) % PDB, (du + 1) & 1, min(u + 1, last));
        mfma_step(du & 1);
        if (!SF) stage((du + 1) % PDA, (du + 1) % PDB, (du + 1) & 1, min(u + 1, last));
        __syncthreads();
      }
    }
  };
  if (wave < 4)
    kloop(std::true_type{});
  else
    kloop(std::false_type{});

  // 16x16 accumulator layout: lane holds column (lane & 15); register r holds
  // row 4*(lane/16) + r.
  static_assert(EP != EP_EPI, "the GEMM tile stores take EP_RES / EP_RES_GATE");
  if constexpr (EP == EP_PLAIN || EP == EP_GLU_ACT) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= live_tm) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wc0 + 16 * j + (lane & 15);
        if (col >= n) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wr0 + 16 * i + 4 * (lane >> 4) + r;
          if (row < mrows) store_out<F16, EP, ACT>(y, m0 + row, col, n, epi, acc[i][j][r]);
        }
      }
    }
  } else {
    // stores that read: each 16-row group's inputs are loaded before its
    // stores, unconditionally (indices clamped into the tile; a clamped
    // element's value is never used), so the loads overlap instead of each
    // waiting behind a branch
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i >= live_tm) continue;
      float pa[TN][4], pb[TN][4];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = min(n0 + wc0 + 16 * j + (lane & 15), n - 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = min(wr0 + 16 * i + 4 * (lane >> 4) + r, mrows - 1);
          pa[j][r] = 0.f;
          pb[j][r] = 1.f;
          epi_load<F16, EP>(y, m0 + row, col, n, epi, pa[j][r], pb[j][r]);
        }
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wc0 + 16 * j + (lane & 15);
        if (col >= n) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wr0 + 16 * i + 4 * (lane >> 4) + r;
          if (row < mrows) store_pre<F16, EP, ACT>(y, m0 + row, col, n, epi, acc[i][j][r], pa[j][r], pb[j][r]);
        }
      }
    }
  }
}

template <int C, int BM, int BN, int WM, int WN, int PDA, int PDB, int EP, int ACT>
hipError_t launch_t(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int64_t m, void* y, int f16,
                    const Epi& epi, hipStream_t s) {
  const int64_t tiles_m = (m + BM - 1) / BM;
  const int64_t tiles = tiles_m * ((n + BN - 1) / BN);
  const int64_t per_xcd = (tiles + NXCD - 1) / NXCD;
  const dim3 grid((unsigned)(per_xcd * NXCD));
  if (f16)
    hipLaunchKernelGGL((qmm_kernel<C, BM, BN, WM, WN, PDA, PDB, true, EP, ACT>), grid, dim3(QMM_THREADS), 0, s, w,
                       (int)n, (int)k, rb, x, (int)m, (int)tiles, (int)per_xcd, y, epi);
  else
    hipLaunchKernelGGL((qmm_kernel<C, BM, BN, WM, WN, PDA, PDB, false, EP, ACT>), grid, dim3(QMM_THREADS), 0, s, w,
                       (int)n, (int)k, rb, x, (int)m, (int)tiles, (int)per_xcd, y, epi);
  return hipGetLastError();
}

template <int C, int EP, int ACT>
hipError_t launch_dense(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int64_t m, void* y,
                        int f16, const Epi& epi, hipStream_t s) {
  // prefill: 256 x 224 tiles (N = 14336 gives 64 tile columns) while they
  // give every CU at least one; fewer (N = 4096: 152) leave CUs idle for the
  // whole K walk, and 128 x 256 tiles fill them
  // Below that, with one M tile (M <= 128), 64-column tiles (four times the
  // tiles of 256 columns) keep the CUs busy when N / 256 tiles cannot: q4_K
  // 14336 x 4096, M = 32 .. 128 measured 49 .. 53 us against 56 .. 82 us.
  // With two M tiles they were slower (M = 192, 256: 87 us against 80).
  constexpr int64_t kCUs = 256;
  if (m > 128 && ((m + 255) / 256) * ((n + 223) / 224) >= kCUs)
    return launch_t<C, 256, 224, 4, 2, 1, 2, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
  const bool narrow = ((m + 127) / 128) * ((n + 255) / 256) < kCUs;
  if (m > 64) {
    if (narrow && m <= 128) return launch_t<C, 128, 64, 4, 2, 2, 4, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
    return launch_t<C, 128, 256, 2, 4, 2, 3, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
  }
  if (narrow) return launch_t<C, 64, 64, 2, 4, 2, 4, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
  return launch_t<C, 64, 256, 2, 4, 2, 4, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
}

template <int C, bool SEG, bool F16, int EP = EP_PLAIN, int ACT = 0>
__global__ __launch_bounds__(256) void qmm_generic_kernel(const uint8_t* __restrict__ w, int n, int k, int64_t rb,
                                                          int64_t estride, int n_experts, const half_t* __restrict__ x,
                                                          int m_total, const uint32_t* __restrict__ map,
                                                          const uint32_t* __restrict__ counts, void* __restrict__ y,
                                                          Epi epi) {
  const int lane = threadIdx.x & 63;
  const int nb = (n + 3) / 4;
  const int by = (int)(blockIdx.x / nb);
  const int col = (int)(blockIdx.x % nb) * 4 + (threadIdx.x >> 6);
  if (col >= n) return;
  int r0, r1;
  const uint8_t* wb = w;
  if (SEG) {
    const int tile = by;
    if (tile >= (int)counts[0]) return;
    const uint32_t* mt = map + 3 * (size_t)tile;
    const uint32_t e = mt[0], rs = mt[1], nr = mt[2];
    if (e >= (uint32_t)n_experts || nr == 0 || nr > 64 || rs >= (uint32_t)m_total || nr > (uint32_t)m_total - rs)
      return;
    r0 = (int)rs; r1 = (int)(rs + nr);
    wb = w + (int64_t)e * estride;
  } else {
    r0 = by * 64;
    r1 = min(m_total, r0 + 64);
  }
  const uint8_t* wrow = wb + (int64_t)col * rb;
  for (int r = r0; r < r1; ++r) {
    float acc = 0.f;
    for (int g = lane; g < k / 8; g += 64) {
      float v[8];
      decode8<C>(wrow, (int64_t)g * 8, v);
      const half8_t xv = *(const half8_t*)(x + (int64_t)r * k + 8 * g);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += v[i] * (float)xv[i];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) store_out<F16, EP, ACT>(y, r, col, n, epi, acc);
  }
}

template <int C, bool SEG, int EP = EP_PLAIN, int ACT = 0>
hipError_t launch_generic(const uint8_t* w, int64_t n, int64_t k, int64_t rb, int64_t estride, int64_t ne,
                          const half_t* x, int64_t m, const uint32_t* map, const uint32_t* counts, int64_t gy, void* y,
                          int f16, hipStream_t s, const Epi& epi = Epi{nullptr, nullptr, nullptr, 1}) {
  const dim3 grid((unsigned)(((n + 3) / 4) * gy));
  if (f16)
    hipLaunchKernelGGL((qmm_generic_kernel<C, SEG, true, EP, ACT>), grid, dim3(256), 0, s, w, (int)n, (int)k, rb,
                       estride, (int)ne, x, (int)m, map, counts, y, epi);
  else
    hipLaunchKernelGGL((qmm_generic_kernel<C, SEG, false, EP, ACT>), grid, dim3(256), 0, s, w, (int)n, (int)k, rb,
                       estride, (int)ne, x, (int)m, map, counts, y, epi);
  return hipGetLastError();
}

// One GEMM pass with output store EP: the matrix-core kernel for K a whole
// number of 64-value units, else the plain kernel (q4_0 / q8_0 only).
template <int EP, int ACT>
hipError_t launch_pass(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int64_t m,
                       void* y, int f16, const Epi& epi, hipStream_t s) {
  if (k % 64 != 0) {
    const int64_t gy = (m + 63) / 64;
    switch (codec) {
      case Q4_0: return launch_generic<Q4_0, false, EP, ACT>(w, n, k, rb, 0, 1, x, m, nullptr, nullptr, gy, y, f16, s, epi);
      case Q8_0: return launch_generic<Q8_0, false, EP, ACT>(w, n, k, rb, 0, 1, x, m, nullptr, nullptr, gy, y, f16, s, epi);
      case Q4_1: return launch_generic<Q4_1, false, EP, ACT>(w, n, k, rb, 0, 1, x, m, nullptr, nullptr, gy, y, f16, s, epi);
      case Q5_0: return launch_generic<Q5_0, false, EP, ACT>(w, n, k, rb, 0, 1, x, m, nullptr, nullptr, gy, y, f16, s, epi);
      case Q5_1: return launch_generic<Q5_1, false, EP, ACT>(w, n, k, rb, 0, 1, x, m, nullptr, nullptr, gy, y, f16, s, epi);
    }
    return hipErrorInvalidValue;
  }
  switch (codec) {
    case Q4_0: return launch_dense<Q4_0, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
    case Q8_0: return launch_dense<Q8_0, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
    case Q4_1: return launch_dense<Q4_1, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
    case Q5_0: return launch_dense<Q5_0, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
    case Q5_1: return launch_dense<Q5_1, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
    case Q2_K: return launch_dense<Q2_K, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
    case Q3_K: return launch_dense<Q3_K, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
    case Q4_K: return launch_dense<Q4_K, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
    case Q5_K: return launch_dense<Q5_K, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
    case Q6_K: return launch_dense<Q6_K, EP, ACT>(w, n, k, rb, x, m, y, f16, epi, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace kq
