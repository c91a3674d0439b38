// kq_units.h -- 64-value weight units shared by the GEMV kernels and the
// expert-segment matrix-core kernel: the loads of one unit's wire bytes, its
// v_dot2 product with float16 activations (GEMV, M <= 8), and its eight
// 8-value float16 MFMA operand slices.
//
// Byte layouts per the codec table of the mlx-kquant README (block geometry)
// read as GGUF's layouts (a unit is whole blocks or whole sub-blocks).
#pragma once

#include "kq_decode.h"

namespace kq {
namespace {

__host__ __device__ constexpr int xpad(int v) { return v + (v >> 6) * 8; }  // padded LDS offset (halves)

// Where the GEMV kernels stage activation value v of a chunk (before the
// padding): in order, except for q6_K, whose 64-value units each take four
// 16-value segments 32 values apart.  For q6_K the segments are put in unit
// order (segment (cc, f) of a 128-value half, value 32 cc + 16 f of it, at
// 64 f + 16 cc), so a unit's 64 values are contiguous: 16 lanes reading one
// segment of 16 consecutive units then hit 16 different LDS bank slots (in
// place order they hit only the even ones), and its four 16-value sums are one
// aligned 16-byte read.
template <int C>
__host__ __device__ constexpr int xperm(int v) {
  if (C == Q6_K) return (v & ~127) | (((v >> 4) & 1) << 6) | (((v >> 5) & 3) << 4) | (v & 15);
  return v;
}

// ---------------------------------------------------------------------------
// Buffer loads: a wave-uniform base and byte count in a resource descriptor,
// a per-lane offset that stays fixed across the K loop, and a wave-uniform
// offset that moves with it.  Bytes past the count read as zero.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t nb = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)(uint32_t)nb, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bld4(rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bld2(rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// ---------------------------------------------------------------------------
// Units.  load(row, u): issue the loads of unit u of a row.
// dot<M>(...): accumulate the unit's v_dot2 product into acc[0..M).
// ---------------------------------------------------------------------------

struct Xv {  // activation views for one chunk
  const half_t* xs;  // LDS [M][xpad(kc)]
  const float* xsum; // LDS [M][kc/16]
  int xstride, sstride, c0;
  __device__ __forceinline__ const uint32_t* pairs(int m, int off) const {  // off: row offset, multiple of 16
    return (const uint32_t*)(xs + m * xstride + xpad(off - c0));
  }
  __device__ __forceinline__ float sum16(int m, int off) const { return xsum[m * sstride + ((off - c0) >> 4)]; }
  // the four 16-value sums from staged position off (a multiple of 64)
  __device__ __forceinline__ float4_t sum64(int m, int off) const {
    return *(const float4_t*)(xsum + m * sstride + ((off - c0) >> 4));
  }
};

// sum over 16 values: (float16 pairs of codes) . (x pairs), 4 code dwords (p01, p23 per dword)
__device__ __forceinline__ float dot16(const uint32_t* cp /*8 pairs*/, const uint32_t* xp, float s) {
  const u32x4 a = *(const u32x4*)xp, b = *(const u32x4*)(xp + 4);
  s = dot2(cp[0], a.x, s); s = dot2(cp[1], a.y, s); s = dot2(cp[2], a.z, s); s = dot2(cp[3], a.w, s);
  s = dot2(cp[4], b.x, s); s = dot2(cp[5], b.y, s); s = dot2(cp[6], b.z, s); s = dot2(cp[7], b.w, s);
  return s;
}

// 4 code-byte dwords (16 codes) -> 8 float16 pairs (1024 + code)
__device__ __forceinline__ void pairs16(const uint32_t c[4], uint32_t p[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { p[2 * i] = pair01(c[i]); p[2 * i + 1] = pair23(c[i]); }
}

struct UnitQ4K {
  u32x4 h, q0, q1;
  __device__ __forceinline__ void load(const uint8_t* row, int u) {
    const uint8_t* blk = row + (u >> 2) * 144;
    h = ld_16B(blk);
    const uint8_t* qs = blk + 16 + 32 * (u & 3);
    q0 = ld_16B(qs);
    q1 = ld_16B(qs + 16);
  }
  // unit u4 + cu of the row at byte rowoff (u4 a multiple of 4, wave-uniform)
  __device__ __forceinline__ void bload(rsrc_t rs, int rowoff, int cu, int u4) {
    const int so = (u4 >> 2) * 144;
    h = bld16(rs, rowoff, so);
    q0 = bld16(rs, rowoff + 16 + 32 * cu, so);
    q1 = bld16(rs, rowoff + 32 + 32 * cu, so);
  }
  template <int M>
  __device__ __forceinline__ void dot(int u, const Xv& xv, float acc[M]) const {
    const float d = f16_to_f32(h.x), dmin = f16_to_f32(h.x >> 16);
    const int j0 = 2 * (u & 3);
    uint32_t sc0, m0, sc1, m1;
    q4k_scale_min(h.y, h.z, h.w, j0, sc0, m0);
    q4k_scale_min(h.y, h.z, h.w, j0 + 1, sc1, m1);
    const float dsc0 = d * (float)sc0, dm0 = dmin * (float)m0;
    const float dsc1 = d * (float)sc1, dm1 = dmin * (float)m1;
    const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    uint32_t lo[16], hi[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t l = qw[i] & 0x0F0F0F0Fu, hh = (qw[i] >> 4) & 0x0F0F0F0Fu;
      lo[2 * i] = pair01(l); lo[2 * i + 1] = pair23(l);
      hi[2 * i] = pair01(hh); hi[2 * i + 1] = pair23(hh);
    }
    const int base = 64 * u;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float s0 = 0.f, s1 = 0.f;
      s0 = dot16(lo, xv.pairs(m, base), s0);
      s0 = dot16(lo + 8, xv.pairs(m, base + 16), s0);
      s1 = dot16(hi, xv.pairs(m, base + 32), s1);
      s1 = dot16(hi + 8, xv.pairs(m, base + 48), s1);
      const float4_t xs = *(const float4_t*)&xv.xsum[m * xv.sstride + ((base - xv.c0) >> 4)];
      const float x0 = xs.x + xs.y, x1 = xs.z + xs.w;
      acc[m] += dsc0 * (s0 - 1024.f * x0) - dm0 * x0 + dsc1 * (s1 - 1024.f * x1) - dm1 * x1;
    }
  }
};

// q5_K: q4_K's unit (the 32 qs bytes of sub-block pair P = u % 4) plus the
// 32 qh bytes, whose bits 2P and 2P + 1 are the fifth bits of the two
// sub-blocks' values.
struct UnitQ5K {
  u32x4 h, q0, q1, e0, e1;
  __device__ __forceinline__ void load(const uint8_t* row, int u) {
    const uint8_t* blk = row + (u >> 2) * 176;
    h = ld_16B(blk);
    e0 = ld_16B(blk + 16);
    e1 = ld_16B(blk + 32);
    const uint8_t* qs = blk + 48 + 32 * (u & 3);
    q0 = ld_16B(qs);
    q1 = ld_16B(qs + 16);
  }
  __device__ __forceinline__ void bload(rsrc_t rs, int rowoff, int cu, int u4) {
    const int so = (u4 >> 2) * 176;
    h = bld16(rs, rowoff, so);
    e0 = bld16(rs, rowoff + 16, so);
    e1 = bld16(rs, rowoff + 32, so);
    q0 = bld16(rs, rowoff + 48 + 32 * cu, so);
    q1 = bld16(rs, rowoff + 64 + 32 * cu, so);
  }
  // 5-bit code bytes of dword i: low nibbles (sub-block 2P) or high (2P + 1)
  static __device__ __forceinline__ uint32_t lo5(uint32_t qw, uint32_t qhs) {
    return (qw & 0x0F0F0F0Fu) | ((qhs << 4) & 0x10101010u);
  }
  static __device__ __forceinline__ uint32_t hi5(uint32_t qw, uint32_t qhs) {
    return ((qw >> 4) & 0x0F0F0F0Fu) | ((qhs << 3) & 0x10101010u);
  }
  template <int M>
  __device__ __forceinline__ void dot(int u, const Xv& xv, float acc[M]) const {
    const float d = f16_to_f32(h.x), dmin = f16_to_f32(h.x >> 16);
    const int j0 = 2 * (u & 3);
    uint32_t sc0, m0, sc1, m1;
    q4k_scale_min(h.y, h.z, h.w, j0, sc0, m0);
    q4k_scale_min(h.y, h.z, h.w, j0 + 1, sc1, m1);
    const float dsc0 = d * (float)sc0, dm0 = dmin * (float)m0;
    const float dsc1 = d * (float)sc1, dm1 = dmin * (float)m1;
    const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    const uint32_t qe[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
    uint32_t lo[16], hi[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t qhs = qe[i] >> j0;
      const uint32_t l = lo5(qw[i], qhs), hh = hi5(qw[i], qhs);
      lo[2 * i] = pair01(l); lo[2 * i + 1] = pair23(l);
      hi[2 * i] = pair01(hh); hi[2 * i + 1] = pair23(hh);
    }
    const int base = 64 * u;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float s0 = 0.f, s1 = 0.f;
      s0 = dot16(lo, xv.pairs(m, base), s0);
      s0 = dot16(lo + 8, xv.pairs(m, base + 16), s0);
      s1 = dot16(hi, xv.pairs(m, base + 32), s1);
      s1 = dot16(hi + 8, xv.pairs(m, base + 48), s1);
      const float4_t xs = *(const float4_t*)&xv.xsum[m * xv.sstride + ((base - xv.c0) >> 4)];
      const float x0 = xs.x + xs.y, x1 = xs.z + xs.w;
      acc[m] += dsc0 * (s0 - 1024.f * x0) - dm0 * x0 + dsc1 * (s1 - 1024.f * x1) - dm1 * x1;
    }
  }
};

// q2_K: unit u' = u % 4 of a superblock is half h = u' / 2 with code shifts
// 2 c0 (values 0..31) and 2 c0 + 2 (32..63), c0 = 2 (u' % 2): the 32 qs
// bytes of half h, the scale bytes of sub-blocks 4u'..4u'+3 and d, dmin.
// Sub-block t of the unit (16 values) is shift c0 + t / 2, qs dwords
// 4 (t % 2) .. 4 (t % 2) + 3.
struct UnitQ2K {
  u32x4 q0, q1;
  uint32_t sc, dd;
  __device__ __forceinline__ void load(const uint8_t* row, int u) {
    const uint8_t* blk = row + (u >> 2) * 84;  // dword aligned
    const int up = u & 3;
    q0 = ld_16B_a4(blk + 16 + 32 * (up >> 1));
    q1 = ld_16B_a4(blk + 32 + 32 * (up >> 1));
    sc = ld_u32(blk + 4 * up);
    dd = ld_u32(blk + 80);
  }
  __device__ __forceinline__ void bload(rsrc_t rs, int rowoff, int cu, int u4) {
    const int so = (u4 >> 2) * 84;
    q0 = bld16(rs, rowoff + 16 + 32 * (cu >> 1), so);
    q1 = bld16(rs, rowoff + 32 + 32 * (cu >> 1), so);
    sc = bld4(rs, rowoff + 4 * cu, so);
    dd = bld4(rs, rowoff + 80, so);
  }
  template <int M>
  __device__ __forceinline__ void dot(int u, const Xv& xv, float acc[M]) const {
    const float d = f16_to_f32(dd), dmin = f16_to_f32(dd >> 16);
    const int c0 = 2 * (u & 1);
    const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    float dsc[4], dm[4];
    uint32_t p[4][8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t b = (sc >> (8 * t)) & 0xFFu;
      dsc[t] = d * (float)(b & 15u);
      dm[t] = dmin * (float)(b >> 4);
      const int shift = 2 * (c0 + (t >> 1));
      uint32_t c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = (qw[4 * (t & 1) + i] >> shift) & 0x03030303u;
      pairs16(c, p[t]);
    }
    const int base = 64 * u;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float4_t xs = *(const float4_t*)&xv.xsum[m * xv.sstride + ((base - xv.c0) >> 4)];
      const float x[4] = {xs.x, xs.y, xs.z, xs.w};
      float tot = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float st = dot16(p[t], xv.pairs(m, base + 16 * t), 0.f);
        tot += dsc[t] * (st - 1024.f * x[t]) - dm[t] * x[t];
      }
      acc[m] += tot;
    }
  }
};

// 16 bytes at a 2-byte aligned address: dwords loaded from the dword-aligned
// address below it, then shifted by (addr & 3) bytes.
struct Shift16 {
  u32x4 a;
  uint32_t b;
  __device__ __forceinline__ void load(const uint8_t* p, uint32_t sh) {
    const uint8_t* q = p - sh;
    a = ld_16B_a4(q);
    b = ld_u32(q + 16 - (sh ? 0 : 4));  // sh == 0: re-read the 4th dword, never past the 16 bytes
  }
  // same from a buffer: va (per lane) and soff (uniform) dword aligned, the
  // 16 bytes start sh bytes past va + soff
  __device__ __forceinline__ void bload(rsrc_t rs, int va, int soff, uint32_t sh) {
    a = bld16(rs, va, soff);
    b = bld4(rs, va + 16 - (sh ? 0 : 4), soff);
  }
  __device__ __forceinline__ void get(uint32_t sh, uint32_t o[4]) const {
    o[0] = alignbyte(a.y, a.x, sh);
    o[1] = alignbyte(a.z, a.y, sh);
    o[2] = alignbyte(a.w, a.z, sh);
    o[3] = alignbyte(b, a.w, sh);
  }
};

struct UnitQ6K {
  Shift16 qa, qb, qhh, scl;
  uint32_t dbits, sh;
  __device__ __forceinline__ void load(const uint8_t* row, int u) {
    const uint8_t* blk = row + (u >> 2) * 210;
    const int h = (u >> 1) & 1, half = u & 1;
    sh = (uint32_t)((uintptr_t)blk & 3);
    qa.load(blk + 64 * h + 16 * half, sh);
    qb.load(blk + 64 * h + 32 + 16 * half, sh);
    qhh.load(blk + 128 + 32 * h + 16 * half, sh);
    scl.load(blk + 192, sh);
    dbits = ld_u16(blk + 208);
  }
  // Buffer offsets must each be dword aligned for the dword loads, and a
  // 210-byte block is not: the uniform offset steps over pairs of blocks, the
  // odd block and the sub-dword shift go into the per-lane offset (rowoff is
  // relative to a dword-aligned descriptor base).
  __device__ __forceinline__ void bload(rsrc_t rs, int rowoff, int cu, int u4) {
    const int blk = u4 >> 2, so = 420 * (blk >> 1);
    const int h = (cu >> 1) & 1, half = cu & 1;
    const int t = rowoff + 210 * (blk & 1);
    sh = (uint32_t)t & 3u;
    const int va = t - (int)sh;
    qa.bload(rs, va + 64 * h + 16 * half, so, sh);
    qb.bload(rs, va + 64 * h + 32 + 16 * half, so, sh);
    qhh.bload(rs, va + 128 + 32 * h + 16 * half, so, sh);
    scl.bload(rs, va + 192, so, sh);
    dbits = bld2(rs, t + 208, so);
  }
  template <int M>
  __device__ __forceinline__ void dot(int u, const Xv& xv, float acc[M]) const {
    const int h = (u >> 1) & 1, half = u & 1;
    uint32_t A[4], B[4], H[4], S[4];
    qa.get(sh, A); qb.get(sh, B); qhh.get(sh, H); scl.get(sh, S);
    const float d = f16_to_f32(dbits);
    const uint32_t slo = h ? S[2] : S[0], shi = h ? S[3] : S[1];
    float dsc[4];
    dsc[0] = d * (float)(int)(int8_t)(slo >> (8 * half));
    dsc[1] = d * (float)(int)(int8_t)(slo >> (8 * (half + 2)));
    dsc[2] = d * (float)(int)(int8_t)(shi >> (8 * half));
    dsc[3] = d * (float)(int)(int8_t)(shi >> (8 * (half + 2)));
    uint32_t c[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[0][i] = (A[i] & 0x0F0F0F0Fu) | ((H[i] << 4) & 0x30303030u);
      c[1][i] = (B[i] & 0x0F0F0F0Fu) | ((H[i] << 2) & 0x30303030u);
      c[2][i] = ((A[i] >> 4) & 0x0F0F0F0Fu) | (H[i] & 0x30303030u);
      c[3][i] = ((B[i] >> 4) & 0x0F0F0F0Fu) | ((H[i] >> 2) & 0x30303030u);
    }
    uint32_t p[4][8];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) pairs16(c[cc], p[cc]);
    // staged in unit order (xperm): segment cc of the unit at 64 u + 16 cc
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float4_t xs = xv.sum64(m, 64 * u);
      float t = 0.f;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const float s = dot16(p[cc], xv.pairs(m, 64 * u + 16 * cc), 0.f);
        t += dsc[cc] * (s - 1056.f * xs[cc]);
      }
      acc[m] += t;
    }
  }
};

struct UnitQ8_0 {  // two 34-byte blocks, 68 bytes, dword aligned
  u32x4 r0, r1, r2, r3;
  uint32_t r4;
  __device__ __forceinline__ void load(const uint8_t* row, int u) {
    const uint8_t* p = row + 68 * u;
    r0 = ld_16B_a4(p); r1 = ld_16B_a4(p + 16); r2 = ld_16B_a4(p + 32); r3 = ld_16B_a4(p + 48);
    r4 = ld_u32(p + 64);
  }
  __device__ __forceinline__ void bload(rsrc_t rs, int rowoff, int cu, int u4) {
    const int vo = rowoff + 68 * cu, so = 68 * u4;
    r0 = bld16(rs, vo, so); r1 = bld16(rs, vo + 16, so); r2 = bld16(rs, vo + 32, so); r3 = bld16(rs, vo + 48, so);
    r4 = bld4(rs, vo + 64, so);
  }
  template <int M>
  __device__ __forceinline__ void dot(int u, const Xv& xv, float acc[M]) const {
    const uint32_t R[17] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w,
                            r2.x, r2.y, r2.z, r2.w, r3.x, r3.y, r3.z, r3.w, r4};
    const float d0 = f16_to_f32(R[0]), d1 = f16_to_f32(R[8] >> 16);
    uint32_t c0[8], c1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      c0[i] = alignbyte(R[i + 1], R[i], 2) ^ 0x80808080u;  // code + 128
      c1[i] = R[9 + i] ^ 0x80808080u;
    }
    uint32_t p0[16], p1[16];
    pairs16(c0, p0); pairs16(c0 + 4, p0 + 8);
    pairs16(c1, p1); pairs16(c1 + 4, p1 + 8);
    const int base = 64 * u;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float s0 = dot16(p0, xv.pairs(m, base), 0.f);
      s0 = dot16(p0 + 8, xv.pairs(m, base + 16), s0);
      float s1 = dot16(p1, xv.pairs(m, base + 32), 0.f);
      s1 = dot16(p1 + 8, xv.pairs(m, base + 48), s1);
      const float4_t xs = *(const float4_t*)&xv.xsum[m * xv.sstride + ((base - xv.c0) >> 4)];
      const float x0 = xs.x + xs.y, x1 = xs.z + xs.w;
      acc[m] += d0 * (s0 - 1152.f * x0) + d1 * (s1 - 1152.f * x1);
    }
  }
};

struct UnitQ4_0 {  // two 18-byte blocks, 36 bytes, dword aligned
  u32x4 r0, r1;
  uint32_t r2;
  __device__ __forceinline__ void load(const uint8_t* row, int u) {
    const uint8_t* p = row + 36 * u;
    r0 = ld_16B_a4(p); r1 = ld_16B_a4(p + 16);
    r2 = ld_u32(p + 32);
  }
  __device__ __forceinline__ void bload(rsrc_t rs, int rowoff, int cu, int u4) {
    const int vo = rowoff + 36 * cu, so = 36 * u4;
    r0 = bld16(rs, vo, so); r1 = bld16(rs, vo + 16, so);
    r2 = bld4(rs, vo + 32, so);
  }
  template <int M>
  __device__ __forceinline__ void dot(int u, const Xv& xv, float acc[M]) const {
    const uint32_t R[9] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w, r2};
    const float d0 = f16_to_f32(R[0]), d1 = f16_to_f32(R[4] >> 16);
    uint32_t q0[4], q1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { q0[i] = alignbyte(R[i + 1], R[i], 2); q1[i] = R[5 + i]; }
    uint32_t l0[4], h0[4], l1[4], h1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      l0[i] = q0[i] & 0x0F0F0F0Fu; h0[i] = (q0[i] >> 4) & 0x0F0F0F0Fu;
      l1[i] = q1[i] & 0x0F0F0F0Fu; h1[i] = (q1[i] >> 4) & 0x0F0F0F0Fu;
    }
    uint32_t pl0[8], ph0[8], pl1[8], ph1[8];
    pairs16(l0, pl0); pairs16(h0, ph0); pairs16(l1, pl1); pairs16(h1, ph1);
    const int base = 64 * u;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float s0 = dot16(pl0, xv.pairs(m, base), 0.f);
      s0 = dot16(ph0, xv.pairs(m, base + 16), s0);
      float s1 = dot16(pl1, xv.pairs(m, base + 32), 0.f);
      s1 = dot16(ph1, xv.pairs(m, base + 48), s1);
      const float4_t xs = *(const float4_t*)&xv.xsum[m * xv.sstride + ((base - xv.c0) >> 4)];
      const float x0 = xs.x + xs.y, x1 = xs.z + xs.w;
      acc[m] += d0 * (s0 - 1032.f * x0) + d1 * (s1 - 1032.f * x1);
    }
  }
};

// q4_1, q5_0, q5_1: a unit is two blocks (40, 44 or 48 bytes), dword
// aligned in a row of whole units.
template <int C>
struct UnitLeg {
  using L = Leg<C>;
  static constexpr int UB = 2 * L::BB, NWD = UB / 4;
  u32x4 a, b;
  uint32_t t0, t1, t2 = 0, t3 = 0;  // dwords 8 .. NWD-1
  __device__ __forceinline__ void load(const uint8_t* row, int u) {
    const uint8_t* p = row + UB * u;
    a = ld_16B_a4(p); b = ld_16B_a4(p + 16);
    t0 = ld_u32(p + 32); t1 = ld_u32(p + 36);
    if constexpr (NWD > 10) t2 = ld_u32(p + 40);
    if constexpr (NWD > 11) t3 = ld_u32(p + 44);
  }
  __device__ __forceinline__ void bload(rsrc_t rs, int rowoff, int cu, int u4) {
    const int vo = rowoff + UB * cu, so = UB * u4;
    a = bld16(rs, vo, so); b = bld16(rs, vo + 16, so);
    t0 = bld4(rs, vo + 32, so); t1 = bld4(rs, vo + 36, so);
    if constexpr (NWD > 10) t2 = bld4(rs, vo + 40, so);
    if constexpr (NWD > 11) t3 = bld4(rs, vo + 44, so);
  }
  // the 4 bytes at unit byte offset O (even)
  template <int O>
  __device__ __forceinline__ uint32_t at() const {
    const uint32_t R[12] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w, t0, t1, t2, t3};
    if constexpr (O % 4 == 0) return R[O / 4];
    else return alignbyte(R[O / 4 + 1], R[O / 4], 2);
  }
  // block B's d, m and code dwords (lo: values 0..15, hi: 16..31)
  template <int B>
  __device__ __forceinline__ void block(float& d, float& m, uint32_t lo[4], uint32_t hi[4]) const {
    constexpr int base = B * L::BB, qso = base + L::QS, qho = base + (L::QH >= 0 ? L::QH : 0);
    const uint32_t w0 = at<base>();
    d = f16_to_f32(w0);
    m = L::MIN ? f16_to_f32(w0 >> 16) : 0.f;
    const uint32_t qh = L::QH >= 0 ? at<qho>() : 0u;
    const uint32_t q[4] = {at<qso>(), at<qso + 4>(), at<qso + 8>(), at<qso + 12>()};
#pragma unroll
    for (int i = 0; i < 4; ++i) { lo[i] = leg_lo<C>(q[i], qh, i); hi[i] = leg_hi<C>(q[i], qh, i); }
  }
  template <int M>
  __device__ __forceinline__ void dot(int u, const Xv& xv, float acc[M]) const {
    float d0, m0, d1, m1;
    uint32_t lo0[4], hi0[4], lo1[4], hi1[4];
    block<0>(d0, m0, lo0, hi0);
    block<1>(d1, m1, lo1, hi1);
    uint32_t pl0[8], ph0[8], pl1[8], ph1[8];
    pairs16(lo0, pl0); pairs16(hi0, ph0); pairs16(lo1, pl1); pairs16(hi1, ph1);
    constexpr float K = 1024.f + (float)L::ZP;  // the float16 code offset
    const int base = 64 * u;
#pragma unroll
    for (int mm = 0; mm < M; ++mm) {
      float s0 = dot16(pl0, xv.pairs(mm, base), 0.f);
      s0 = dot16(ph0, xv.pairs(mm, base + 16), s0);
      float s1 = dot16(pl1, xv.pairs(mm, base + 32), 0.f);
      s1 = dot16(ph1, xv.pairs(mm, base + 48), s1);
      const float4_t xs = *(const float4_t*)&xv.xsum[mm * xv.sstride + ((base - xv.c0) >> 4)];
      const float x0 = xs.x + xs.y, x1 = xs.z + xs.w;
      float t = d0 * (s0 - K * x0) + d1 * (s1 - K * x1);
      if constexpr (L::MIN) t += m0 * x0 + m1 * x1;
      acc[mm] += t;
    }
  }
};

// q3_K: unit u' = u % 4 is half h = u' / 2 at code shifts c0 = 2 (u' % 2)
// and c0 + 1, as q2_K: the 32 qs bytes of half h, the 32 hmask bytes (bits
// 4h + c), the scale bytes and d.  Blocks are 2-byte aligned (110 bytes):
// every span is read from the dword below it (Shift16) and placed so that
// the read stays inside the block; the scales come from the span [92, 108).
struct UnitQ3K {
  Shift16 qa, qb, ha, hb, sc;
  uint32_t dbits, sh;
  __device__ __forceinline__ void load(const uint8_t* row, int u) {
    const uint8_t* blk = row + (u >> 2) * 110;
    const int h = (u >> 1) & 1;
    sh = (uint32_t)((uintptr_t)blk & 3);
    qa.load(blk + 32 + 32 * h, sh);
    qb.load(blk + 48 + 32 * h, sh);
    ha.load(blk, sh);
    hb.load(blk + 16, sh);
    sc.load(blk + 92, sh);
    dbits = ld_u16(blk + 108);
  }
  // as q6_K: the uniform offset steps over pairs of blocks (220 bytes), the
  // odd block and the sub-dword shift go into the per-lane offset
  __device__ __forceinline__ void bload(rsrc_t rs, int rowoff, int cu, int u4) {
    const int blk = u4 >> 2, so = 220 * (blk >> 1);
    const int h = (cu >> 1) & 1;
    const int t = rowoff + 110 * (blk & 1);
    sh = (uint32_t)t & 3u;
    const int va = t - (int)sh;
    qa.bload(rs, va + 32 + 32 * h, so, sh);
    qb.bload(rs, va + 48 + 32 * h, so, sh);
    ha.bload(rs, va, so, sh);
    hb.bload(rs, va + 16, so, sh);
    sc.bload(rs, va + 92, so, sh);
    dbits = bld2(rs, t + 108, so);
  }
  // the unit's four signed sub-block scales times d, and its 3-bit codes
  // (u = q + 4) of sub-block t as four dwords
  __device__ __forceinline__ void fields(int u, float s[4], uint32_t cw[4][4]) const {
    const int up = u & 3, h = up >> 1, c0 = 2 * (up & 1);
    uint32_t Q[8], H[8], S[4];
    qa.get(sh, Q); qb.get(sh, Q + 4); ha.get(sh, H); hb.get(sh, H + 4); sc.get(sh, S);
    const float d = f16_to_f32(dbits);
    const uint32_t A = (up & 1) ? S[2] : S[1], B = S[3];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = d * (float)q3k_scale(A, B, up, t);
      const int c = c0 + (t >> 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = 4 * (t & 1) + i;
        cw[t][i] = ((Q[k] >> (2 * c)) & 0x03030303u) | (((H[k] >> (4 * h + c)) & 0x01010101u) << 2);
      }
    }
  }
  template <int M>
  __device__ __forceinline__ void dot(int u, const Xv& xv, float acc[M]) const {
    float s[4];
    uint32_t cw[4][4], p[4][8];
    fields(u, s, cw);
#pragma unroll
    for (int t = 0; t < 4; ++t) pairs16(cw[t], p[t]);
    const int base = 64 * u;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float4_t xs = *(const float4_t*)&xv.xsum[m * xv.sstride + ((base - xv.c0) >> 4)];
      const float x[4] = {xs.x, xs.y, xs.z, xs.w};
      float tot = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) tot += s[t] * (dot16(p[t], xv.pairs(m, base + 16 * t), 0.f) - 1028.f * x[t]);
      acc[m] += tot;
    }
  }
};

template <int C> struct UnitOf;
template <> struct UnitOf<Q4_K> { typedef UnitQ4K T; };
template <> struct UnitOf<Q2_K> { typedef UnitQ2K T; };
template <> struct UnitOf<Q3_K> { typedef UnitQ3K T; };
template <> struct UnitOf<Q5_K> { typedef UnitQ5K T; };
template <> struct UnitOf<Q6_K> { typedef UnitQ6K T; };
template <> struct UnitOf<Q8_0> { typedef UnitQ8_0 T; };
template <> struct UnitOf<Q4_0> { typedef UnitQ4_0 T; };
template <> struct UnitOf<Q4_1> { typedef UnitLeg<Q4_1> T; };
template <> struct UnitOf<Q5_0> { typedef UnitLeg<Q5_0> T; };
template <> struct UnitOf<Q5_1> { typedef UnitLeg<Q5_1> T; };

// ---------------------------------------------------------------------------
// Matrix-core operand slices of a unit.
// ---------------------------------------------------------------------------

// Slice S (8 consecutive K values) of a unit: get<S> gives its float16
// weights f[4] (all zero for a lane that keeps nothing); koff(u) is the row
// offset of the unit's first value and xstep<S> the slice's offset from it in
// padded LDS units.
template <int C> struct MmaSlices;

template <> struct MmaSlices<Q4_K> {
  // values 0..31: low nibbles of the 32 qs bytes (sub-block 2P), 32..63: high
  // nibbles (sub-block 2P + 1); weight = d sc q - dmin m.  High nibbles are
  // used in place (16 q, no shift), so their step s1 carries a factor 1/16
  // (exact: d sc / 16 is a float16 value times a small integer).
  float s0, c0, s1, c1;
  uint32_t qw[8];
  __device__ __forceinline__ MmaSlices(const UnitQ4K& un, int u, bool keep) {
    const float d = keep ? f16_to_f32(un.h.x) : 0.f, dmin = keep ? f16_to_f32(un.h.x >> 16) : 0.f;
    uint32_t sc0, m0, sc1, m1;
    q4k_scale_min_pair(un.h.y, un.h.z, un.h.w, u & 3, sc0, m0, sc1, m1);
    s0 = d * (float)sc0; c0 = -(1024.f * s0 + dmin * (float)m0);
    s1 = (0.0625f * d) * (float)sc1; c1 = -(1024.f * s1 + dmin * (float)m1);
    qw[0] = un.q0.x; qw[1] = un.q0.y; qw[2] = un.q0.z; qw[3] = un.q0.w;
    qw[4] = un.q1.x; qw[5] = un.q1.y; qw[6] = un.q1.z; qw[7] = un.q1.w;
  }
  static __device__ __forceinline__ int koff(int u) { return 64 * u; }
  template <int S>
  static constexpr int xstep() { return 8 * S; }
  template <int S>
  __device__ __forceinline__ void get(uint32_t f[4]) const {
    constexpr int t = S & 3;
    if (S < 4)
      slice8(qw[2 * t] & 0x0F0F0F0Fu, qw[2 * t + 1] & 0x0F0F0F0Fu, s0, c0, f);
    else
      slice8(qw[2 * t] & 0xF0F0F0F0u, qw[2 * t + 1] & 0xF0F0F0F0u, s1, c1, f);
  }
};

template <> struct MmaSlices<Q2_K> {
  // slice S: sub-block t = S / 2 (its own scale and min), qs dwords
  // 4 (t % 2) + 2 (S % 2) and the next, code shift 2 c0 + 2 (S / 4); the
  // codes are kept shifted by 2 c0 so that the rest is compile-time.
  // weight = fma(1024 + q, d sc, -(1024 d sc + dmin m))
  uint32_t qs[8];
  float s[4], c[4];
  __device__ __forceinline__ MmaSlices(const UnitQ2K& un, int u, bool keep) {
    const float d = keep ? f16_to_f32(un.dd) : 0.f, dmin = keep ? f16_to_f32(un.dd >> 16) : 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t b = (un.sc >> (8 * t)) & 0xFFu;
      s[t] = d * (float)(b & 15u);
      c[t] = -(1024.f * s[t] + dmin * (float)(b >> 4));
    }
    const int sh = 4 * (u & 1);
    qs[0] = un.q0.x >> sh; qs[1] = un.q0.y >> sh; qs[2] = un.q0.z >> sh; qs[3] = un.q0.w >> sh;
    qs[4] = un.q1.x >> sh; qs[5] = un.q1.y >> sh; qs[6] = un.q1.z >> sh; qs[7] = un.q1.w >> sh;
  }
  static __device__ __forceinline__ int koff(int u) { return 64 * u; }
  template <int S>
  static constexpr int xstep() { return 8 * S; }
  template <int S>
  __device__ __forceinline__ void get(uint32_t f[4]) const {
    constexpr int t = S >> 1, i0 = 4 * (t & 1) + 2 * (S & 1), sh = 2 * (S >> 2);
    slice8((qs[i0] >> sh) & 0x03030303u, (qs[i0 + 1] >> sh) & 0x03030303u, s[t], c[t], f);
  }
};

template <> struct MmaSlices<Q3_K> {
  // slice S: sub-block t = S / 2, code dwords 2 (S % 2) .. of it; weight =
  // fma(1024 + u, d sc, -1028 d sc) = d sc (u - 4)
  uint32_t cw[4][4];
  float s[4];
  __device__ __forceinline__ MmaSlices(const UnitQ3K& un, int u, bool keep) {
    un.fields(u, s, cw);
    if (!keep) s[0] = s[1] = s[2] = s[3] = 0.f;
  }
  static __device__ __forceinline__ int koff(int u) { return 64 * u; }
  template <int S>
  static constexpr int xstep() { return 8 * S; }
  template <int S>
  __device__ __forceinline__ void get(uint32_t f[4]) const {
    constexpr int t = S >> 1, i = 2 * (S & 1);
    slice8(cw[t][i], cw[t][i + 1], s[t], -1028.f * s[t], f);
  }
};

template <> struct MmaSlices<Q5_K> {
  // q4_K's slices with 5-bit codes: values 0..31 sub-block 2P (low nibbles,
  // fifth bit from bit 2P of qh), 32..63 sub-block 2P + 1 (high nibbles, bit
  // 2P + 1); weight = d sc q - dmin m.  qhs holds qh >> 2P.
  float s0, c0, s1, c1;
  uint32_t qw[8], qhs[8];
  __device__ __forceinline__ MmaSlices(const UnitQ5K& un, int u, bool keep) {
    const float d = keep ? f16_to_f32(un.h.x) : 0.f, dmin = keep ? f16_to_f32(un.h.x >> 16) : 0.f;
    uint32_t sc0, m0, sc1, m1;
    q4k_scale_min_pair(un.h.y, un.h.z, un.h.w, u & 3, sc0, m0, sc1, m1);
    s0 = d * (float)sc0; c0 = -(1024.f * s0 + dmin * (float)m0);
    s1 = d * (float)sc1; c1 = -(1024.f * s1 + dmin * (float)m1);
    qw[0] = un.q0.x; qw[1] = un.q0.y; qw[2] = un.q0.z; qw[3] = un.q0.w;
    qw[4] = un.q1.x; qw[5] = un.q1.y; qw[6] = un.q1.z; qw[7] = un.q1.w;
    const int j0 = 2 * (u & 3);
    qhs[0] = un.e0.x >> j0; qhs[1] = un.e0.y >> j0; qhs[2] = un.e0.z >> j0; qhs[3] = un.e0.w >> j0;
    qhs[4] = un.e1.x >> j0; qhs[5] = un.e1.y >> j0; qhs[6] = un.e1.z >> j0; qhs[7] = un.e1.w >> j0;
  }
  static __device__ __forceinline__ int koff(int u) { return 64 * u; }
  template <int S>
  static constexpr int xstep() { return 8 * S; }
  template <int S>
  __device__ __forceinline__ void get(uint32_t f[4]) const {
    constexpr int t = S & 3;
    if (S < 4)
      slice8(UnitQ5K::lo5(qw[2 * t], qhs[2 * t]), UnitQ5K::lo5(qw[2 * t + 1], qhs[2 * t + 1]), s0, c0, f);
    else
      slice8(UnitQ5K::hi5(qw[2 * t], qhs[2 * t]), UnitQ5K::hi5(qw[2 * t + 1], qhs[2 * t + 1]), s1, c1, f);
  }
};

template <> struct MmaSlices<Q6_K> {
  // four 16-value segments cc at base + 32 cc; weight = d sc (q - 32)
  uint32_t c[4][4];
  float sc[4];
  int base;
  __device__ __forceinline__ MmaSlices(const UnitQ6K& un, int u, bool keep) {
    const int h = (u >> 1) & 1, half = u & 1;
    uint32_t A[4], B[4], H[4], S[4];
    un.qa.get(un.sh, A); un.qb.get(un.sh, B); un.qhh.get(un.sh, H); un.scl.get(un.sh, S);
    const float d = keep ? f16_to_f32(un.dbits) : 0.f;
    const uint32_t slo = h ? S[2] : S[0], shi = h ? S[3] : S[1];
    sc[0] = d * (float)(int)(int8_t)(slo >> (8 * half));
    sc[1] = d * (float)(int)(int8_t)(slo >> (8 * (half + 2)));
    sc[2] = d * (float)(int)(int8_t)(shi >> (8 * half));
    sc[3] = d * (float)(int)(int8_t)(shi >> (8 * (half + 2)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[0][i] = (A[i] & 0x0F0F0F0Fu) | ((H[i] << 4) & 0x30303030u);
      c[1][i] = (B[i] & 0x0F0F0F0Fu) | ((H[i] << 2) & 0x30303030u);
      c[2][i] = ((A[i] >> 4) & 0x0F0F0F0Fu) | (H[i] & 0x30303030u);
      c[3][i] = ((B[i] >> 4) & 0x0F0F0F0Fu) | ((H[i] >> 2) & 0x30303030u);
    }
    base = 256 * (u >> 2) + 128 * h + 16 * half;
  }
  // the unit starts 0 or 16 values into a 64-value block and spans 128
  // values, so segments 2 and 3 sit one padding step further in LDS
  static __device__ __forceinline__ int koff(int u) { return 256 * (u >> 2) + 128 * ((u >> 1) & 1) + 16 * (u & 1); }
  template <int S>
  static constexpr int xstep() { return 32 * (S >> 1) + 8 * (S & 1) + 8 * (S >> 2); }
  template <int S>
  __device__ __forceinline__ void get(uint32_t f[4]) const {
    constexpr int cc = S >> 1, sub = S & 1;
    slice8(c[cc][2 * sub], c[cc][2 * sub + 1], sc[cc], -1056.f * sc[cc], f);
  }
};

// Eight codes -> eight float16 weights d (code - k), for codecs whose weight
// is the scale times an exact integer: the byte permute builds 1024 + code,
// the packed subtract of k is exact, and the packed multiply by d rounds the
// exact product once to nearest even -- the same bits as slice8's float32
// FMA and conversion (d (code - k) is exact in float32), in two packed
// operations per pair instead of three.  d2 holds d in both halves, k2 holds
// k (an integer below 2048) in both halves.
__device__ __forceinline__ void slice8_dq(uint32_t c0, uint32_t c1, uint32_t k2, uint32_t d2, uint32_t f[4]) {
  const uint32_t p[4] = {pair01(c0), pair23(c0), pair01(c1), pair23(c1)};
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = as_u32((as_h2(p[i]) - as_h2(k2)) * as_h2(d2));
}

template <> struct MmaSlices<Q8_0> {
  // block b = S >> 2 (values 32 b ..); code + 128 from a sign-bit flip; weight = d q
  uint32_t c[2][8];
  uint32_t d[2];  // the block's float16 d in both halves (zero for a lane that keeps nothing)
  __device__ __forceinline__ MmaSlices(const UnitQ8_0& un, int, bool keep) {
    const uint32_t R[17] = {un.r0.x, un.r0.y, un.r0.z, un.r0.w, un.r1.x, un.r1.y, un.r1.z, un.r1.w,
                            un.r2.x, un.r2.y, un.r2.z, un.r2.w, un.r3.x, un.r3.y, un.r3.z, un.r3.w, un.r4};
    d[0] = keep ? perm(R[0], R[0], 0x01000100u) : 0u;
    d[1] = keep ? perm(R[8], R[8], 0x03020302u) : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      c[0][i] = alignbyte(R[i + 1], R[i], 2) ^ 0x80808080u;
      c[1][i] = R[9 + i] ^ 0x80808080u;
    }
  }
  static __device__ __forceinline__ int koff(int u) { return 64 * u; }
  template <int S>
  static constexpr int xstep() { return 8 * S; }
  template <int S>
  __device__ __forceinline__ void get(uint32_t f[4]) const {
    constexpr int b = S >> 2, t = S & 3;
    slice8_dq(c[b][2 * t], c[b][2 * t + 1], 0x64806480u, d[b], f);  // (1024 + 128 + q) - 1152 = q
  }
};

template <> struct MmaSlices<Q4_0> {
  // block b = S >> 2: values 0..15 low nibbles of its 16 bytes, 16..31 high;
  // weight = d (q - 8).  High nibbles are used in place (16 q) with step d / 16.
  uint32_t q[2][4];
  uint32_t d[2];  // the block's float16 d in both halves (zero for a lane that keeps nothing)
  __device__ __forceinline__ MmaSlices(const UnitQ4_0& un, int, bool keep) {
    const uint32_t R[9] = {un.r0.x, un.r0.y, un.r0.z, un.r0.w, un.r1.x, un.r1.y, un.r1.z, un.r1.w, un.r2};
    d[0] = keep ? perm(R[0], R[0], 0x01000100u) : 0u;
    d[1] = keep ? perm(R[4], R[4], 0x03020302u) : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[0][i] = alignbyte(R[i + 1], R[i], 2);
      q[1][i] = R[5 + i];
    }
  }
  static __device__ __forceinline__ int koff(int u) { return 64 * u; }
  template <int S>
  static constexpr int xstep() { return 8 * S; }
  template <int S>
  __device__ __forceinline__ void get(uint32_t f[4]) const {
    constexpr int b = S >> 2, t = S & 3, dw = 2 * (t & 1);
    if (t < 2)  // ((1024 + q) - 1032) d = d (q - 8)
      slice8_dq(q[b][dw] & 0x0F0F0F0Fu, q[b][dw + 1] & 0x0F0F0F0Fu, 0x64086408u, d[b], f);
    else  // the high nibbles shifted down, same map
      slice8_dq((q[b][dw] >> 4) & 0x0F0F0F0Fu, (q[b][dw + 1] >> 4) & 0x0F0F0F0Fu, 0x64086408u, d[b], f);
  }
};

// q4_1, q5_0, q5_1: block b = S >> 2 (values 32 b ..): slices t < 2 are the
// low-nibble codes (values 8t..), t >= 2 the high ones; weight =
// fma(1024 + q, d, m - 1024 d) or fma(1024 + q, d, -(1024 + 16) d).
template <int C>
struct MmaSlicesLeg {
  using L = Leg<C>;
  uint32_t lo[2][4], hi[2][4];
  float s[2], c[2];
  __device__ __forceinline__ MmaSlicesLeg(const UnitLeg<C>& un, int, bool keep) {
    float d0, m0, d1, m1;
    un.template block<0>(d0, m0, lo[0], hi[0]);
    un.template block<1>(d1, m1, lo[1], hi[1]);
    s[0] = keep ? d0 : 0.f;
    s[1] = keep ? d1 : 0.f;
    if constexpr (L::MIN) {
      c[0] = keep ? fmaf(-1024.f, d0, m0) : 0.f;
      c[1] = keep ? fmaf(-1024.f, d1, m1) : 0.f;
    } else {
      c[0] = -(1024.f + L::ZP) * s[0];
      c[1] = -(1024.f + L::ZP) * s[1];
    }
  }
  static __device__ __forceinline__ int koff(int u) { return 64 * u; }
  template <int S>
  static constexpr int xstep() { return 8 * S; }
  template <int S>
  __device__ __forceinline__ void get(uint32_t f[4]) const {
    constexpr int b = S >> 2, t = S & 3, dw = 2 * (t & 1);
    if (t < 2)
      slice8(lo[b][dw], lo[b][dw + 1], s[b], c[b], f);
    else
      slice8(hi[b][dw], hi[b][dw + 1], s[b], c[b], f);
  }
};
template <> struct MmaSlices<Q4_1> : MmaSlicesLeg<Q4_1> { using MmaSlicesLeg<Q4_1>::MmaSlicesLeg; };
template <> struct MmaSlices<Q5_0> : MmaSlicesLeg<Q5_0> { using MmaSlicesLeg<Q5_0>::MmaSlicesLeg; };
template <> struct MmaSlices<Q5_1> : MmaSlicesLeg<Q5_1> { using MmaSlicesLeg<Q5_1>::MmaSlicesLeg; };

}  // namespace
}  // namespace kq
