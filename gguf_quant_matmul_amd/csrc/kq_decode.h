// Scalar reference-style decode of 8 consecutive values of a weight row,
// shared by kq_dequantize and the generic (odd-shape) GEMV.  Every value is
// the codec formula rounded once to float32 (see kq_dequant.hip).
#pragma once

#include "kq_internal.h"

namespace kq {

// 8 bytes at a 2-byte-aligned address as two dwords.
__device__ __forceinline__ u32x2 ld8_a2(const uint8_t* p) {
  const uint32_t a = ld_u16(p), b = ld_u16(p + 2), c = ld_u16(p + 4), d = ld_u16(p + 6);
  return u32x2{a | (b << 16), c | (d << 16)};
}

template <int C>
__device__ __forceinline__ void decode8(const uint8_t* __restrict__ row, int64_t v0, float out[8]);

template <>
__device__ __forceinline__ void decode8<Q8_0>(const uint8_t* __restrict__ row, int64_t v0, float out[8]) {
  const uint8_t* blk = row + (v0 / 32) * 34;
  const float d = f16_to_f32(ld_u16(blk));
  const u32x2 c = ld8_a2(blk + 2 + (v0 % 32));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = (int)(int8_t)(((i < 4 ? c.x : c.y) >> (8 * (i & 3))) & 0xFFu);
    out[i] = d * (float)q;
  }
}

template <>
__device__ __forceinline__ void decode8<Q4_0>(const uint8_t* __restrict__ row, int64_t v0, float out[8]) {
  const uint8_t* blk = row + (v0 / 32) * 18;
  const float d = f16_to_f32(ld_u16(blk));
  const int vb = (int)(v0 % 32);
  const u32x2 c = ld8_a2(blk + 2 + (vb & 15));
  const int sh = vb >= 16 ? 4 : 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = (int)((((i < 4 ? c.x : c.y) >> (8 * (i & 3) + sh))) & 15u);
    out[i] = d * (float)(q - 8);
  }
}

// q4_1, q5_0, q5_1: d*q + m by one fma (the exact value rounded once), or
// d*(q - 16) (exact)
template <int C>
__device__ __forceinline__ void decode8_leg(const uint8_t* __restrict__ row, int64_t v0, float out[8]) {
  using L = Leg<C>;
  const uint8_t* blk = row + (v0 / 32) * L::BB;  // 2-byte aligned
  const int vb = (int)(v0 % 32);
  const float d = f16_to_f32(ld_u16(blk));
  const float m = L::MIN ? f16_to_f32(ld_u16(blk + 2)) : 0.f;
  const uint32_t qh = L::QH >= 0 ? (ld_u16(blk + (L::QH >= 0 ? L::QH : 0)) |
                                    (ld_u16(blk + (L::QH >= 0 ? L::QH : 0) + 2) << 16))
                                 : 0u;
  const u32x2 c = ld8_a2(blk + L::QS + (vb & 15));
  const int sh = vb >= 16 ? 4 : 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo4 = ((i < 4 ? c.x : c.y) >> (8 * (i & 3) + sh)) & 15u;
    const int q = (int)(lo4 | (((qh >> (vb + i)) & 1u) << 4));
    out[i] = L::MIN ? fmaf(d, (float)q, m) : d * (float)(q - L::ZP);
  }
}
template <>
__device__ __forceinline__ void decode8<Q4_1>(const uint8_t* __restrict__ row, int64_t v0, float out[8]) {
  decode8_leg<Q4_1>(row, v0, out);
}
template <>
__device__ __forceinline__ void decode8<Q5_0>(const uint8_t* __restrict__ row, int64_t v0, float out[8]) {
  decode8_leg<Q5_0>(row, v0, out);
}
template <>
__device__ __forceinline__ void decode8<Q5_1>(const uint8_t* __restrict__ row, int64_t v0, float out[8]) {
  decode8_leg<Q5_1>(row, v0, out);
}

template <>
__device__ __forceinline__ void decode8<Q2_K>(const uint8_t* __restrict__ row, int64_t v0, float out[8]) {
  const uint8_t* blk = row + (v0 / 256) * 84;  // 4-byte aligned: rows are multiples of 84 bytes
  const int vi = (int)(v0 % 256);
  const int h = vi / 128, c = (vi % 128) / 32, l0 = vi % 32;
  const uint32_t sb = blk[vi / 16];
  const uint32_t dd = ld_u32(blk + 80);
  const float dsc = f16_to_f32(dd) * (float)(sb & 15u);        // exact
  const float dm = f16_to_f32(dd >> 16) * (float)(sb >> 4);    // exact
  const u32x2 q = *(const u32x2*)(blk + 16 + 32 * h + l0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t code = ((i < 4 ? q.x : q.y) >> (8 * (i & 3) + 2 * c)) & 3u;
    out[i] = dsc * (float)code - dm;  // one rounding
  }
}

template <>
__device__ __forceinline__ void decode8<Q3_K>(const uint8_t* __restrict__ row, int64_t v0, float out[8]) {
  const uint8_t* blk = row + (v0 / 256) * 110;  // 2-byte aligned
  const int vi = (int)(v0 % 256);
  const int h = vi / 128, c = (vi % 128) / 32, l0 = vi % 32, j = vi / 16;
  const uint32_t lo4 = (j < 8 ? blk[96 + j] : (blk[96 + j - 8] >> 4)) & 15u;
  const uint32_t hi2 = (blk[104 + (j & 3)] >> (2 * (j >> 2))) & 3u;
  const float dsc = f16_to_f32(ld_u16(blk + 108)) * (float)((int)(lo4 | (hi2 << 4)) - 32);  // exact
  const u32x2 q = ld8_a2(blk + 32 + 32 * h + l0);
  const u32x2 hm = ld8_a2(blk + l0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t low2 = ((i < 4 ? q.x : q.y) >> (8 * (i & 3) + 2 * c)) & 3u;
    const uint32_t hb = ((i < 4 ? hm.x : hm.y) >> (8 * (i & 3) + 4 * h + c)) & 1u;
    out[i] = dsc * (float)((int)(low2 | (hb << 2)) - 4);  // exact
  }
}

template <>
__device__ __forceinline__ void decode8<Q4_K>(const uint8_t* __restrict__ row, int64_t v0, float out[8]) {
  const uint8_t* blk = row + (v0 / 256) * 144;  // 16-byte aligned: rows are multiples of 144 bytes
  const int vi = (int)(v0 % 256);
  const int j = vi / 32, l0 = vi % 32;
  const u32x4 h = ld_16B(blk);
  const float d = f16_to_f32(h.x), dmin = f16_to_f32(h.x >> 16);
  uint32_t sc, m;
  q4k_scale_min(h.y, h.z, h.w, j, sc, m);
  const float dsc = d * (float)sc;   // exact
  const float dm = dmin * (float)m;  // exact
  const u32x2 c = *(const u32x2*)(blk + 16 + 32 * (j / 2) + l0);
  const int sh = (j & 1) ? 4 : 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t q = (((i < 4 ? c.x : c.y) >> (8 * (i & 3) + sh))) & 15u;
    out[i] = dsc * (float)q - dm;  // one rounding
  }
}

template <>
__device__ __forceinline__ void decode8<Q5_K>(const uint8_t* __restrict__ row, int64_t v0, float out[8]) {
  const uint8_t* blk = row + (v0 / 256) * 176;  // 16-byte aligned: rows are multiples of 176 bytes
  const int vi = (int)(v0 % 256);
  const int j = vi / 32, l0 = vi % 32;
  const u32x4 h = ld_16B(blk);
  const float d = f16_to_f32(h.x), dmin = f16_to_f32(h.x >> 16);
  uint32_t sc, m;
  q4k_scale_min(h.y, h.z, h.w, j, sc, m);
  const float dsc = d * (float)sc;   // exact
  const float dm = dmin * (float)m;  // exact
  const u32x2 c = *(const u32x2*)(blk + 48 + 32 * (j / 2) + l0);
  const u32x2 hb = *(const u32x2*)(blk + 16 + l0);
  const int sh = (j & 1) ? 4 : 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo = (((i < 4 ? c.x : c.y) >> (8 * (i & 3) + sh))) & 15u;
    const uint32_t hi = (((i < 4 ? hb.x : hb.y) >> (8 * (i & 3) + j))) & 1u;
    out[i] = dsc * (float)(lo | (hi << 4)) - dm;  // one rounding
  }
}

template <>
__device__ __forceinline__ void decode8<Q6_K>(const uint8_t* __restrict__ row, int64_t v0, float out[8]) {
  const uint8_t* blk = row + (v0 / 256) * 210;
  const int vi = (int)(v0 % 256);
  const int h = vi / 128, r = vi % 128, c = r / 32, l0 = r % 32;
  const u32x2 ql = ld8_a2(blk + 64 * h + l0 + 32 * (c & 1));
  const u32x2 qh = ld8_a2(blk + 128 + 32 * h + l0);
  const float d = f16_to_f32(ld_u16(blk + 208));
  const float dsc = d * (float)(int8_t)blk[192 + vi / 16];  // exact
  const int lsh = c < 2 ? 0 : 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lw = i < 4 ? ql.x : ql.y, hw = i < 4 ? qh.x : qh.y;
    const uint32_t lo4 = (lw >> (8 * (i & 3) + lsh)) & 15u;
    const uint32_t hi2 = (hw >> (8 * (i & 3) + 2 * c)) & 3u;
    out[i] = dsc * (float)((int)(lo4 | (hi2 << 4)) - 32);
  }
}

// Eight codes (two dwords of code bytes) -> eight float16 weights
// fma(1024 + code, s, c), each rounded to float32 and then to float16 (both to
// nearest even): per byte pair one v_perm_b32 builds the float16 pair
// (1024 + code), two v_fma_mix_f32 take its halves through the affine map,
// one v_cvt_pk_f16_f32 packs the results.  The float32 results pass through
// an empty register-only asm statement so the compiler does not fold each map
// and conversion into v_fma_mixlo/hi_f16, which write half a register and
// issue at about half the rate of this sequence on gfx950.
__device__ __forceinline__ void slice8(uint32_t c0, uint32_t c1, float s, float c, uint32_t f[4]) {
  const uint32_t p[4] = {pair01(c0), pair23(c0), pair01(c1), pair23(c1)};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2_t h = as_h2(p[i]);
    v[2 * i] = fmaf((float)h.x, s, c);
    v[2 * i + 1] = fmaf((float)h.y, s, c);
  }
  asm("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = pack_h2(v[2 * i], v[2 * i + 1]);
}

}  // namespace kq
