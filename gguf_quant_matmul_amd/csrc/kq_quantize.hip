// kq_quantize: float32 weights -> wire bytes (mlx-kquant bindings.cpp page,
// quantize docstring; no importance vector).
//
// The algorithm is not on the pages; this is plain round-to-nearest against
// the STORED fp16 block parameters, every step an IEEE float32 operation
// (correctly rounded division, rint = round half to even, float16 by RNE) in
// this order:
//   q8_0 : d = f16(amax/127);            q = rint(w/D)
//   q4_0 : d = f16(amax/7);              q = rint(w/D) + 8
//   q4_K : per 32 values lo = min(0, min w), hi = max w,
//          scale = (hi - lo)/15, min = -lo;
//          d = f16(max scale/63), dmin = f16(max min/63);
//          sc = rint(scale/D), m = rint(min/DM) (0..63);
//          q = rint((w + DM*m)/(D*sc))
//   q4_1 : d = f16((max w - min w)/15), m = f16(min w); q = rint((w - M)/D)
//   q5_0 : d = f16(amax/15);             q = rint(w/D) + 16
//   q5_1 : d = f16((max w - min w)/31), m = f16(min w); q = rint((w - M)/D)
//   q5_K : as q4_K with scale = (hi - lo)/31 and q in 0..31
//   q2_K : per 16 values lo = min(0, min w), hi = max w, scale = (hi-lo)/3,
//          min = -lo; d = f16(max scale/15), dmin = f16(max min/15);
//          sc = rint(scale/D), m = rint(min/DM) (0..15);
//          q = rint((w + DM*m)/(D*sc)) (0..3)
//   q3_K : per 16 values scale = amax/3; d = f16(max scale/31);
//          sc = rint(scale/D) (-32..31); q = rint(w/(D*sc)) (-4..3)
//   q6_K : per 16 values scale = amax/31; d = f16(max scale/127);
//          sc = rint(scale/D) (-128..127); q = rint(w/(D*sc)) + 32
// Codes are clamped to the codec's range, then moved to the nearest point of
// the block's decoded grid among q-1, q, q+1 (distance |w - decode(q)| in
// float64, ties to the lower code).  A zero grid step gives the zero-point
// code (q8_0 0, q4_0 8, q4_1 and q5_1 0, q5_0 16, q2_K, q3_K, q4_K and q5_K
// 0, q6_K 32).  One thread per block (32-value codecs) or superblock (the K
// codecs);
// not a hot path.
#include "kq_internal.h"

#pragma clang fp contract(off)

namespace kq {
namespace {

__device__ __forceinline__ uint32_t f16_bits(float v) { return __builtin_bit_cast(uint16_t, (half_t)v); }
__device__ __forceinline__ float f16_val(uint32_t b) { return (float)__builtin_bit_cast(half_t, (uint16_t)b); }
__device__ __forceinline__ float clampf(float v, float lo, float hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Nearest grid point among q0-1, q0, q0+1 (clamped), first minimum wins.
template <typename Dec>
__device__ __forceinline__ int nearest(float w, int q0, int lo, int hi, Dec dec) {
  const double w64 = (double)w;
  int best = q0 - 1 < lo ? lo : q0 - 1;
  double be = fabs(w64 - (double)dec(best));
#pragma unroll
  for (int dlt = 0; dlt <= 1; ++dlt) {
    int c = q0 + dlt;
    c = c < lo ? lo : (c > hi ? hi : c);
    const double e = fabs(w64 - (double)dec(c));
    if (e < be) { be = e; best = c; }
  }
  return best;
}

__device__ __forceinline__ void st_u16(uint8_t* p, uint32_t v) { *(uint16_t*)p = (uint16_t)v; }

__global__ __launch_bounds__(256) void quant_q8_0(const float* __restrict__ w, int64_t nblocks, int kb,
                                                  int64_t row_bytes, uint8_t* __restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nblocks) return;
  const int64_t r = g / kb, b = g % kb;
  const float* x = w + (r * kb + b) * 32;
  float amax = 0.f;
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const uint32_t db = f16_bits(amax / 127.f);
  const float D = f16_val(db);
  uint8_t* o = out + r * row_bytes + b * 34;
  st_u16(o, db);
  for (int i = 0; i < 32; i += 2) {
    int q[2];
    for (int t = 0; t < 2; ++t) {
      if (D == 0.f) { q[t] = 0; continue; }
      const float v = x[i + t];
      const int q0 = (int)clampf(rintf(v / D), -128.f, 127.f);
      q[t] = nearest(v, q0, -128, 127, [D](int c) { return D * (float)c; });
    }
    st_u16(o + 2 + i, (uint32_t)(q[0] & 255) | ((uint32_t)(q[1] & 255) << 8));
  }
}

__global__ __launch_bounds__(256) void quant_q4_0(const float* __restrict__ w, int64_t nblocks, int kb,
                                                  int64_t row_bytes, uint8_t* __restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nblocks) return;
  const int64_t r = g / kb, b = g % kb;
  const float* x = w + (r * kb + b) * 32;
  float amax = 0.f;
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const uint32_t db = f16_bits(amax / 7.f);
  const float D = f16_val(db);
  int q[32];
  for (int i = 0; i < 32; ++i) {
    if (D == 0.f) { q[i] = 8; continue; }
    const float v = x[i];
    const int q0 = (int)clampf(rintf(v / D) + 8.f, 0.f, 15.f);
    q[i] = nearest(v, q0, 0, 15, [D](int c) { return D * (float)(c - 8); });
  }
  uint8_t* o = out + r * row_bytes + b * 18;
  st_u16(o, db);
  for (int i = 0; i < 16; i += 2)
    st_u16(o + 2 + i, (uint32_t)(q[i] | (q[i + 16] << 4)) | ((uint32_t)(q[i + 1] | (q[i + 17] << 4)) << 8));
}

// q4_1, q5_0, q5_1: d, [m], [qh as a little-endian uint32], qs; blocks are
// 2-byte aligned, so every store is 2 bytes.
template <int C>
__global__ __launch_bounds__(256) void quant_leg(const float* __restrict__ w, int64_t nblocks, int kb,
                                                 int64_t row_bytes, uint8_t* __restrict__ out) {
  using L = Leg<C>;
  constexpr int QMAX = C == Q4_1 ? 15 : 31;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nblocks) return;
  const int64_t r = g / kb, b = g % kb;
  const float* x = w + (r * kb + b) * 32;
  uint32_t db, mb = 0;
  float D, M = 0.f;
  if constexpr (L::MIN) {
    float lo = x[0], hi = x[0];
    for (int i = 1; i < 32; ++i) { lo = fminf(lo, x[i]); hi = fmaxf(hi, x[i]); }
    db = f16_bits((hi - lo) / (float)QMAX);
    mb = f16_bits(lo);
    D = f16_val(db);
    M = f16_val(mb);
  } else {
    float amax = 0.f;
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
    db = f16_bits(amax / 15.f);
    D = f16_val(db);
  }
  int q[32];
  for (int i = 0; i < 32; ++i) {
    const float v = x[i];
    if (D == 0.f) {
      q[i] = L::ZP;
    } else if constexpr (L::MIN) {
      const int q0 = (int)clampf(rintf((v - M) / D), 0.f, (float)QMAX);
      q[i] = nearest(v, q0, 0, QMAX, [D, M](int c) { return D * (float)c + M; });
    } else {
      const int q0 = (int)clampf(rintf(v / D) + 16.f, 0.f, 31.f);
      q[i] = nearest(v, q0, 0, 31, [D](int c) { return D * (float)(c - 16); });
    }
  }
  uint8_t* o = out + r * row_bytes + b * L::BB;
  st_u16(o, db);
  if constexpr (L::MIN) st_u16(o + 2, mb);
  if constexpr (L::QH >= 0) {
    uint32_t qh = 0;
    for (int i = 0; i < 32; ++i) qh |= (uint32_t)(q[i] >> 4) << i;
    st_u16(o + L::QH, qh & 0xFFFFu);
    st_u16(o + L::QH + 2, qh >> 16);
  }
  for (int i = 0; i < 16; i += 2)
    st_u16(o + L::QS + i, (uint32_t)((q[i] & 15) | ((q[i + 16] & 15) << 4)) |
                              ((uint32_t)((q[i + 1] & 15) | ((q[i + 17] & 15) << 4)) << 8));
}

// q4_K (QMAX 15, 144-byte superblocks) and q5_K (QMAX 31, 176 bytes: the
// same header, then qh[32] with bit j of qh[l] the fifth bit of value l of
// sub-block j, then the low nibbles laid out as q4_K's qs)
template <int QMAX>
__global__ __launch_bounds__(256) void quant_k_affine(const float* __restrict__ w, int64_t nsb, int kb,
                                                      int64_t row_bytes, uint8_t* __restrict__ out) {
  constexpr bool Q5 = QMAX == 31;
  constexpr int BB = Q5 ? 176 : 144, QS = Q5 ? 48 : 16;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nsb) return;
  const int64_t r = g / kb, b = g % kb;
  const float* x = w + (r * kb + b) * 256;
  float scale[8], mins[8];
  float smax = 0.f, mmax = 0.f;
  for (int j = 0; j < 8; ++j) {
    float lo = x[32 * j], hi = x[32 * j];
    for (int i = 1; i < 32; ++i) { lo = fminf(lo, x[32 * j + i]); hi = fmaxf(hi, x[32 * j + i]); }
    lo = fminf(0.f, lo);
    scale[j] = (hi - lo) / (float)QMAX;
    mins[j] = -lo;
    smax = j ? fmaxf(smax, scale[j]) : scale[j];
    mmax = j ? fmaxf(mmax, mins[j]) : mins[j];
  }
  const uint32_t db = f16_bits(smax / 63.f), mb = f16_bits(mmax / 63.f);
  const float D = f16_val(db), DM = f16_val(mb);
  int sc[8], m[8];
  for (int j = 0; j < 8; ++j) {
    sc[j] = D > 0.f ? (int)clampf(rintf(scale[j] / D), 0.f, 63.f) : 0;
    m[j] = DM > 0.f ? (int)clampf(rintf(mins[j] / DM), 0.f, 63.f) : 0;
  }
  uint8_t* o = out + r * row_bytes + b * BB;  // 16-byte aligned
  uint32_t s[12];
  for (int j = 0; j < 4; ++j) {
    s[j] = (uint32_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
    s[j + 4] = (uint32_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
    s[j + 8] = (uint32_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
  }
  u32x4 hdr;
  hdr.x = db | (mb << 16);
  hdr.y = s[0] | (s[1] << 8) | (s[2] << 16) | (s[3] << 24);
  hdr.z = s[4] | (s[5] << 8) | (s[6] << 16) | (s[7] << 24);
  hdr.w = s[8] | (s[9] << 8) | (s[10] << 16) | (s[11] << 24);
  *(u32x4*)o = hdr;
  uint32_t qh[8];
  for (int i = 0; i < 8; ++i) qh[i] = 0;
  for (int p = 0; p < 4; ++p) {  // sub-block pair (2p low nibbles, 2p+1 high nibbles)
    uint32_t word[8];
    for (int i = 0; i < 8; ++i) word[i] = 0;
    for (int half = 0; half < 2; ++half) {
      const int j = 2 * p + half;
      const float S = D * (float)sc[j], MN = DM * (float)m[j];
      for (int l = 0; l < 32; ++l) {
        int q;
        if (S == 0.f) {
          q = 0;
        } else {
          const float v = x[32 * j + l];
          const int q0 = (int)clampf(rintf((v + MN) / S), 0.f, (float)QMAX);
          q = nearest(v, q0, 0, QMAX, [S, MN](int c) { return S * (float)c - MN; });
        }
        word[l >> 2] |= (uint32_t)(q & 15) << (8 * (l & 3) + 4 * half);
        if (Q5) qh[l >> 2] |= (uint32_t)(q >> 4) << (8 * (l & 3) + j);
      }
    }
    *(u32x4*)(o + QS + 32 * p) = u32x4{word[0], word[1], word[2], word[3]};
    *(u32x4*)(o + QS + 32 * p + 16) = u32x4{word[4], word[5], word[6], word[7]};
  }
  if (Q5) {
    *(u32x4*)(o + 16) = u32x4{qh[0], qh[1], qh[2], qh[3]};
    *(u32x4*)(o + 32) = u32x4{qh[4], qh[5], qh[6], qh[7]};
  }
}

__global__ __launch_bounds__(256) void quant_q2_k(const float* __restrict__ w, int64_t nsb, int kb, int64_t row_bytes,
                                                  uint8_t* __restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nsb) return;
  const int64_t r = g / kb, b = g % kb;
  const float* x = w + (r * kb + b) * 256;
  float scale[16], mins[16];
  float smax = 0.f, mmax = 0.f;
  for (int j = 0; j < 16; ++j) {
    float lo = x[16 * j], hi = x[16 * j];
    for (int i = 1; i < 16; ++i) { lo = fminf(lo, x[16 * j + i]); hi = fmaxf(hi, x[16 * j + i]); }
    lo = fminf(0.f, lo);
    scale[j] = (hi - lo) / 3.f;
    mins[j] = -lo;
    smax = j ? fmaxf(smax, scale[j]) : scale[j];
    mmax = j ? fmaxf(mmax, mins[j]) : mins[j];
  }
  const uint32_t db = f16_bits(smax / 15.f), mb = f16_bits(mmax / 15.f);
  const float D = f16_val(db), DM = f16_val(mb);
  uint8_t* o = out + r * row_bytes + b * 84;  // 4-byte aligned
  uint32_t sw[4] = {0, 0, 0, 0}, qw[16];
  for (int i = 0; i < 16; ++i) qw[i] = 0;
  for (int j = 0; j < 16; ++j) {
    const int sc = D > 0.f ? (int)clampf(rintf(scale[j] / D), 0.f, 15.f) : 0;
    const int m = DM > 0.f ? (int)clampf(rintf(mins[j] / DM), 0.f, 15.f) : 0;
    sw[j >> 2] |= (uint32_t)(sc | (m << 4)) << (8 * (j & 3));
    const float S = D * (float)sc, MN = DM * (float)m;
    for (int i = 0; i < 16; ++i) {
      const int v = 16 * j + i;
      int q;
      if (S == 0.f) {
        q = 0;
      } else {
        const float xv = x[v];
        const int q0 = (int)clampf(rintf((xv + MN) / S), 0.f, 3.f);
        q = nearest(xv, q0, 0, 3, [S, MN](int c) { return S * (float)c - MN; });
      }
      const int h = v / 128, c = (v % 128) / 32, l = v % 32, p = 32 * h + l;
      qw[p >> 2] |= (uint32_t)q << (8 * (p & 3) + 2 * c);
    }
  }
  for (int i = 0; i < 4; ++i) *(uint32_t*)(o + 4 * i) = sw[i];
  for (int i = 0; i < 16; ++i) *(uint32_t*)(o + 16 + 4 * i) = qw[i];
  *(uint32_t*)(o + 80) = db | (mb << 16);
}

__global__ __launch_bounds__(256) void quant_q3_k(const float* __restrict__ w, int64_t nsb, int kb, int64_t row_bytes,
                                                  uint8_t* __restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nsb) return;
  const int64_t r = g / kb, b = g % kb;
  const float* x = w + (r * kb + b) * 256;
  float scale[16];
  float smax = 0.f;
  for (int j = 0; j < 16; ++j) {
    float amax = 0.f;
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[16 * j + i]));
    scale[j] = amax / 3.f;
    smax = j ? fmaxf(smax, scale[j]) : scale[j];
  }
  const uint32_t db = f16_bits(smax / 31.f);
  const float D = f16_val(db);
  uint8_t* o = out + r * row_bytes + b * 110;  // 2-byte aligned
  uint32_t hm[8], qw[16], sb[3] = {0, 0, 0};
  for (int i = 0; i < 8; ++i) hm[i] = 0;
  for (int i = 0; i < 16; ++i) qw[i] = 0;
  for (int j = 0; j < 16; ++j) {
    const int sc = D > 0.f ? (int)clampf(rintf(scale[j] / D), -32.f, 31.f) : 0;
    const uint32_t st = (uint32_t)(sc + 32);
    const int lb = j & 7;
    sb[lb >> 2] |= (st & 15u) << (8 * (lb & 3) + 4 * (j >> 3));
    sb[2] |= (st >> 4) << (8 * (j & 3) + 2 * (j >> 2));
    const float S = D * (float)sc;
    for (int i = 0; i < 16; ++i) {
      const int v = 16 * j + i;
      int q;
      if (S == 0.f) {
        q = 0;
      } else {
        const float xv = x[v];
        const int q0 = (int)clampf(rintf(xv / S), -4.f, 3.f);
        q = nearest(xv, q0, -4, 3, [S](int c) { return S * (float)c; });
      }
      const uint32_t u = (uint32_t)(q + 4);
      const int h = v / 128, c = (v % 128) / 32, l = v % 32, p = 32 * h + l;
      qw[p >> 2] |= (u & 3u) << (8 * (p & 3) + 2 * c);
      hm[l >> 2] |= (u >> 2) << (8 * (l & 3) + 4 * h + c);
    }
  }
  for (int i = 0; i < 8; ++i) { st_u16(o + 4 * i, hm[i] & 0xFFFFu); st_u16(o + 4 * i + 2, hm[i] >> 16); }
  for (int i = 0; i < 16; ++i) { st_u16(o + 32 + 4 * i, qw[i] & 0xFFFFu); st_u16(o + 32 + 4 * i + 2, qw[i] >> 16); }
  for (int i = 0; i < 3; ++i) { st_u16(o + 96 + 4 * i, sb[i] & 0xFFFFu); st_u16(o + 96 + 4 * i + 2, sb[i] >> 16); }
  st_u16(o + 108, db);
}

__global__ __launch_bounds__(256) void quant_q6_k(const float* __restrict__ w, int64_t nsb, int kb, int64_t row_bytes,
                                                  uint8_t* __restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nsb) return;
  const int64_t r = g / kb, b = g % kb;
  const float* x = w + (r * kb + b) * 256;
  float scale[16];
  float smax = 0.f;
  for (int j = 0; j < 16; ++j) {
    float amax = 0.f;
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[16 * j + i]));
    scale[j] = amax / 31.f;
    smax = j ? fmaxf(smax, scale[j]) : scale[j];
  }
  const uint32_t db = f16_bits(smax / 127.f);
  const float D = f16_val(db);
  int sc[16];
  for (int j = 0; j < 16; ++j) sc[j] = D > 0.f ? (int)clampf(rintf(scale[j] / D), -128.f, 127.f) : 0;
  uint8_t* o = out + r * row_bytes + b * 210;  // 2-byte aligned
  uint32_t ql[32], qh[16];
  for (int i = 0; i < 32; ++i) ql[i] = 0;
  for (int i = 0; i < 16; ++i) qh[i] = 0;
  for (int v = 0; v < 256; ++v) {
    const int j = v / 16;
    const float S = D * (float)sc[j];
    int q;
    if (S == 0.f) {
      q = 32;
    } else {
      const float xv = x[v];
      const int q0 = (int)clampf(rintf(xv / S) + 32.f, 0.f, 63.f);
      q = nearest(xv, q0, 0, 63, [S](int c) { return S * (float)(c - 32); });
    }
    const int h = v / 128, rr = v % 128, c = rr / 32, l = rr % 32;
    const int qi = 64 * h + l + 32 * (c & 1);
    ql[qi >> 2] |= (uint32_t)(q & 15) << (8 * (qi & 3) + (c < 2 ? 0 : 4));
    const int hi = 32 * h + l;
    qh[hi >> 2] |= (uint32_t)(q >> 4) << (8 * (hi & 3) + 2 * c);
  }
  for (int i = 0; i < 32; ++i) { st_u16(o + 4 * i, ql[i] & 0xFFFFu); st_u16(o + 4 * i + 2, ql[i] >> 16); }
  for (int i = 0; i < 16; ++i) { st_u16(o + 128 + 4 * i, qh[i] & 0xFFFFu); st_u16(o + 128 + 4 * i + 2, qh[i] >> 16); }
  for (int j = 0; j < 16; j += 2) st_u16(o + 192 + j, (uint32_t)(sc[j] & 255) | ((uint32_t)(sc[j + 1] & 255) << 8));
  st_u16(o + 208, db);
}

}  // namespace

hipError_t launch_quantize(int codec, const float* w, int64_t rows, int64_t k, int64_t rb, uint8_t* out,
                           hipStream_t s) {
  const int bv = (codec == Q2_K || codec == Q3_K || codec == Q4_K || codec == Q5_K || codec == Q6_K) ? 256 : 32;
  const int kb = (int)(k / bv);
  const int64_t nblk = rows * kb;
  const dim3 grid((unsigned)((nblk + 255) / 256)), block(256);
  switch (codec) {
    case Q8_0: hipLaunchKernelGGL(quant_q8_0, grid, block, 0, s, w, nblk, kb, rb, out); break;
    case Q4_0: hipLaunchKernelGGL(quant_q4_0, grid, block, 0, s, w, nblk, kb, rb, out); break;
    case Q4_1: hipLaunchKernelGGL(quant_leg<Q4_1>, grid, block, 0, s, w, nblk, kb, rb, out); break;
    case Q5_0: hipLaunchKernelGGL(quant_leg<Q5_0>, grid, block, 0, s, w, nblk, kb, rb, out); break;
    case Q5_1: hipLaunchKernelGGL(quant_leg<Q5_1>, grid, block, 0, s, w, nblk, kb, rb, out); break;
    case Q2_K: hipLaunchKernelGGL(quant_q2_k, grid, block, 0, s, w, nblk, kb, rb, out); break;
    case Q3_K: hipLaunchKernelGGL(quant_q3_k, grid, block, 0, s, w, nblk, kb, rb, out); break;
    case Q4_K: hipLaunchKernelGGL(quant_k_affine<15>, grid, block, 0, s, w, nblk, kb, rb, out); break;
    case Q5_K: hipLaunchKernelGGL(quant_k_affine<31>, grid, block, 0, s, w, nblk, kb, rb, out); break;
    case Q6_K: hipLaunchKernelGGL(quant_q6_k, grid, block, 0, s, w, nblk, kb, rb, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kq
