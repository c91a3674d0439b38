// Internal declarations shared by the libkq translation units (HIP, gfx950).
//
// Codec geometry: mlx-kquant README, "Codec reference" table.  Byte layouts
// inside a block are GGUF's:
//   q4_0  18 B: [0:2] d f16, [2:18] 16 bytes; value v<16 low nibble of byte v,
//         v>=16 high nibble of byte v-16; value = d*(q-8)
//   q8_0  34 B: [0:2] d f16, [2:34] int8 codes; value = d*q
//   q4_K 144 B: [0:2] d, [2:4] dmin, [4:16] twelve bytes of 6-bit (sc, m)
//         pairs, [16:144] qs; sub-block j = v/32, byte qs[32*(j/2) + v%32],
//         low nibble for even j; value = (d*sc_j)*q - dmin*m_j
//   q4_1  20 B: [0:2] d, [2:4] m, [4:20] qs (nibbles as q4_0); value = d*q + m
//   q5_0  22 B: [0:2] d, [2:6] qh (uint32), [6:22] qs; fifth bit of value v
//         is bit v of qh; value = d*(q-16)
//   q5_1  24 B: [0:2] d, [2:4] m, [4:8] qh, [8:24] qs; value = d*q + m
//   q2_K  84 B: [0:16] scales (byte j: sub-block j of 16 values, scale in the
//         low nibble, min in the high), [16:80] qs, [80:82] d, [82:84] dmin;
//         v -> h=v/128, c=(v%128)/32, l=v%32: code = (qs[32h+l] >> 2c) & 3;
//         value = (d*sc_j)*q - dmin*m_j, j = v/16
//   q3_K 110 B: [0:32] hmask, [32:96] qs, [96:108] 16 packed 6-bit scales
//         (stored + 32), [108:110] d; v -> h, c, l as q2_K: u = low2 |
//         hbit << 2 with low2 = (qs[32h+l] >> 2c) & 3, hbit = bit 4h+c of
//         hmask[l]; value = d*sc_j*(u - 4)
//   q5_K 176 B: [0:16] as q4_K, [16:48] qh, [48:176] qs; the low four bits
//         as q4_K's nibbles (at qs), the fifth bit of value l of sub-block j
//         is bit j of qh[l]; value = (d*sc_j)*q - dmin*m_j, q in 0..31
//   q6_K 210 B: [0:128] ql, [128:192] qh, [192:208] int8 scales, [208:210] d;
//         v -> h=v/128, c=(v%128)/32, l=v%32: low 4 bits from
//         ql[64h + l + 32(c&1)] (low nibble if c<2), high 2 bits
//         (qh[32h+l] >> 2c) & 3; value = (d*scales[v/16])*(q-32)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

enum Codec : int { Q4_0 = 2, Q4_1 = 3, Q5_0 = 6, Q5_1 = 7, Q8_0 = 8, Q2_K = 10, Q3_K = 11, Q4_K = 12, Q5_K = 13, Q6_K = 14 };

template <int C> struct Geo;
template <> struct Geo<Q4_0> { static constexpr int BV = 32;  static constexpr int BB = 18; };
template <> struct Geo<Q8_0> { static constexpr int BV = 32;  static constexpr int BB = 34; };
template <> struct Geo<Q4_1> { static constexpr int BV = 32;  static constexpr int BB = 20; };
template <> struct Geo<Q5_0> { static constexpr int BV = 32;  static constexpr int BB = 22; };
template <> struct Geo<Q5_1> { static constexpr int BV = 32;  static constexpr int BB = 24; };
template <> struct Geo<Q4_K> { static constexpr int BV = 256; static constexpr int BB = 144; };
template <> struct Geo<Q2_K> { static constexpr int BV = 256; static constexpr int BB = 84; };
template <> struct Geo<Q3_K> { static constexpr int BV = 256; static constexpr int BB = 110; };
template <> struct Geo<Q5_K> { static constexpr int BV = 256; static constexpr int BB = 176; };
template <> struct Geo<Q6_K> { static constexpr int BV = 256; static constexpr int BB = 210; };

static_assert(Geo<Q4_K>::BB == 2 + 2 + 12 + 128, "q4_K superblock bytes");
static_assert(Geo<Q5_K>::BB == 2 + 2 + 12 + 32 + 128, "q5_K superblock bytes");
static_assert(Geo<Q6_K>::BB == 128 + 64 + 16 + 2, "q6_K superblock bytes");
static_assert(Geo<Q8_0>::BB == 2 + 32 && Geo<Q4_0>::BB == 2 + 16, "block bytes");

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
// 16-byte vector with only 4-byte alignment promised: multi-dword global
// loads need dword alignment only.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The legacy 32-value codecs with a minimum or a fifth bit (q4_1, q5_0, q5_1):
// block bytes, whether an fp16 minimum follows d, the byte offsets of qh
// (-1: none) and qs, and the code offset of a codec without a minimum.
template <int C> struct Leg;
template <> struct Leg<Q4_1> { static constexpr int BB = 20, QH = -1, QS = 4, ZP = 0; static constexpr bool MIN = true; };
template <> struct Leg<Q5_0> { static constexpr int BB = 22, QH = 2, QS = 6, ZP = 16; static constexpr bool MIN = false; };
template <> struct Leg<Q5_1> { static constexpr int BB = 24, QH = 4, QS = 8, ZP = 0; static constexpr bool MIN = true; };
template <int C> constexpr bool is_leg() { return C == Q4_1 || C == Q5_0 || C == Q5_1; }
template <int C> constexpr bool is_block32() { return C == Q4_0 || C == Q8_0 || is_leg<C>(); }

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(half_t, (uint16_t)(bits16 & 0xFFFFu));
}

__device__ __forceinline__ uint32_t ld_u16(const uint8_t* p) { return *(const uint16_t*)p; }
__device__ __forceinline__ uint32_t ld_u32(const uint8_t* p) { return *(const uint32_t*)p; }
__device__ __forceinline__ u32x4 ld_16B(const uint8_t* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 ld_16B_a4(const uint8_t* p) {
  u32x4_a4 v = *(const u32x4_a4*)p;
  return u32x4{v.x, v.y, v.z, v.w};
}

// v_perm_b32: byte i of the result is byte sel.byte[i] of the 64-bit value
// {hi, lo} (selectors 0-3 pick lo's bytes, 4-7 hi's bytes).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// ({hi, lo} >> (8 * shift))[31:0]
__device__ __forceinline__ uint32_t alignbyte(uint32_t hi, uint32_t lo, uint32_t shift) {
  return __builtin_amdgcn_alignbyte(hi, lo, shift);
}

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// float32 accumulate += dot(a, b) over two float16 pairs.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// Byte B of a dword as float32 (v_cvt_f32_ubyteB).
template <int B>
__device__ __forceinline__ float byte_f32(uint32_t v) { return (float)((v >> (8 * B)) & 0xFFu); }
// Two float32 -> float16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return __builtin_bit_cast(uint32_t, half2_t{(half_t)a, (half_t)b});
}

// Code bytes (each < 256 after any bias) -> two float16 (1024 + byte) per
// pair: 0x64 as the high byte makes the half 2^10 * (1 + byte/1024).
constexpr uint32_t MAGIC = 0x64646464u;
constexpr uint32_t SEL01 = 0x00050004u;  // [b0, 0x64, b1, 0x64]
constexpr uint32_t SEL23 = 0x00070006u;  // [b2, 0x64, b3, 0x64]
__device__ __forceinline__ uint32_t pair01(uint32_t bytes) { return perm(bytes, MAGIC, SEL01); }
__device__ __forceinline__ uint32_t pair23(uint32_t bytes) { return perm(bytes, MAGIC, SEL23); }

// q4_K: 6-bit scale and min of sub-block j (0..7) from the three packed
// dwords s0 = bytes 0..3, s1 = bytes 4..7, s2 = bytes 8..11 (branch-free).
__device__ __forceinline__ void q4k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int j,
                                              uint32_t& sc, uint32_t& m) {
  const uint32_t sh = 8u * (uint32_t)(j & 3);
  const uint32_t b0 = (s0 >> sh) & 0xFFu, b1 = (s1 >> sh) & 0xFFu, b2 = (s2 >> sh) & 0xFFu;
  const uint32_t sc_lo = b0 & 63u, m_lo = b1 & 63u;
  const uint32_t sc_hi = (b2 & 15u) | ((b0 >> 6) << 4);
  const uint32_t m_hi = (b2 >> 4) | ((b1 >> 6) << 4);
  sc = j < 4 ? sc_lo : sc_hi;
  m = j < 4 ? m_lo : m_hi;
}

// Both sub-blocks 2P and 2P + 1 (P = 0..3) at once.  They sit in bytes
// 2 (P & 1) and 2 (P & 1) + 1 of each scale dword; for P < 2 the six bits are
// whole in s0 (scale) and s1 (min), for P >= 2 the low four come from s2 and
// the top two from s0 / s1.  When P is uniform over a loop, the field offsets
// and widths are computed once outside it.
__device__ __forceinline__ void q4k_scale_min_pair(uint32_t s0, uint32_t s1, uint32_t s2, int P, uint32_t& sc0,
                                                   uint32_t& m0, uint32_t& sc1, uint32_t& m1) {
  const uint32_t sh = 16u * (uint32_t)(P & 1);
  const bool hi = P >= 2;
  const uint32_t a = hi ? s2 : s0, b = hi ? (s2 >> 4) : s1;  // low bits of scale, min
  const uint32_t w = hi ? 4u : 6u, t = hi ? 2u : 0u;        // their width; width of the top bits
  sc0 = __builtin_amdgcn_ubfe(a, sh, w) | (__builtin_amdgcn_ubfe(s0, sh + 6u, t) << 4);
  sc1 = __builtin_amdgcn_ubfe(a, sh + 8u, w) | (__builtin_amdgcn_ubfe(s0, sh + 14u, t) << 4);
  m0 = __builtin_amdgcn_ubfe(b, sh, w) | (__builtin_amdgcn_ubfe(s1, sh + 6u, t) << 4);
  m1 = __builtin_amdgcn_ubfe(b, sh + 8u, w) | (__builtin_amdgcn_ubfe(s1, sh + 14u, t) << 4);
}

// Bit 4 of byte b of the result is bit b of t (b < 4): the fifth bits of
// four consecutive values of a legacy block moved next to their nibbles.
__device__ __forceinline__ uint32_t spread4(uint32_t t) { return (((t & 0xFu) * 0x00204081u) & 0x01010101u) << 4; }
// 5-bit (or 4-bit) code bytes of qs dword i (values 4i..4i+3 low nibbles,
// 16+4i.. high nibbles) of a legacy block with fifth bits qh
template <int C>
__device__ __forceinline__ uint32_t leg_lo(uint32_t qs, uint32_t qh, int i) {
  if constexpr (Leg<C>::QH < 0) return qs & 0x0F0F0F0Fu;
  else return (qs & 0x0F0F0F0Fu) | spread4(qh >> (4 * i));
}
template <int C>
__device__ __forceinline__ uint32_t leg_hi(uint32_t qs, uint32_t qh, int i) {
  if constexpr (Leg<C>::QH < 0) return (qs >> 4) & 0x0F0F0F0Fu;
  else return ((qs >> 4) & 0x0F0F0F0Fu) | spread4(qh >> (16 + 4 * i));
}

// q3_K: signed scale t of the four sub-blocks 4u' + t (u' = unit % 4) from the
// scale dwords A (bytes 4 (u' % 2) .. of the 12, low nibbles for u' < 2, high
// for u' >= 2) and B (bytes 8..11, bits 2u'..2u'+1 of byte t)
__device__ __forceinline__ int q3k_scale(uint32_t A, uint32_t B, int up, int t) {
  const uint32_t lo4 = (A >> (8 * t + 4 * (up >> 1))) & 15u;
  const uint32_t hi2 = (B >> (8 * t + 2 * up)) & 3u;
  return (int)(lo4 | (hi2 << 4)) - 32;
}

// GLU epilogues (kq.h KQ_GLU_* carry the same values)
constexpr int GLU_SILU = 0, GLU_GELU_TANH = 1, GLU_SILU_LIMIT = 2;
// activation rows the GEMV takes (the matrix-core GEMV's A operand has 16)
constexpr int QMV_MAX_M = 16;
// activation rows up to which kq_quantized_matmul takes the matrix-core GEMV
// with several A operands per decoded weight operand (kq_qmv_wide.hip)
constexpr int QMV_WIDE_MAX_M = 64;
// A matrix with so few rows that the wide GEMV's 32-row workgroups leave CUs
// idle (a 256-CU part): it splits K four ways per row group instead of two.
__host__ __device__ constexpr bool wide_narrow(int64_t n) { return (n + 31) / 32 < 256; }
// activation rows up to which the GLU product runs on the GEMV body (two
// matrices' q3_K units fill the registers from two rows on)
constexpr int QMV_GLU_MAX_M = 3;
__host__ __device__ constexpr int qmv_glu_max_m(int codec) { return codec == Q3_K ? 1 : QMV_GLU_MAX_M; }

// Matmul epilogue (mlx-kquant bindings.cpp page, quantized_matmul_residual
// and quantized_matmul_qmv_bias docstrings): per output element
// y = fma(gate, acc, resid) + bias in float32, rounded once to y's type; a
// null term is left out.  All three terms are in y's type: resid [M][N],
// gate [G][N] with row m taking gate row m / gate_div, bias [N].
struct Epi {
  const void* resid;
  const void* gate;
  const void* bias;
  int gate_div;
};
template <bool F16>
__device__ __forceinline__ float ld_out(const void* p, int64_t i) {
  return F16 ? (float)((const half_t*)p)[i] : ((const float*)p)[i];
}
template <bool F16>
__device__ __forceinline__ float epi_apply(const Epi& e, int64_t m, int64_t col, int64_t n, float acc) {
  const float g = e.gate ? ld_out<F16>(e.gate, (int64_t)((int)m / e.gate_div) * n + col) : 1.f;
  const float r = e.resid ? ld_out<F16>(e.resid, m * n + col) : 0.f;
  float v = fmaf(g, acc, r);
  if (e.bias) v += ld_out<F16>(e.bias, col);
  return v;
}

// A finite value beyond the float16 range becomes the largest finite half of
// its sign; infinities and NaN pass (the float16 store of the GLU product).
__device__ __forceinline__ float sat_half(float v) {
  return fabsf(v) <= 3.40282347e38f ? fminf(fmaxf(v, -65504.f), 65504.f) : v;
}
// v rounded to y's type (float16 saturating, float32 unchanged)
template <bool F16>
__device__ __forceinline__ float round_out(float v) {
  return F16 ? (float)(half_t)sat_half(v) : v;
}

// v * sigmoid(t) = v / (1 + 2^(-t log2 e)) from the hardware exp2 and
// reciprocal (about 1 ulp each): a few float32 ulps in all, far below the
// float16 rounding the activations of the GLU matmul take.  t -> -inf gives
// exp2 = inf and a product of 0 (of v's sign); NaN passes.
__device__ __forceinline__ float sigmoid_mul(float v, float t) {
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * t);
  return v * __builtin_amdgcn_rcpf(1.f + e);
}

// GLU epilogues of the mlx-kquant bindings.cpp page (moe_glu_gather_kq
// docstring, its act argument), in float32 on the two float32 products g
// (gate) and u (up):
//   GLU_SILU        silu(g) * u, silu(g) = g sigmoid(g)
//   GLU_GELU_TANH   gelu(g) * u with the tanh form of gelu,
//                   0.5 g (1 + tanh(z)), z = sqrt(2/pi) (g + 0.044715 g^3),
//                   evaluated as g sigmoid(2 z) (the same function:
//                   0.5 (1 + tanh z) = sigmoid(2 z))
//   GLU_SILU_LIMIT  silu(min(g, limit)) * clip(u, -limit, limit)
template <int ACT>
__device__ __forceinline__ float glu_act(float g, float u, float limit) {
  if constexpr (ACT == GLU_SILU) {
    return sigmoid_mul(g, g) * u;
  } else if constexpr (ACT == GLU_GELU_TANH) {
    const float c2 = 1.5957691216057308f;  // 2 sqrt(2 / pi)
    return sigmoid_mul(g, c2 * fmaf(0.044715f * g, g * g, g)) * u;
  } else {
    const float gg = fminf(g, limit);
    return sigmoid_mul(gg, gg) * fminf(fmaxf(u, -limit), limit);
  }
}

// The GLU product of quantized_matmul_glu (mlx-kquant bindings.cpp page, its
// docstring): the activation of the gate product is rounded to y's type, then
// multiplied by the up product in float32 and rounded again.
template <int ACT, bool F16>
__device__ __forceinline__ float glu_rounded(float g, float u) {
  return round_out<F16>(round_out<F16>(glu_act<ACT>(g, 1.f, 0.f)) * u);
}

// Output stores of the GEMM kernels.  EP_EPI applies epi_apply (null terms
// tested per element); EP_RES (y = acc + resid) and EP_RES_GATE (y =
// fma(gate, acc, resid)) are the same store with the terms known present, so
// a kernel can load them without branches.  The GLU product is two passes
// over K: EP_GLU_ACT stores the rounded activation of the gate product in y,
// EP_GLU_MUL multiplies the up product by it.
constexpr int EP_PLAIN = 0, EP_EPI = 1, EP_GLU_ACT = 2, EP_GLU_MUL = 3, EP_RES = 4, EP_RES_GATE = 5;
// The values a store reads (residual and gate, or y's activation), split
// from the store so that a kernel writing many elements can load them all
// first: a load placed after a store to y waits for it, y possibly aliasing.
template <bool F16, int EP>
__device__ __forceinline__ void epi_load(const void* y, int64_t row, int64_t col, int64_t n, const Epi& e, float& a,
                                         float& b) {
  if constexpr (EP == EP_RES || EP == EP_RES_GATE) a = ld_out<F16>(e.resid, row * n + col);
  if constexpr (EP == EP_RES_GATE) b = ld_out<F16>(e.gate, (int64_t)((int)row / e.gate_div) * n + col);
  if constexpr (EP == EP_GLU_MUL) a = ld_out<F16>(y, row * n + col);
}
template <bool F16, int EP, int ACT>
__device__ __forceinline__ void store_pre(void* y, int64_t row, int64_t col, int64_t n, const Epi& e, float v, float a,
                                          float b) {
  if constexpr (EP == EP_EPI) v = epi_apply<F16>(e, row, col, n, v);
  if constexpr (EP == EP_RES) v += a;
  if constexpr (EP == EP_RES_GATE) v = fmaf(b, v, a);
  if constexpr (EP == EP_GLU_ACT) v = round_out<F16>(glu_act<ACT>(v, 1.f, 0.f));
  if constexpr (EP == EP_GLU_MUL) v = round_out<F16>(a * v);
  const int64_t o = row * n + col;
  if (F16)
    ((half_t*)y)[o] = (half_t)v;
  else
    ((float*)y)[o] = v;
}
template <bool F16, int EP, int ACT>
__device__ __forceinline__ void store_out(void* y, int64_t row, int64_t col, int64_t n, const Epi& e, float v) {
  float a = 0.f, b = 1.f;
  epi_load<F16, EP>(y, row, col, n, e, a, b);
  store_pre<F16, EP, ACT>(y, row, col, n, e, v, a, b);
}

// ---------------------------------------------------------------------------
// launchers (defined in the kernel translation units)
// ---------------------------------------------------------------------------

hipError_t launch_dequantize(int codec, const uint8_t* w, int64_t rows, int64_t k, int64_t row_bytes,
                             void* out, int f16out, hipStream_t s);
hipError_t launch_qmv(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t row_bytes,
                      const half_t* x, int m, void* y, int f16out, hipStream_t s);
hipError_t launch_qmv_wide(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t row_bytes,
                           const half_t* x, int m, void* y, int f16out, hipStream_t s);
hipError_t launch_qmv_wide_epi(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t row_bytes,
                               const half_t* x, int m, const Epi& epi, void* y, int f16out, hipStream_t s);
hipError_t launch_qmv_wide_glu_act(int codec, const uint8_t* w_gate, int64_t n, int64_t k, int64_t row_bytes,
                                   const half_t* x, int m, int act, void* y, int f16out, hipStream_t s);
hipError_t launch_qmv_wide_glu_mul(int codec, const uint8_t* w_up, int64_t n, int64_t k, int64_t row_bytes,
                                   const half_t* x, int m, void* y, int f16out, hipStream_t s);
hipError_t launch_qmm(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t row_bytes,
                      const half_t* x, int64_t m, void* y, int f16out, hipStream_t s);
hipError_t launch_gather_qmm_seg(int codec, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k,
                                 int64_t row_bytes, const half_t* x, int64_t rows, const uint32_t* map,
                                 const uint32_t* counts, int64_t cap, void* y, int f16out, hipStream_t s);
hipError_t launch_seg_mma(int codec, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k, int64_t row_bytes,
                          const half_t* x, int64_t rows, const uint32_t* map, const uint32_t* counts, int64_t cap,
                          void* y, int f16out, hipStream_t s);
bool seg_exact_ok(int codec, int64_t k);
hipError_t launch_seg_exact(const uint8_t* w, int64_t n_experts, int64_t n, int64_t k, int64_t row_bytes,
                            const half_t* x, int64_t rows, const uint32_t* map, const uint32_t* counts, int64_t cap,
                            void* y, int f16out, hipStream_t s);
hipError_t launch_gather_qmv(int codec, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k,
                             int64_t row_bytes, const half_t* x, const uint32_t* ids, int64_t rows, void* y,
                             int f16out, hipStream_t s);
hipError_t launch_moe_glu_gather(int codec, const uint8_t* gate_w, const uint8_t* up_w, int64_t n_experts, int64_t n,
                                 int64_t k, int64_t row_bytes, const half_t* x, const uint32_t* ids, int64_t rows,
                                 int64_t top_k, int act, float limit, void* y, int f16out, hipStream_t s);
hipError_t launch_gather_mix(const void* y, int64_t rows, int64_t n, const uint32_t* inv_order, const float* scores,
                             int64_t tokens, int64_t top_k, void* out, int f16, hipStream_t s);
hipError_t launch_qmv_epi(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t row_bytes, const half_t* x,
                          int m, const Epi& epi, void* y, int f16out, hipStream_t s);
hipError_t launch_qmm_epi(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t row_bytes, const half_t* x,
                          int64_t m, const Epi& epi, void* y, int f16out, hipStream_t s);
hipError_t launch_qmm_glu_mul(int codec, const uint8_t* w_up, int64_t n, int64_t k, int64_t row_bytes,
                              const half_t* x, int64_t m, void* y, int f16out, hipStream_t s);
hipError_t launch_qmv_glu(int codec, const uint8_t* w_gate, const uint8_t* w_up, int64_t n, int64_t k,
                          int64_t row_bytes, const half_t* x, int m, int act, void* y, int f16out, hipStream_t s);
hipError_t launch_qmm_glu(int codec, const uint8_t* w_gate, const uint8_t* w_up, int64_t n, int64_t k,
                          int64_t row_bytes, const half_t* x, int64_t m, int act, void* y, int f16out, hipStream_t s);
hipError_t launch_tile_map(const uint32_t* ids, int64_t rows, int64_t n_experts, uint32_t* map,
                           uint32_t* counts, int64_t cap, uint32_t* status, hipStream_t s);
hipError_t launch_quantize(int codec, const float* w, int64_t rows, int64_t k, int64_t row_bytes,
                           uint8_t* out, hipStream_t s);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* out, int64_t groups, hipStream_t s);
// bfloat16 activations; out: 0 float32, 1 float16, 2 bfloat16
hipError_t launch_mm_bf16(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t rb, const void* x, int64_t m,
                          void* y, int out, hipStream_t s);
hipError_t launch_seg_bf16(int codec, const uint8_t* w, int64_t ne, int64_t n, int64_t k, int64_t rb, const void* x,
                           int64_t rows, const uint32_t* map, const uint32_t* counts, int64_t cap, void* y, int out,
                           hipStream_t s);


// Row m and piece r of the 16-byte activation pieces c, c + step, c + 2 step,
// ... of a block whose rows hold kp pieces each: one division for the first
// piece, then an exact carry per step (c + step = (m + step / kp) kp + r +
// step % kp, and r + step % kp < 2 kp), instead of a division by the run-time
// kp for every piece.
struct PieceWalk {
  int m, r, kp, qs, rs;
  __device__ __forceinline__ PieceWalk(int c, int kp_, int step) : kp(kp_) {
    m = c / kp;
    r = c - m * kp;
    qs = step / kp;
    rs = step - qs * kp;
  }
  __device__ __forceinline__ void next() {
    m += qs;
    r += rs;
    if (r >= kp) {
      r -= kp;
      ++m;
    }
  }
};

}  // namespace kq
