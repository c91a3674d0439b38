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
//   q6_K 210 B: [0:128] ql, [128:192] qh, [192:208] int8 scales, [208:210] d;
//         v -> h=v/128, c=(v%128)/32, l=v%32: low 4 bits from
//         ql[64h + l + 32(c&1)] (low nibble if c<2), high 2 bits
//         (qh[32h+l] >> 2c) & 3; value = (d*scales[v/16])*(q-32)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

enum Codec : int { Q4_0 = 2, Q8_0 = 8, Q4_K = 12, Q6_K = 14 };

template <int C> struct Geo;
template <> struct Geo<Q4_0> { static constexpr int BV = 32;  static constexpr int BB = 18; };
template <> struct Geo<Q8_0> { static constexpr int BV = 32;  static constexpr int BB = 34; };
template <> struct Geo<Q4_K> { static constexpr int BV = 256; static constexpr int BB = 144; };
template <> struct Geo<Q6_K> { static constexpr int BV = 256; static constexpr int BB = 210; };

static_assert(Geo<Q4_K>::BB == 2 + 2 + 12 + 128, "q4_K superblock bytes");
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

// ---------------------------------------------------------------------------
// launchers (defined in the kernel translation units)
// ---------------------------------------------------------------------------

hipError_t launch_dequantize(int codec, const uint8_t* w, int64_t rows, int64_t k, int64_t row_bytes,
                             void* out, int f16out, hipStream_t s);
hipError_t launch_qmv(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t row_bytes,
                      const half_t* x, int m, void* y, int f16out, hipStream_t s);
hipError_t launch_qmm(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t row_bytes,
                      const half_t* x, int64_t m, void* y, int f16out, hipStream_t s);
hipError_t launch_gather_qmm_seg(int codec, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k,
                                 int64_t row_bytes, const half_t* x, int64_t rows, const uint32_t* map,
                                 const uint32_t* counts, int64_t cap, void* y, int f16out, hipStream_t s);
hipError_t launch_seg_mma(int codec, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k, int64_t row_bytes,
                          const half_t* x, int64_t rows, const uint32_t* map, const uint32_t* counts, int64_t cap,
                          void* y, int f16out, hipStream_t s);
hipError_t launch_gather_qmv(int codec, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k,
                             int64_t row_bytes, const half_t* x, const uint32_t* ids, int64_t rows, void* y,
                             int f16out, hipStream_t s);
// GLU epilogues of the MoE GLU gather (kq.h KQ_GLU_* carry the same values)
constexpr int GLU_SILU = 0, GLU_GELU_TANH = 1, GLU_SILU_LIMIT = 2;
hipError_t launch_moe_glu_gather(int codec, const uint8_t* gate_w, const uint8_t* up_w, int64_t n_experts, int64_t n,
                                 int64_t k, int64_t row_bytes, const half_t* x, const uint32_t* ids, int64_t rows,
                                 int64_t top_k, int act, float limit, void* y, int f16out, hipStream_t s);
hipError_t launch_gather_mix(const void* y, int64_t rows, int64_t n, const uint32_t* inv_order, const float* scores,
                             int64_t tokens, int64_t top_k, void* out, int f16, hipStream_t s);
hipError_t launch_tile_map(const uint32_t* ids, int64_t rows, int64_t n_experts, uint32_t* map,
                           uint32_t* counts, int64_t cap, uint32_t* status, hipStream_t s);
hipError_t launch_quantize(int codec, const float* w, int64_t rows, int64_t k, int64_t row_bytes,
                           uint8_t* out, hipStream_t s);

}  // namespace kq
