// bfloat16 activations: kq_qmv_bf16, kq_qmm_bf16, kq_gather_qmm_seg_bf16.
//
// mlx-kquant bindings.cpp page: quantized_matmul and gather_qmm_seg return
// x's dtype (a float32 x promoted to bfloat16), so a bfloat16 activation is a
// first-class input of the quantized matmuls; the product is
// y = x @ dequant(w)^T as for float16 activations.
//
// Design.  Two codec-generic matrix-core kernels serve the three shapes: a
// GEMV of up to 16 activation rows (bf_mv_kernel), and the prefill GEMM and
// the expert-segment GEMM over a tile map (bl_tile, activations staged in
// LDS):
//  * a GEMV workgroup of sixteen waves shares 16 weight rows and splits K; a
//    matmul workgroup takes 128 weight rows (2 x 16 per wave) and one row
//    tile of up to 16 * XG activation rows (XG 16-row groups);
//  * per 32-value K step each lane decodes 8 consecutive weights of its row
//    (row l & 15 of the wave's group, K values 8 (l >> 4) ..) to their exact
//    float32 values (decode8, one rounding where the codec formula has one)
//    and splits each into a bfloat16 high part and a bfloat16 remainder, so
//    the weight carries 16 significant bits (relative error below 2^-16);
//  * v_mfma_f32_16x16x32_bf16 multiplies the exact bfloat16 activations
//    (lane l holds row l & 15 of a group, K values 8 (l >> 4) ..; the GEMV
//    reads them from global memory, the matmul tile from LDS) by both weight
//    parts, with float32 accumulation;
//  * the store rounds once to float32, float16 or bfloat16 (nearest even).
// The float16 paths' exact integer-code tricks do not carry over: a
// bfloat16 holds integers exactly only below 257, and sc * q reaches 945.
#include "kq_decode.h"

namespace kq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int BF_THREADS = 256;

// 8 float32 -> bfloat16 high parts (truncated) and bfloat16 remainders
// (truncated): v = hi + lo with |v - hi - lo| < 2^-16 |v|.
__device__ __forceinline__ void split8(const float v[8], bf16x8_t& hi, bf16x8_t& lo) {
  u16x8 h, l;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v[i]);
    const float r = v[i] - __builtin_bit_cast(float, b & 0xFFFF0000u);
    h[i] = (uint16_t)(b >> 16);
    l[i] = (uint16_t)(__builtin_bit_cast(uint32_t, r) >> 16);
  }
  hi = __builtin_bit_cast(bf16x8_t, h);
  lo = __builtin_bit_cast(bf16x8_t, l);
}

template <int OUT>
__device__ __forceinline__ void bf_store(void* y, int64_t i, float v) {
  if constexpr (OUT == 0)
    ((float*)y)[i] = v;
  else if constexpr (OUT == 1)
    ((half_t*)y)[i] = (half_t)v;
  else
    ((__bf16*)y)[i] = (__bf16)v;
}

// GEMV (at most 16 activation rows): BV_WAVES waves share 16 weight rows and
// split the 32-value K steps into contiguous ranges; each wave decodes four
// steps before their products, so their loads are in flight together, and the
// waves' parts are added in LDS in wave order.  Many waves per row block keep
// the serial chain of load latencies per wave short (K = 4096: 8 steps).
constexpr int BV_WAVES = 16;

template <int C, int OUT>
__global__ __launch_bounds__(64 * BV_WAVES) void bf_mv_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                             int64_t row_bytes, const __bf16* __restrict__ x, int m,
                                                             void* __restrict__ y) {
  constexpr int G = 4;  // K steps decoded together
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, cu = lane >> 4;
  const int wrow = blockIdx.x * 16 + r;
  const uint8_t* wr = w + (int64_t)(wrow < n ? wrow : n - 1) * row_bytes;  // rows past N: a valid row, not stored
  const __bf16* xr = x + (int64_t)min(r, m - 1) * k + 8 * cu;            // rows past M repeat the last (dropped)
  float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
  const int steps = k / 32;
  const int s0 = (steps * wave) / BV_WAVES, s1 = (steps * (wave + 1)) / BV_WAVES;
  for (int st = s0; st < s1; st += G) {
    bf16x8_t a[G], bh[G], bl[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int sg = min(st + g, s1 - 1);  // a step past the range re-reads the last (its products are skipped)
      float v[8];
      decode8<C>(wr, 32 * sg + 8 * cu, v);
      split8(v, bh[g], bl[g]);
      a[g] = *(const bf16x8_t*)(xr + 32 * sg);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (st + g < s1) {  // uniform
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[g], bh[g], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[g], bl[g], acc, 0, 0, 0);
      }
    }
  }
  __shared__ float4_t part[BV_WAVES - 1][64];
  if (wave > 0) part[wave - 1][lane] = acc;
  __syncthreads();
  if (wave > 0 || wrow >= n) return;
#pragma unroll
  for (int p = 0; p < BV_WAVES - 1; ++p) acc += part[p][lane];
  // lane l holds activation rows 4 (l >> 4) + q of weight row wrow
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 4 * cu + q;
    if (row < m) bf_store<OUT>(y, (int64_t)row * n + wrow, acc[q]);
  }
}

// The matmul tile for more than 16 activation rows: the row tile (16 XG rows)
// is staged in LDS once per 128-value K chunk and shared by the four waves,
// each of which decodes 2 x 16 weight rows (128 per workgroup), so every
// activation fragment comes from LDS and serves four MFMAs (two weight rows,
// two weight parts).  Without the staging each wave read its fragments from
// L2, about 8 KiB per wave per 32-value step.
//
// LDS: a chunk row is 16 chunks of 16 bytes in two planes of 128-byte rows:
// chunk c of row r sits in plane c & 1 at slot (c >> 1) ^ ((r >> 1) & 7).  On
// gfx950 16-byte reads are served per 32-lane half over sixteen 16-byte bank
// slots, lanes exactly 16 apart sharing one without conflict, and 16-byte
// writes 8 lanes at a time over 128 bytes: a fragment read (lane (r, cu), row
// r, chunk 4 s + cu) has lanes 16 apart read the two planes of one chunk pair
// at one slot and each 16 lanes cover all sixteen slots; the staging map below
// has 8 consecutive lanes write 8 slots of one plane row.
constexpr int BL_RG = 2;                // 16-row weight groups per wave
constexpr int BL_BN = 4 * 16 * BL_RG;   // weight rows per workgroup (128)
constexpr int BL_KC = 128;              // K values per staged chunk

__device__ __forceinline__ int bl_off(int rows, int r, int c) {  // bfloat16 elements
  return (c & 1) * rows * 64 + r * 64 + 8 * ((c >> 1) ^ ((r >> 1) & 7));
}

template <int C, int XG, int OUT>
__device__ __forceinline__ void bl_tile(const uint8_t* __restrict__ w, int n, int k, int64_t row_bytes,
                                        const __bf16* __restrict__ x, int64_t r0, int nr, int n0,
                                        void* __restrict__ y) {
  constexpr int ROWS = 16 * XG, XPT = ROWS * (BL_KC / 8) / BF_THREADS;  // 16-byte pieces per thread per chunk
  static_assert(XPT * BF_THREADS == ROWS * (BL_KC / 8), "whole pieces");
  __shared__ __attribute__((aligned(16))) __bf16 xs[2][ROWS * BL_KC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, cu = lane >> 4;
  const uint8_t* wr[BL_RG];
#pragma unroll
  for (int j = 0; j < BL_RG; ++j) {
    const int row = n0 + wave * 16 * BL_RG + 16 * j + r;
    wr[j] = w + (int64_t)(row < n ? row : n - 1) * row_bytes;  // rows past N: a valid row, not stored
  }
  const int xg = (nr + 15) >> 4;  // live 16-row groups
  // staging: piece i of this thread is g = tid + 256 i; its wave-level lane
  // l = g & 63 takes row 4 (g >> 6) + 2 (l >> 5) + ((l & 15) >> 3) and chunk
  // 2 (l & 7) + ((l >> 4) & 1).  Rows past the tile repeat its last row.
  const __bf16* xp[XPT];
  int so[XPT], pc[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int g = tid + BF_THREADS * i, l = g & 63;
    const int row = 4 * (g >> 6) + 2 * (l >> 5) + ((l & 15) >> 3), c = 2 * (l & 7) + ((l >> 4) & 1);
    xp[i] = x + (r0 + min(row, nr - 1)) * (int64_t)k + 8 * c;
    so[i] = bl_off(ROWS, row, c);
    pc[i] = 8 * c;
  }
  u32x4 xr[XPT];
  auto load_x = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) xr[i] = k0 + pc[i] < k ? *(const u32x4*)(xp[i] + k0) : u32x4{0u, 0u, 0u, 0u};
  };
  auto store_x = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) *(u32x4*)(&xs[buf][so[i]]) = xr[i];
  };
  float4_t acc[BL_RG][XG];
#pragma unroll
  for (int j = 0; j < BL_RG; ++j)
#pragma unroll
    for (int i = 0; i < XG; ++i) acc[j][i] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int chunks = (k + BL_KC - 1) / BL_KC;
  load_x(0);
  store_x(0);
  __syncthreads();
  for (int ch = 0; ch < chunks; ++ch) {
    const int k0 = ch * BL_KC, buf = ch & 1;
    if (ch + 1 < chunks) load_x(k0 + BL_KC);  // uniform; stored after this chunk's products
    const int steps = min(BL_KC, k - k0) / 32;
    // the chunk's weights are decoded before its products, so all of their
    // loads are in flight together (a step past K re-reads the chunk's first)
    bf16x8_t bh[BL_KC / 32][BL_RG], bl[BL_KC / 32][BL_RG];
#pragma unroll
    for (int st = 0; st < BL_KC / 32; ++st) {
#pragma unroll
      for (int j = 0; j < BL_RG; ++j) {
        float v[8];
        decode8<C>(wr[j], k0 + 32 * (st < steps ? st : 0) + 8 * cu, v);
        split8(v, bh[st][j], bl[st][j]);
      }
    }
#pragma unroll
    for (int st = 0; st < BL_KC / 32; ++st) {
      if (st < steps) {  // uniform
#pragma unroll
        for (int i = 0; i < XG; ++i) {
          if (i < xg) {  // uniform
            const bf16x8_t a = *(const bf16x8_t*)(&xs[buf][bl_off(ROWS, 16 * i + r, 4 * st + cu)]);
#pragma unroll
            for (int j = 0; j < BL_RG; ++j) {
              acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh[st][j], acc[j][i], 0, 0, 0);
              acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl[st][j], acc[j][i], 0, 0, 0);
            }
          }
        }
      }
    }
    if (ch + 1 < chunks) store_x(buf ^ 1);  // that buffer was last read before the previous barrier
    __syncthreads();
  }
  // lane l holds rows 16 i + 4 (l >> 4) + q of weight row n0 + 32 wave + 16 j + (l & 15)
#pragma unroll
  for (int j = 0; j < BL_RG; ++j) {
    const int wrow = n0 + wave * 16 * BL_RG + 16 * j + r;
    if (wrow >= n) continue;
#pragma unroll
    for (int i = 0; i < XG; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 16 * i + 4 * cu + q;
        if (row < nr) bf_store<OUT>(y, (r0 + row) * (int64_t)n + wrow, acc[j][i][q]);
      }
    }
  }
}

template <int C, int XG, int OUT>
__global__ __launch_bounds__(BF_THREADS, 2) void bl_mm_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                              int64_t row_bytes, const __bf16* __restrict__ x, int m,
                                                              int nbx, void* __restrict__ y) {
  const int64_t tile = blockIdx.x / nbx;
  const int64_t r0 = tile * 16 * XG;
  const int nr = (int)min((int64_t)16 * XG, (int64_t)m - r0);
  bl_tile<C, XG, OUT>(w, n, k, row_bytes, x, r0, nr, (int)(blockIdx.x % nbx) * BL_BN, y);
}

template <int C, int OUT>
__global__ __launch_bounds__(BF_THREADS, 2) void bl_seg_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                               int64_t row_bytes, int64_t expert_stride, int n_experts,
                                                               const __bf16* __restrict__ x, int m_total,
                                                               const uint32_t* __restrict__ map,
                                                               const uint32_t* __restrict__ counts, int nbx,
                                                               void* __restrict__ y) {
  const uint32_t t = blockIdx.x / nbx;
  if (t >= counts[0]) return;
  const uint32_t* mt = map + 3 * (size_t)t;
  const uint32_t e = mt[0], rs = mt[1], nr = mt[2];
  if (e >= (uint32_t)n_experts || nr == 0 || nr > 64 || rs >= (uint32_t)m_total || nr > (uint32_t)m_total - rs)
    return;
  bl_tile<C, 4, OUT>(w + (int64_t)e * expert_stride, n, k, row_bytes, x, rs, (int)nr, (int)(blockIdx.x % nbx) * BL_BN,
                     y);
}

template <int C, int XG, int OUT>
hipError_t launch_bl(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const __bf16* x, int64_t m, void* y,
                     hipStream_t s) {
  const int64_t nbx = (n + BL_BN - 1) / BL_BN, tiles = (m + 16 * XG - 1) / (16 * XG);
  if (nbx * tiles >= (1ll << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bl_mm_kernel<C, XG, OUT>), dim3((unsigned)(nbx * tiles)), dim3(BF_THREADS), 0, s, w, (int)n,
                     (int)k, rb, x, (int)m, (int)nbx, y);
  return hipGetLastError();
}

template <int C, int OUT>
hipError_t launch_mm_o(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const __bf16* x, int64_t m, void* y,
                       hipStream_t s) {
  if (m <= 16) {  // GEMV: K split over the waves
    hipLaunchKernelGGL((bf_mv_kernel<C, OUT>), dim3((unsigned)((n + 15) / 16)), dim3(64 * BV_WAVES), 0, s, w, (int)n,
                       (int)k, rb, x, (int)m, y);
    return hipGetLastError();
  }
  if (m <= 64) return launch_bl<C, 4, OUT>(w, n, k, rb, x, m, y, s);
  return launch_bl<C, 8, OUT>(w, n, k, rb, x, m, y, s);
}

template <int C>
hipError_t launch_mm_codec(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const __bf16* x, int64_t m, void* y,
                           int out, hipStream_t s) {
  switch (out) {
    case 0: return launch_mm_o<C, 0>(w, n, k, rb, x, m, y, s);
    case 1: return launch_mm_o<C, 1>(w, n, k, rb, x, m, y, s);
    case 2: return launch_mm_o<C, 2>(w, n, k, rb, x, m, y, s);
  }
  return hipErrorInvalidValue;
}

template <int C, int OUT>
hipError_t launch_seg_o(const uint8_t* w, int64_t ne, int64_t n, int64_t k, int64_t rb, const __bf16* x, int64_t rows,
                        const uint32_t* map, const uint32_t* counts, int64_t cap, void* y, hipStream_t s) {
  const int64_t nbx = (n + BL_BN - 1) / BL_BN;
  if (nbx * cap >= (1ll << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bl_seg_kernel<C, OUT>), dim3((unsigned)(nbx * cap)), dim3(BF_THREADS), 0, s, w, (int)n, (int)k,
                     rb, n * rb, (int)ne, x, (int)rows, map, counts, (int)nbx, y);
  return hipGetLastError();
}

template <int C>
hipError_t launch_seg_codec(const uint8_t* w, int64_t ne, int64_t n, int64_t k, int64_t rb, const __bf16* x,
                            int64_t rows, const uint32_t* map, const uint32_t* counts, int64_t cap, void* y, int out,
                            hipStream_t s) {
  switch (out) {
    case 0: return launch_seg_o<C, 0>(w, ne, n, k, rb, x, rows, map, counts, cap, y, s);
    case 1: return launch_seg_o<C, 1>(w, ne, n, k, rb, x, rows, map, counts, cap, y, s);
    case 2: return launch_seg_o<C, 2>(w, ne, n, k, rb, x, rows, map, counts, cap, y, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// out: 0 float32, 1 float16, 2 bfloat16
hipError_t launch_mm_bf16(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t rb, const void* x, int64_t m,
                          void* y, int out, hipStream_t s) {
  const __bf16* xb = (const __bf16*)x;
  switch (codec) {
    case Q4_0: return launch_mm_codec<Q4_0>(w, n, k, rb, xb, m, y, out, s);
    case Q8_0: return launch_mm_codec<Q8_0>(w, n, k, rb, xb, m, y, out, s);
    case Q4_1: return launch_mm_codec<Q4_1>(w, n, k, rb, xb, m, y, out, s);
    case Q5_0: return launch_mm_codec<Q5_0>(w, n, k, rb, xb, m, y, out, s);
    case Q5_1: return launch_mm_codec<Q5_1>(w, n, k, rb, xb, m, y, out, s);
    case Q2_K: return launch_mm_codec<Q2_K>(w, n, k, rb, xb, m, y, out, s);
    case Q3_K: return launch_mm_codec<Q3_K>(w, n, k, rb, xb, m, y, out, s);
    case Q4_K: return launch_mm_codec<Q4_K>(w, n, k, rb, xb, m, y, out, s);
    case Q5_K: return launch_mm_codec<Q5_K>(w, n, k, rb, xb, m, y, out, s);
    case Q6_K: return launch_mm_codec<Q6_K>(w, n, k, rb, xb, m, y, out, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_seg_bf16(int codec, const uint8_t* w, int64_t ne, int64_t n, int64_t k, int64_t rb, const void* x,
                           int64_t rows, const uint32_t* map, const uint32_t* counts, int64_t cap, void* y, int out,
                           hipStream_t s) {
  const __bf16* xb = (const __bf16*)x;
  switch (codec) {
    case Q4_0: return launch_seg_codec<Q4_0>(w, ne, n, k, rb, xb, rows, map, counts, cap, y, out, s);
    case Q8_0: return launch_seg_codec<Q8_0>(w, ne, n, k, rb, xb, rows, map, counts, cap, y, out, s);
    case Q4_1: return launch_seg_codec<Q4_1>(w, ne, n, k, rb, xb, rows, map, counts, cap, y, out, s);
    case Q5_0: return launch_seg_codec<Q5_0>(w, ne, n, k, rb, xb, rows, map, counts, cap, y, out, s);
    case Q5_1: return launch_seg_codec<Q5_1>(w, ne, n, k, rb, xb, rows, map, counts, cap, y, out, s);
    case Q2_K: return launch_seg_codec<Q2_K>(w, ne, n, k, rb, xb, rows, map, counts, cap, y, out, s);
    case Q3_K: return launch_seg_codec<Q3_K>(w, ne, n, k, rb, xb, rows, map, counts, cap, y, out, s);
    case Q4_K: return launch_seg_codec<Q4_K>(w, ne, n, k, rb, xb, rows, map, counts, cap, y, out, s);
    case Q5_K: return launch_seg_codec<Q5_K>(w, ne, n, k, rb, xb, rows, map, counts, cap, y, out, s);
    case Q6_K: return launch_seg_codec<Q6_K>(w, ne, n, k, rb, xb, rows, map, counts, cap, y, out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kq
