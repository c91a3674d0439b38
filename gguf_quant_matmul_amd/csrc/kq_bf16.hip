// bfloat16 activations: kq_qmv_bf16, kq_qmm_bf16, kq_gather_qmm_seg_bf16.
//
// mlx-kquant bindings.cpp page: quantized_matmul and gather_qmm_seg return
// x's dtype (a float32 x promoted to bfloat16), so a bfloat16 activation is a
// first-class input of the quantized matmuls; the product is
// y = x @ dequant(w)^T as for float16 activations.
//
// Design.  One codec-generic matrix-core kernel serves the three shapes (a
// GEMV of up to 16 activation rows, the prefill GEMM, and the expert-segment
// GEMM over a tile map):
//  * a workgroup of four waves takes 64 weight rows (16 per wave; for a GEMV
//    of at most 16 rows the four waves share 16 weight rows and split K) and
//    one "row tile" of up to 16 * XG activation rows (XG 16-row groups);
//  * per 32-value K step each lane decodes 8 consecutive weights of its row
//    (row l & 15 of the wave's group, K values 8 (l >> 4) ..) to their exact
//    float32 values (decode8, one rounding where the codec formula has one)
//    and splits each into a bfloat16 high part and a bfloat16 remainder, so
//    the weight carries 16 significant bits (relative error below 2^-16);
//  * v_mfma_f32_16x16x32_bf16 multiplies the exact bfloat16 activations
//    (read from global memory straight into the A operand: lane l holds row
//    l & 15 of a group, K values 8 (l >> 4) ..) by both weight parts, with
//    float32 accumulation;
//  * the store rounds once to float32, float16 or bfloat16 (nearest even).
// The float16 paths' exact integer-code tricks do not carry over: a
// bfloat16 holds integers exactly only below 257, and sc * q reaches 945.
#include "kq_decode.h"

namespace kq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int BF_THREADS = 256;
constexpr int BF_BN = 64;  // weight rows per workgroup (16 per wave)

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

// One row tile (rows r0 .. r0 + nr of x and y, nr <= 16 XG) against 16 * 4 /
// KS weight rows from n0: with KS = 1 each wave takes its own 16 rows over
// all of K; with KS = 4 the four waves share 16 rows and each takes a quarter
// of the 32-value K steps, the parts added in LDS at the end (four times the
// workgroups for a GEMV).  Two K steps per iteration keep both steps' loads
// in flight before either is decoded.
template <int C, int XG, int OUT, int KS>
__device__ __forceinline__ void bf_tile(const uint8_t* __restrict__ w, int n, int k, int64_t row_bytes,
                                        const __bf16* __restrict__ x, int64_t r0, int nr, int n0,
                                        void* __restrict__ y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, cu = lane >> 4;
  const int wrow = n0 + (KS == 1 ? 16 * wave : 0) + r;
  const uint8_t* wr = w + (int64_t)(wrow < n ? wrow : n - 1) * row_bytes;  // rows past N: a valid row, not stored
  const int xg = (nr + 15) >> 4;  // live 16-row groups
  const __bf16* xr[XG];
#pragma unroll
  for (int i = 0; i < XG; ++i) {
    const int row = min(16 * i + r, nr - 1);  // rows past the tile repeat its last row (outputs dropped)
    xr[i] = x + (r0 + row) * (int64_t)k + 8 * cu;
  }
  float4_t acc[XG];
#pragma unroll
  for (int i = 0; i < XG; ++i) acc[i] = float4_t{0.f, 0.f, 0.f, 0.f};
  const int steps = k / 32;
  const int s0 = KS == 1 ? 0 : (steps * wave) / KS, s1 = KS == 1 ? steps : (steps * (wave + 1)) / KS;
  auto mfmas = [&](int k0, const float* v) __attribute__((always_inline)) {
    bf16x8_t bh, bl;
    split8(v, bh, bl);
#pragma unroll
    for (int i = 0; i < XG; ++i) {
      if (i < xg) {  // uniform
        const bf16x8_t a = *(const bf16x8_t*)(xr[i] + k0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc[i], 0, 0, 0);
      }
    }
  };
  int st = s0;
  for (; st + 1 < s1; st += 2) {
    float v0[8], v1[8];
    decode8<C>(wr, 32 * st + 8 * cu, v0);
    decode8<C>(wr, 32 * st + 32 + 8 * cu, v1);
    mfmas(32 * st, v0);
    mfmas(32 * st + 32, v1);
  }
  if (st < s1) {
    float v0[8];
    decode8<C>(wr, 32 * st + 8 * cu, v0);
    mfmas(32 * st, v0);
  }
  if constexpr (KS > 1) {
    // waves 1..KS-1 hand their parts to wave 0 through LDS
    __shared__ float4_t part[KS - 1][XG][64];
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < XG; ++i) part[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int p = 0; p < KS - 1; ++p)
#pragma unroll
      for (int i = 0; i < XG; ++i) acc[i] += part[p][i][lane];
  }
  // lane l holds rows 16 i + 4 (l >> 4) + q of weight row wrow
  if (wrow >= n) return;
#pragma unroll
  for (int i = 0; i < XG; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 16 * i + 4 * cu + q;
      if (row < nr) bf_store<OUT>(y, (r0 + row) * (int64_t)n + wrow, acc[i][q]);
    }
  }
}

// qmv / qmm: workgroup b takes column block b % nbx of row tile b / nbx
// (16 XG rows each).
template <int C, int XG, int OUT, int KS>
__global__ __launch_bounds__(BF_THREADS) void bf_mm_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                           int64_t row_bytes, const __bf16* __restrict__ x, int m,
                                                           int nbx, void* __restrict__ y) {
  const int64_t tile = blockIdx.x / nbx;
  const int64_t r0 = tile * 16 * XG;
  const int nr = (int)min((int64_t)16 * XG, (int64_t)m - r0);
  bf_tile<C, XG, OUT, KS>(w, n, k, row_bytes, x, r0, nr, (int)(blockIdx.x % nbx) * (BF_BN / KS), y);
}

// gather_qmm_seg: workgroup b takes column block b % nbx of tile-map slot
// b / nbx; slots past the count or out of range are skipped, so uncovered
// rows stay unwritten.
template <int C, int OUT>
__global__ __launch_bounds__(BF_THREADS) void bf_seg_kernel(const uint8_t* __restrict__ w, int n, int k,
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
  bf_tile<C, 4, OUT, 1>(w + (int64_t)e * expert_stride, n, k, row_bytes, x, rs, (int)nr, (int)(blockIdx.x % nbx) * BF_BN,
                     y);
}

template <int C, int XG, int OUT, int KS = 1>
hipError_t launch_mm_c(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const __bf16* x, int64_t m, void* y,
                       hipStream_t s) {
  constexpr int BN = BF_BN / KS;
  const int64_t nbx = (n + BN - 1) / BN, tiles = (m + 16 * XG - 1) / (16 * XG);
  if (nbx * tiles >= (1ll << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bf_mm_kernel<C, XG, OUT, KS>), dim3((unsigned)(nbx * tiles)), dim3(BF_THREADS), 0, s, w, (int)n,
                     (int)k, rb, x, (int)m, (int)nbx, y);
  return hipGetLastError();
}

template <int C, int OUT>
hipError_t launch_mm_o(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const __bf16* x, int64_t m, void* y,
                       hipStream_t s) {
  if (m <= 16) return launch_mm_c<C, 1, OUT, 4>(w, n, k, rb, x, m, y, s);  // GEMV: K split over the waves
  if (m <= 64) return launch_mm_c<C, 4, OUT>(w, n, k, rb, x, m, y, s);
  return launch_mm_c<C, 8, OUT>(w, n, k, rb, x, m, y, s);
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
  const int64_t nbx = (n + BF_BN - 1) / BF_BN;
  if (nbx * cap >= (1ll << 31)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bf_seg_kernel<C, OUT>), dim3((unsigned)(nbx * cap)), dim3(BF_THREADS), 0, s, w, (int)n, (int)k,
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
