// kq_qmv_wide_impl.h -- the matrix-core GEMV for small prefill batches (up to
// 64 activation rows), shared by kq_qmv_wide.hip (the plain product of
// kq_quantized_matmul), kq_qmv_wide_epi.hip (its residual epilogue),
// kq_qmv_wide_glu.hip and kq_qmv_wide_glum.hip (the two passes of its GLU
// product).
//
// mlx-kquant bindings.cpp page, quantized_matmul docstring; the README's
// remark that a matmul over few rows amortizes one weight read over all of
// them.  It is the 16-row matrix-core GEMV of kq_qmv_impl.h with several A
// operands per decoded B operand.
#pragma once

#include "kq_qmv_impl.h"

namespace kq {
namespace {

// K values per LDS chunk: 64 KiB of activations for 16 T rows, at most 1024
// (a wave's two register rings then hold at most 2 x 2 unit groups), and at
// least one unit group (256 values) for each of the KS waves that share a
// row group (64 rows of 1024 values: 148 KiB of LDS, one workgroup per CU).
__host__ __device__ constexpr int wide_kchunk(int t, int ks) {
  const int fit = mma_kchunk(16 * t) < 1024 ? mma_kchunk(16 * t) : 1024;
  return fit > 256 * ks ? fit : 256 * ks;
}

// The matrix-core GEMV for M <= 16 T activation rows: each decoded B operand
// meets T 16-row A operands (activation rows 16 t + (l & 15); rows past M
// repeat row M - 1 and their outputs are dropped), so a weight is still
// decoded once for every row.  The activation chunk is at most 1024 values
// (512 for four operands split two ways), and a wave takes only G unit
// groups of each; the next chunk's groups are loaded while the current one
// is staged and consumed.  M is a run-time argument: the kernel is sized for
// 16 T rows.
// KS waves of the workgroup share a 16-row group, each a part of every chunk
// (2, or 4 when the matrix has few rows, so that the grid still covers the
// CUs).  EP: the store mode (kq_internal.h: plain, epi_apply, or one pass of
// the GLU product; the gate pass's activation is act, GLU_SILU or
// GLU_GELU_TANH).
template <int C, int T, int KS, bool F16, int EP>
__global__ __launch_bounds__(MMA_THREADS) void qmv_mma_wide_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                                   int64_t row_bytes, const half_t* __restrict__ x,
                                                                   int m, Epi epi, int act, void* __restrict__ y) {
  typedef typename UnitOf<C>::T Unit;
  static_assert(T >= 1 && T <= 4, "A operands per B operand");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int MT = 16 * T, KC = wide_kchunk(T, KS);
  static_assert(KS == 2 || KS == 4, "waves per row group");
  constexpr int G = KC / 256 / KS;  // unit groups (4 units each) of a wave per full chunk
  static_assert(G >= 1 && KC % (256 * KS) == 0, "chunk split");
  const int kc_alloc = k < KC ? k : KC;
  half_t* xs = (half_t*)smem;
  const int xstride = mma_xstride(kc_alloc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rgroup = blockIdx.x * (4 / KS) + wave / KS, kpart = wave % KS;
  const int r = lane & 15, cu = lane >> 4;
  const int row = rgroup * 16 + r;
  const uint8_t* wrow = w + (int64_t)min(row, n - 1) * row_bytes;
  int xm[T];
#pragma unroll
  for (int t = 0; t < T; ++t) xm[t] = min(16 * t + r, m - 1);

  float4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  // This wave's unit groups of the chunk at c0: [g0, g1), loaded into ring
  // slots 0..G-1 (unit 4 g + (l >> 4) of group g; past the chunk, clamped).
  auto load_chunk = [&](int c0, Unit (&ring)[G]) __attribute__((always_inline)) {
    const int kc = (k - c0) < KC ? (k - c0) : KC;
    const int ub = c0 / 64, ue = (c0 + kc) / 64;
    const int ngroups = (ue - ub + 3) / 4, gper = (ngroups + KS - 1) / KS;  // gper <= G
    const int g0 = min(kpart * gper, ngroups);
#pragma unroll
    for (int j = 0; j < G; ++j) ring[j].load(wrow, min(ub + 4 * (g0 + j) + cu, ue - 1));
  };
  // One chunk: its activations are loaded and the next chunk's units go out
  // (into the other ring) before the staging, so their latency overlaps this
  // chunk's staging and matrix work; then this chunk's ring is consumed.
  auto chunk = [&](int c0, Unit (&cur)[G], Unit (&nxt)[G]) __attribute__((always_inline)) {
    const int kc = (k - c0) < KC ? (k - c0) : KC;
    const int ub = c0 / 64, ue = (c0 + kc) / 64;
    const int ngroups = (ue - ub + 3) / 4, gper = (ngroups + KS - 1) / KS;
    const int g0 = min(kpart * gper, ngroups), g1 = min(g0 + gper, ngroups);
    const int last = ue - 1;
    constexpr int XPT = (MT * KC / 8 + MMA_THREADS - 1) / MMA_THREADS;
    const int xpieces = m * (kc / 8);
    u32x4 xr[XPT];
    {
      PieceWalk pw(tid, kc / 8, MMA_THREADS);  // pieces past the block re-read its last one
#pragma unroll
      for (int i = 0; i < XPT; ++i, pw.next()) {
        const bool in = tid + i * MMA_THREADS < xpieces;
        const int mr = in ? pw.m : m - 1, v = (in ? pw.r : kc / 8 - 1) * 8;
        xr[i] = *(const u32x4*)(x + (int64_t)mr * k + c0 + v);
      }
    }
    if (c0 + KC < k) load_chunk(c0 + KC, nxt);  // uniform across the block
    if (c0) __syncthreads();  // previous chunk done with LDS
    {
      PieceWalk pw(tid, kc / 8, MMA_THREADS);
#pragma unroll
      for (int i = 0; i < XPT; ++i, pw.next()) {
        if (tid + i * MMA_THREADS < xpieces) *(u32x4*)(xs + pw.m * xstride + xpad(pw.r * 8)) = xr[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int u = ub + 4 * (g0 + j) + cu;
      const bool valid = g0 + j < g1 && u < ue;  // else this lane adds zeros
      const int uc = valid ? u : last;           // (and reads in-range x)
      const MmaSlices<C> sl(cur[j], uc, valid);
      const int xoff = xpad(MmaSlices<C>::koff(uc) - c0);
      auto step = [&](auto sc) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        uint32_t f[4];
        sl.template get<S>(f);
        const half8_t b = __builtin_bit_cast(half8_t, u32x4{f[0], f[1], f[2], f[3]});
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const half8_t a = *(const half8_t*)(xs + xm[t] * xstride + xoff + MmaSlices<C>::template xstep<S>());
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t], 0, 0, 0);
        }
      };
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      step(std::integral_constant<int, 2>{});
      step(std::integral_constant<int, 3>{});
      step(std::integral_constant<int, 4>{});
      step(std::integral_constant<int, 5>{});
      step(std::integral_constant<int, 6>{});
      step(std::integral_constant<int, 7>{});
    }
  };
  // Two rings in turn, so no register is copied while its load is in flight.
  Unit ring_a[G], ring_b[G];
  load_chunk(0, ring_a);
  for (int c0 = 0; c0 < k; c0 += 2 * KC) {
    chunk(c0, ring_a, ring_b);
    if (c0 + KC < k) chunk(c0 + KC, ring_b, ring_a);
  }

  // Combine the K parts: for tile t, lane l holds activation rows
  // 16 t + 4 (l >> 4) + i of weight row 16 rgroup + (l & 15).
  __syncthreads();
  float4_t* part = (float4_t*)smem;
  const int pbase = (wave / KS) * (KS - 1) * 64 * T;
  if (kpart) {
#pragma unroll
    for (int t = 0; t < T; ++t) part[pbase + ((kpart - 1) * T + t) * 64 + lane] = acc[t];
  }
  __syncthreads();
  if (kpart == 0) {
    const int col = rgroup * 16 + (lane & 15);
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int p = 0; p + 1 < KS; ++p) acc[t] += part[pbase + (p * T + t) * 64 + lane];
      if (col < n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mr = 16 * t + 4 * (lane >> 4) + i;
          if (mr < m) {
            if constexpr (EP == EP_GLU_ACT) {
              if (act == GLU_SILU)
                store_out<F16, EP, GLU_SILU>(y, mr, col, n, epi, acc[t][i]);
              else
                store_out<F16, EP, GLU_GELU_TANH>(y, mr, col, n, epi, acc[t][i]);
            } else {
              store_out<F16, EP, 0>(y, mr, col, n, epi, acc[t][i]);
            }
          }
        }
      }
    }
  }
}

// m <= 16 T activation rows; K a whole number of 64-value units.
template <int C, int T, int KS, int EP>
hipError_t launch_mma_wide(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int m, const Epi& epi,
                           int act, void* y, int f16, hipStream_t s) {
  const int kc = (int)(k < wide_kchunk(T, KS) ? k : wide_kchunk(T, KS));
  size_t lds = (size_t)(16 * T) * mma_xstride(kc) * 2;
  const size_t part_bytes = (size_t)(4 / KS) * (KS - 1) * 64 * T * sizeof(float4_t);
  if (lds < part_bytes) lds = part_bytes;
  constexpr int rows_per_block = 16 * (4 / KS);
  const dim3 grid((unsigned)((n + rows_per_block - 1) / rows_per_block));
  if (f16)
    hipLaunchKernelGGL((qmv_mma_wide_kernel<C, T, KS, true, EP>), grid, dim3(MMA_THREADS), lds, s, w, (int)n, (int)k,
                       rb, x, m, epi, act, y);
  else
    hipLaunchKernelGGL((qmv_mma_wide_kernel<C, T, KS, false, EP>), grid, dim3(MMA_THREADS), lds, s, w, (int)n,
                       (int)k, rb, x, m, epi, act, y);
  return hipGetLastError();
}

// Four waves per row group when two would leave CUs without a workgroup (a
// 256-CU part); with enough rows, two (four measured 1.4 to 2.4 times slower
// at N = 14336).
template <int C, int T, int EP>
hipError_t launch_mma_wide_ks(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int m,
                              const Epi& epi, int act, void* y, int f16, hipStream_t s) {
  if (wide_narrow(n)) return launch_mma_wide<C, T, 4, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
  return launch_mma_wide<C, T, 2, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
}

// One A operand up to 16 rows, two up to 32, four up to 64.  An epilogue or
// GLU pass over 3..8 rows takes the 16-row kernel of kq_qmv_impl.h instead:
// its single 4096-value chunk at K = 4096 beats the one-operand wide kernel
// there (as kq_qmv's own 3..8 rows do).
template <int C, int EP>
hipError_t launch_wide_c(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int m, const Epi& epi,
                         int act, void* y, int f16, hipStream_t s) {
  if constexpr (EP != EP_PLAIN) {
    switch (m) {
      case 3: return launch_mma_ep<C, 3, EP>(w, n, k, rb, x, epi, act, y, f16, s);
      case 4: return launch_mma_ep<C, 4, EP>(w, n, k, rb, x, epi, act, y, f16, s);
      case 5: return launch_mma_ep<C, 5, EP>(w, n, k, rb, x, epi, act, y, f16, s);
      case 6: return launch_mma_ep<C, 6, EP>(w, n, k, rb, x, epi, act, y, f16, s);
      case 7: return launch_mma_ep<C, 7, EP>(w, n, k, rb, x, epi, act, y, f16, s);
      case 8: return launch_mma_ep<C, 8, EP>(w, n, k, rb, x, epi, act, y, f16, s);
    }
  }
  if (m <= 16) return launch_mma_wide_ks<C, 1, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
  if (m <= 32) return launch_mma_wide_ks<C, 2, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
  return launch_mma_wide_ks<C, 4, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
}

template <int EP>
hipError_t launch_wide(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int m,
                       const Epi& epi, int act, void* y, int f16, hipStream_t s) {
  switch (codec) {
    case Q4_0: return launch_wide_c<Q4_0, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
    case Q8_0: return launch_wide_c<Q8_0, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
    case Q4_1: return launch_wide_c<Q4_1, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
    case Q5_0: return launch_wide_c<Q5_0, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
    case Q5_1: return launch_wide_c<Q5_1, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
    case Q2_K: return launch_wide_c<Q2_K, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
    case Q3_K: return launch_wide_c<Q3_K, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
    case Q4_K: return launch_wide_c<Q4_K, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
    case Q5_K: return launch_wide_c<Q5_K, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
    case Q6_K: return launch_wide_c<Q6_K, EP>(w, n, k, rb, x, m, epi, act, y, f16, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace kq
