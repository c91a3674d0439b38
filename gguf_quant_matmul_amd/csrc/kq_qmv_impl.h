// kq_qmv_impl.h -- decode-shaped quantized GEMV kernels and launchers, shared
// by kq_qmv.hip, kq_qmv_fused.hip and kq_qmv_gather.hip:
// y[m][n] = sum_k x[m][k] * W[n][k], 1 <= M <= 16 activation rows, float32
// accumulation.
//
// mlx-kquant bindings.cpp page, quantized_matmul docstring (transpose=True
// weights [N, K]); the README's remark that small-row-count matmuls amortize
// one weight read over all rows is the reason every decoded weight here is
// used for all M rows before it leaves registers.
//
// Design (HBM-bound: one pass over the wire bytes).
//  * A "unit" is 64 weights of one row: q4_K one sub-block pair (its 16-byte
//    header + 32 bytes of qs), q6_K one (h, half) slice of a superblock (16 B
//    of each ql half, 16 B of qh, 4 scales), q8_0 / q4_0 two blocks.
//  * A row is split over 16 lanes (a wave owns 4 rows) or, for one
//    activation row and a matrix with few rows, over a whole wave; the lanes
//    walk the row's units with a stride of the lane count.  Every load is a 16-byte (or 4-byte
//    aligned multi-dword) load of raw wire bytes; all loads of a lane's units
//    are issued before any is used.
//  * Codes become float16 pairs by byte permutes onto a 0x64 exponent byte
//    (value 1024 + code); v_dot2 with float16 activations accumulates in
//    float32, and the 1024 offset (plus each codec's zero point) is removed
//    with per-16-value activation sums: sum((1024+q) x) - 1024 sum(x).
//  * x is staged once per workgroup in LDS as float16 (with 16 bytes of
//    padding per 64 values against bank conflicts) together with its 16-value
//    sums.  Long K is processed in chunks that fit LDS.
//  * Partial sums of a row's lanes are reduced with DPP row rotations (and
//    lane swaps across 16-lane rows).
#pragma once

#include <algorithm>
#include <type_traits>

#include "kq_units.h"

namespace kq {
namespace {

constexpr int QMV_THREADS = 256;
// A row is split over LPR lanes (16, 32 or 64); a lane takes UNITS_PER_GROUP /
// LPR units per load group, so a group is always 64 units of a row.
constexpr int UNITS_PER_GROUP = 64;
__host__ __device__ constexpr int rows_per_block(int lpr) { return (64 / lpr) * (QMV_THREADS / 64); }

// K values per LDS chunk for M activation rows: at most 8192 activation
// values per chunk, so each thread stages at most four 16-byte pieces of x
// (held in registers while the weight loads go out).
__host__ __device__ constexpr int kchunk_max(int m) {
  return m <= 2 ? 4096 : m <= 4 ? 2048 : 1024;
}

// Sum over the 16 lanes of a DPP row (every lane receives the total).
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));  // row_ror:8
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));  // row_ror:4
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));  // row_ror:2
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));  // row_ror:1
  return v;
}

// Sum over the 64 lanes of a wave, complete in lane 63 only: DPP row sums,
// then row_bcast:15 (row r - 1's last lane into rows 1 and 3) and
// row_bcast:31 (lane 31 into rows 2 and 3), without an LDS round trip.
__device__ __forceinline__ float wave_sum_last(float v) {
  v = row16_sum(v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
  return v;
}

// Sum over the LPR lanes of a row: DPP within 16-lane rows, then swaps
// across them.
template <int LPR>
__device__ __forceinline__ float lanes_sum(float v) {
  v = row16_sum(v);
  if (LPR >= 32) v += __shfl_xor(v, 16);
  if (LPR >= 64) v += __shfl_xor(v, 32);
  return v;
}

// The GEMV of one workgroup: rows [blk * rows_per_block, ...) of w.
// NW = 2: the same rows of a second matrix w2 go through the same pass,
// sharing each staged activation chunk, and activation row m's lane stores
// glu_act<ACT>(row of w, row of w2) instead of both products (with EPI, the
// twice-rounded glu_rounded of quantized_matmul_glu).  EPI with NW = 1: the
// products go through epi_apply before the store.
template <int C, int M, int LPR, bool F16, int NW = 1, int ACT = 0, bool EPI = false>
__device__ __forceinline__ void qmv_rows(const uint8_t* __restrict__ w, int n, int k, int64_t row_bytes,
                                         const half_t* __restrict__ x, void* __restrict__ y, int blk,
                                         const uint8_t* __restrict__ w2 = nullptr, float limit = 0.f,
                                         Epi epi = Epi{nullptr, nullptr, nullptr, 1}) {
  static_assert(NW == 1 || NW == 2, "one or two matrices");
  typedef typename UnitOf<C>::T Unit;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int KC = kchunk_max(M);
  const int kc_alloc = k < KC ? k : KC;
  half_t* xs = (half_t*)smem;
  const int xstride = xpad(kc_alloc);
  float* xsum = (float*)(smem + (size_t)M * xstride * 2);
  const int sstride = kc_alloc / 16;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int LANES_PER_ROW = LPR, ROWS_PER_WAVE = 64 / LPR, UNROLL = UNITS_PER_GROUP / LPR;
  const int rslot = lane / LANES_PER_ROW, uslot = lane % LANES_PER_ROW;
  const int row = (blk * (QMV_THREADS / 64) + wave) * ROWS_PER_WAVE + rslot;
  const bool row_ok = row < n;
  const uint8_t* wrow = w + (int64_t)(row_ok ? row : 0) * row_bytes;
  const uint8_t* wrow2 = NW == 2 ? w2 + (int64_t)(row_ok ? row : 0) * row_bytes : nullptr;

  float acc[M], acc2[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = acc2[m] = 0.f;

  for (int c0 = 0; c0 < k; c0 += KC) {
    const int kc = (k - c0) < KC ? (k - c0) : KC;
    const int ub = c0 / 64, ue = (c0 + kc) / 64;
    // Unit u of this lane in group g is ub + uslot + LANES_PER_ROW * (g * UNROLL + j).
    // Loads are never predicated: an index past the chunk is clamped to its
    // last unit (and its product skipped), so all loads of a group go out
    // back to back with no wait between them.
    const int ngroups = (ue - ub + LANES_PER_ROW * UNROLL - 1) / (LANES_PER_ROW * UNROLL);
    // Activation loads first, then the first group's weight loads: loads
    // retire in order, so the LDS staging below waits for x only, and the
    // weights keep streaming in while x is staged and summed.
    constexpr int XPT = (M * KC / 8 + QMV_THREADS - 1) / QMV_THREADS;
    const int xpieces = M * (kc / 8);
    u32x4 xr[XPT];
    {
      PieceWalk pw(tid, kc / 8, QMV_THREADS);  // pieces past the block re-read its last one
#pragma unroll
      for (int i = 0; i < XPT; ++i, pw.next()) {
        const bool in = tid + i * QMV_THREADS < xpieces;
        const int m = in ? pw.m : M - 1, v = (in ? pw.r : kc / 8 - 1) * 8;
        xr[i] = *(const u32x4*)(x + (int64_t)m * k + c0 + v);
      }
    }
    Unit cur[UNROLL], cur2[NW == 2 ? UNROLL : 1];
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      const int u = ub + uslot + LANES_PER_ROW * j;
      cur[j].load(wrow, u < ue ? u : ue - 1);
      if constexpr (NW == 2) cur2[j].load(wrow2, u < ue ? u : ue - 1);
    }
    if (c0) __syncthreads();  // previous chunk done with LDS
    // Stage x and its 16-value sums in one pass: pieces 2g and 2g + 1 (8
    // values each) sit in adjacent lanes, so each lane sums its own 8 values
    // and adds its neighbour's with a DPP quad permutation [1, 0, 3, 2].
    {
      PieceWalk pw(tid, kc / 8, QMV_THREADS);
#pragma unroll
      for (int i = 0; i < XPT; ++i, pw.next()) {
        const int c = tid + i * QMV_THREADS;
        const uint32_t one2 = 0x3C003C00u;  // (1.0, 1.0)
        float s = 0.f;
        s = dot2(xr[i].x, one2, s); s = dot2(xr[i].y, one2, s); s = dot2(xr[i].z, one2, s); s = dot2(xr[i].w, one2, s);
        s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, false));
        if (c < xpieces) {
          const int m = pw.m, v = xperm<C>(pw.r * 8);
          *(u32x4*)(xs + m * xstride + xpad(v)) = xr[i];
          if ((c & 1) == 0) xsum[m * sstride + (v >> 4)] = s;
        }
      }
    }
    __syncthreads();
    const Xv xv{xs, xsum, xstride, sstride, c0};
    for (int g = 0; g < ngroups; ++g) {
      const int u0 = ub + uslot + LANES_PER_ROW * UNROLL * g;
      Unit nxt[UNROLL], nxt2[NW == 2 ? UNROLL : 1];
      if (g + 1 < ngroups) {  // uniform across the block
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) {
          const int u = u0 + LANES_PER_ROW * (UNROLL + j);
          nxt[j].load(wrow, u < ue ? u : ue - 1);
          if constexpr (NW == 2) nxt2[j].load(wrow2, u < ue ? u : ue - 1);
        }
      }
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        const int u = u0 + LANES_PER_ROW * j;
        if (row_ok && u < ue) {
          cur[j].template dot<M>(u, xv, acc);
          if constexpr (NW == 2) cur2[j].template dot<M>(u, xv, acc2);
        }
      }
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        cur[j] = nxt[j];
        if constexpr (NW == 2) cur2[j] = nxt2[j];
      }
    }
  }

  if constexpr (NW == 2) {
    float v = 0.f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float g = lanes_sum<LPR>(acc[m]), u = lanes_sum<LPR>(acc2[m]);
      if (uslot == m) {
        if constexpr (EPI)
          v = glu_rounded<ACT, F16>(g, u);
        else
          v = glu_act<ACT>(g, u, limit);
      }
    }
    if (row_ok && uslot < M) {
      if (F16)
        ((half_t*)y)[(int64_t)uslot * n + row] = (half_t)v;
      else
        ((float*)y)[(int64_t)uslot * n + row] = v;
    }
    return;
  }
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = lanes_sum<LPR>(acc[m]);
  if (row_ok && uslot < M) {
    float v = acc[0];
#pragma unroll
    for (int m = 1; m < M; ++m)
      if (uslot == m) v = acc[m];
    if constexpr (EPI) v = epi_apply<F16>(epi, uslot, row, n, v);
    if (F16)
      ((half_t*)y)[(int64_t)uslot * n + row] = (half_t)v;
    else
      ((float*)y)[(int64_t)uslot * n + row] = v;
  }
}

template <int C, int M, int LPR, bool F16>
__global__ __launch_bounds__(QMV_THREADS) void qmv_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                          int64_t row_bytes, const half_t* __restrict__ x,
                                                          void* __restrict__ y) {
  qmv_rows<C, M, LPR, F16>(w, n, k, row_bytes, x, y, blockIdx.x);
}

// Streaming GEMV for one or two activation rows with K <= 4096 (a row's
// units fit one load group) over many weight rows: each workgroup stages x
// once and walks the row blocks b, b + G, b + 2G, ... (G workgroups),
// loading block b + G's units into registers while block b's are consumed,
// so the activation staging and its barrier are paid once per workgroup
// rather than once per block.
template <int C, int M, int LPR, bool F16, int PD = 1>
__global__ __launch_bounds__(QMV_THREADS) void qmv_stream_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                                 int64_t row_bytes, const half_t* __restrict__ x,
                                                                 void* __restrict__ y, int nblocks) {
  typedef typename UnitOf<C>::T Unit;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  half_t* xs = (half_t*)smem;
  const int xstride = xpad(k);
  float* xsum = (float*)(smem + (size_t)M * xstride * 2);
  const int sstride = k / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int ROWS_PER_WAVE = 64 / LPR, UNROLL = UNITS_PER_GROUP / LPR;
  const int rslot = lane / LPR, uslot = lane % LPR;
  const int ue = k / 64;
  auto row_of = [&](int b) { return (b * (QMV_THREADS / 64) + wave) * ROWS_PER_WAVE + rslot; };
  auto load_block = [&](Unit* dst, int b) __attribute__((always_inline)) {
    const int row = row_of(b);
    const uint8_t* wrow = w + (int64_t)(row < n ? row : n - 1) * row_bytes;
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      const int u = uslot + LPR * j;
      dst[j].load(wrow, u < ue ? u : ue - 1);
    }
  };

  // x first (its loads retire before the weights'), then the first block's units
  constexpr int XPT = (M * 4096 / 8 + QMV_THREADS - 1) / QMV_THREADS;
  const int xpieces = M * (k / 8);
  u32x4 xr[XPT];
  {
    PieceWalk pw(tid, k / 8, QMV_THREADS);  // pieces past x re-read its last one
#pragma unroll
    for (int i = 0; i < XPT; ++i, pw.next()) {
      const bool in = tid + i * QMV_THREADS < xpieces;
      const int m = in ? pw.m : M - 1, v = (in ? pw.r : k / 8 - 1) * 8;
      xr[i] = *(const u32x4*)(x + (int64_t)m * k + v);
    }
  }
  int b = blockIdx.x;
  Unit ring[PD][UNROLL];
#pragma unroll
  for (int p = 0; p < PD; ++p) load_block(ring[p], min(b + p * (int)gridDim.x, nblocks - 1));
  {
    PieceWalk pw(tid, k / 8, QMV_THREADS);
#pragma unroll
    for (int i = 0; i < XPT; ++i, pw.next()) {
      const int c = tid + i * QMV_THREADS;
      const uint32_t one2 = 0x3C003C00u;  // (1.0, 1.0)
      float s = 0.f;
      s = dot2(xr[i].x, one2, s); s = dot2(xr[i].y, one2, s); s = dot2(xr[i].z, one2, s); s = dot2(xr[i].w, one2, s);
      s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, false));
      if (c < xpieces) {
        const int m = pw.m, v = xperm<C>(pw.r * 8);
        *(u32x4*)(xs + m * xstride + xpad(v)) = xr[i];
        if ((c & 1) == 0) xsum[m * sstride + (v >> 4)] = s;
      }
    }
  }
  __syncthreads();
  const Xv xv{xs, xsum, xstride, sstride, 0};

  for (; b < nblocks; b += gridDim.x) {
    Unit nxt[UNROLL];
    if (b + PD * (int)gridDim.x < nblocks) load_block(nxt, b + PD * gridDim.x);  // uniform
    Unit* cur = ring[0];
    const int row = row_of(b);
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      const int u = uslot + LPR * j;
      if (row < n && u < ue) cur[j].template dot<M>(u, xv, acc);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = lanes_sum<LPR>(acc[m]);
    if (row < n && uslot < M) {
      float v = acc[0];
#pragma unroll
      for (int m = 1; m < M; ++m)
        if (uslot == m) v = acc[m];
      if (F16)
        ((half_t*)y)[(int64_t)uslot * n + row] = (half_t)v;
      else
        ((float*)y)[(int64_t)uslot * n + row] = v;
    }
#pragma unroll
    for (int p = 0; p + 1 < PD; ++p)
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) ring[p][j] = ring[p + 1][j];
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) ring[PD - 1][j] = nxt[j];
  }
}

// One to four activation rows on a matrix of at least 4096 rows whose rows
// are a multiple of 16 bytes: a wave per weight row, as in qmv_stream_kernel
// for one activation row, but the row reaches the lanes through LDS.
// The units' own loads (16-byte fields scattered over a block, several per
// 128-byte line) run the lm-head's weight stream at 78 us where a plain read
// of the same bytes takes 64 us; read as consecutive 16-byte pieces per lane
// with the nontemporal hint, the same bytes stream at the plain-read rate.
// So each wave copies its row into its own LDS buffer with such loads (the
// next row's pieces in flight in registers while the current row is
// dotted) and the units load their fields from the LDS copy.
__host__ __device__ constexpr int64_t qmv_stage_xbytes(int m, int64_t k) {
  return (m * ((int64_t)xpad((int)k) * 2 + (k / 16) * 4) + 15) / 16 * 16;
}
// 16-byte pieces per lane that cover a row of K <= 4096 values
template <int C>
__host__ __device__ constexpr int qmv_stage_pieces() {
  return (Geo<C>::BB * (4096 / Geo<C>::BV) + 1023) / 1024;
}
// K <= 4096 (the activation rows whole in LDS) and at least 4096 weight
// rows.  One or two rows: against the one-pass and streaming kernels, q4_K
// 4096 x 4096 4.50 -> 4.40 us, the q6_K lm-head 81 -> 70 us, q8_0 14336 x
// 4096 13.2 -> 12.1 us (M = 1) and 16.7 -> 13.4 us (M = 2).  Three rows, and
// four for the codecs whose matrix-core decode is dearest, against the
// matrix-core GEMV (14336 x 4096 unless noted): q3_K 26.2 -> 14.1 us (M = 3)
// and 26.3 -> 17.9 us (M = 4), q6_K 25.8 -> 15.9 / 26.0 -> 20.2, q8_0 22.5 ->
// 17.8 / 24.0 -> 19.1, q5_K 18.9 -> 14.8 / 19.0 -> 17.3, q4_K 4096 x 4096
// 7.20 -> 6.23 at M = 3 but 7.32 -> 7.71 at M = 4.
template <int C>
__host__ __device__ constexpr int qmv_stage_max_m() {
  return C == Q8_0 || C == Q5_K || C == Q3_K || C == Q6_K || C == Q5_0 ? 4 : 3;
}
__host__ inline bool qmv_stage_use(int64_t n, int64_t k) { return k <= 4096 && n >= 4096; }
template <int C>
__host__ inline bool qmv_stage_ok(const void* w, int64_t rb) {
  return ((uintptr_t)w & 15) == 0 && rb % 16 == 0 && rb <= qmv_stage_pieces<C>() * 64 * 16;
}

template <int C, int M, bool F16>
__global__ __launch_bounds__(QMV_THREADS) void qmv_stage_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                                int64_t row_bytes, const half_t* __restrict__ x,
                                                                void* __restrict__ y, int nblocks) {
  typedef typename UnitOf<C>::T Unit;
  constexpr int NPL = qmv_stage_pieces<C>();
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  half_t* xs = (half_t*)smem;
  const int xstride = xpad(k);
  float* xsum = (float*)(smem + (size_t)M * xstride * 2);
  const int sstride = k / 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ue = k / 64;
  const int np = (int)(row_bytes / 16);  // 16-byte pieces per row
  uint8_t* wl = smem + qmv_stage_xbytes(M, k) + (int64_t)wave * row_bytes;  // this wave's row copy
  auto row_of = [&](int b) { return b * (QMV_THREADS / 64) + wave; };

  // the pieces of one row, lane l taking pieces l + 64 i (indices past the
  // row re-read its last piece and are not stored)
  auto issue = [&](u32x4* pr, int row) __attribute__((always_inline)) {
    const u32x4* src = (const u32x4*)(w + (int64_t)(row < n ? row : n - 1) * row_bytes);
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int p = lane + 64 * i;
      pr[i] = __builtin_nontemporal_load(src + (p < np ? p : np - 1));
    }
  };
  // the row's pieces into the wave's buffer: the previous row's unit fields
  // were read from it before that row's dot, earlier in the wave's program
  // order (a wave's LDS accesses are performed in order)
  auto stage = [&](const u32x4* pr) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int p = lane + 64 * i;
      if (p < np) *(u32x4*)(wl + 16 * p) = pr[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto xv_of = [&]() { return Xv{xs, xsum, xstride, sstride, 0}; };
  auto row_dot = [&](int b) __attribute__((always_inline)) {
    const int row = row_of(b);
    const int u = lane < ue ? lane : ue - 1;
    Unit un;
    un.load(wl, u);
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;
    if (lane < ue) un.template dot<M>(u, xv_of(), acc);
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = wave_sum_last(acc[m]);
    if (row < n && lane == 63) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (F16)
          ((half_t*)y)[(int64_t)m * n + row] = (half_t)acc[m];
        else
          ((float*)y)[(int64_t)m * n + row] = acc[m];
      }
    }
  };

  // x first (its loads retire before the weights'), then the first rows' pieces
  // piece c of x: row m = c / kp, K offset 8 (c - m kp)
  constexpr int XPT = M * 4096 / 8 / QMV_THREADS;
  const int kp = k / 8, xpieces = M * kp;
  u32x4 xr[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    int c = tid + i * QMV_THREADS;
    c = c < xpieces ? c : xpieces - 1;
    xr[i] = *(const u32x4*)(x + (int64_t)c * 8);  // rows are contiguous: row m, K offset v at m k + v = 8 c
  }
  const int g = gridDim.x;
  int b = blockIdx.x;
  u32x4 pa[NPL];
  issue(pa, row_of(b));
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = tid + i * QMV_THREADS;
    const uint32_t one2 = 0x3C003C00u;  // (1.0, 1.0)
    float s = 0.f;
    s = dot2(xr[i].x, one2, s); s = dot2(xr[i].y, one2, s); s = dot2(xr[i].z, one2, s); s = dot2(xr[i].w, one2, s);
    s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, false));
    if (c < xpieces) {
      int m = 0;
#pragma unroll
      for (int j = 1; j < M; ++j) m += c >= j * kp ? 1 : 0;
      const int v = xperm<C>((c - m * kp) * 8);
      *(u32x4*)(xs + m * xstride + xpad(v)) = xr[i];
      if ((c & 1) == 0) xsum[m * sstride + (v >> 4)] = s;
    }
  }
  __syncthreads();

  for (; b < nblocks; b += g) {
    stage(pa);
    if (b + g < nblocks) issue(pa, row_of(b + g));  // uniform
    row_dot(b);
  }
}

// GEMV with the matmul epilogue (residual, gate, bias), and the GLU product
// of two matrices sharing x (mlx-kquant bindings.cpp page,
// quantized_matmul_residual / _qmv_bias / _glu docstrings), on the dot2 body.
// The callers route the residual epilogue here for M <= 2 (q8_0: M <= 4), and
// for M <= 8 when K is not a multiple of 64; 3 .. 8 rows otherwise take the
// 16-row matrix-core GEMV and 9 .. 64 the wide one, each with the same store.
// The GLU product takes this body for M <= QMV_GLU_MAX_M (two matrices' units
// for more rows overflow the registers).
template <int C, int M, int LPR, bool F16>
__global__ __launch_bounds__(QMV_THREADS) void qmv_epi_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                              int64_t row_bytes, const half_t* __restrict__ x,
                                                              Epi epi, void* __restrict__ y) {
  qmv_rows<C, M, LPR, F16, 1, 0, true>(w, n, k, row_bytes, x, y, blockIdx.x, nullptr, 0.f, epi);
}

template <int C, int M, int LPR, bool F16, int ACT>
__global__ __launch_bounds__(QMV_THREADS) void qmv_glu_kernel(const uint8_t* __restrict__ w_gate,
                                                              const uint8_t* __restrict__ w_up, int n, int k,
                                                              int64_t row_bytes, const half_t* __restrict__ x,
                                                              void* __restrict__ y) {
  qmv_rows<C, M, LPR, F16, 2, ACT, true>(w_gate, n, k, row_bytes, x, y, blockIdx.x, w_up);
}

// Gathered GEMV (mlx-kquant bindings.cpp page, gather_qmv_kq docstring: one
// activation row per expert slot, output row r = x[r] times expert ids[r]'s
// dequantized weight, transposed).  blockIdx.y is the routed row; a row
// whose id is not below n_experts is left unwritten.
template <int C, int LPR, bool F16>
__global__ __launch_bounds__(QMV_THREADS) void gather_qmv_kernel(const uint8_t* __restrict__ w, int n_experts,
                                                                 int64_t expert_stride, int n, int k,
                                                                 int64_t row_bytes, const half_t* __restrict__ x,
                                                                 const uint32_t* __restrict__ ids, int row0,
                                                                 void* __restrict__ y) {
  const int r = row0 + (int)blockIdx.y;
  const uint32_t e = ids[r];
  if (e >= (uint32_t)n_experts) return;  // the whole workgroup leaves before any barrier
  void* yr = F16 ? (void*)((half_t*)y + (int64_t)r * n) : (void*)((float*)y + (int64_t)r * n);
  qmv_rows<C, 1, LPR, F16>(w + (int64_t)e * expert_stride, n, k, row_bytes, x + (int64_t)r * k, yr, blockIdx.x);
}

// MoE GLU gather (mlx-kquant bindings.cpp page, moe_glu_gather_kq
// docstring): routed slot r of token t = r / top_k gives y[r] =
// act(x[t] . gate[e]) * (x[t] . up[e]) row by row, e = ids[r]; gate and up
// rows of the expert share each staged activation chunk.  blockIdx.y is the
// routed slot; a slot whose id is not below n_experts is left unwritten.
template <int C, int LPR, bool F16, int ACT>
__global__ __launch_bounds__(QMV_THREADS) void moe_glu_gather_kernel(
    const uint8_t* __restrict__ gate_w, const uint8_t* __restrict__ up_w, int n_experts, int64_t expert_stride, int n,
    int k, int64_t row_bytes, const half_t* __restrict__ x, const uint32_t* __restrict__ ids, int top_k, int row0,
    float limit, void* __restrict__ y) {
  const int r = row0 + (int)blockIdx.y;
  const uint32_t e = ids[r];
  if (e >= (uint32_t)n_experts) return;  // the whole workgroup leaves before any barrier
  void* yr = F16 ? (void*)((half_t*)y + (int64_t)r * n) : (void*)((float*)y + (int64_t)r * n);
  qmv_rows<C, 1, LPR, F16, 2, ACT>(gate_w + (int64_t)e * expert_stride, n, k, row_bytes, x + (int64_t)(r / top_k) * k,
                                   yr, blockIdx.x, up_w + (int64_t)e * expert_stride, limit);
}

// Generic GEMV for shapes the unit kernels do not take (q8_0 / q4_0 with an
// odd number of blocks per row): one wave per row, 8 values per lane step.
// EP / ACT / epi: the output store, as in the GEMM (store_out).
template <int C, bool F16, int EP = EP_PLAIN, int ACT = 0>
__global__ __launch_bounds__(256) void qmv_generic_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                          int64_t row_bytes, const half_t* __restrict__ x, int m,
                                                          void* __restrict__ y, Epi epi) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  float acc[QMV_MAX_M];
#pragma unroll
  for (int mm = 0; mm < QMV_MAX_M; ++mm) acc[mm] = 0.f;
  const uint8_t* wrow = w + (int64_t)row * row_bytes;
  for (int g = lane; g < k / 8; g += 64) {
    float v[8];
    decode8<C>(wrow, (int64_t)g * 8, v);
#pragma unroll
    for (int mm = 0; mm < QMV_MAX_M; ++mm) {
      if (mm < m) {
        const half8_t xv = *(const half8_t*)(x + (int64_t)mm * k + 8 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[mm] += v[i] * (float)xv[i];
      }
    }
  }
#pragma unroll
  for (int mm = 0; mm < QMV_MAX_M; ++mm) {
    float s = acc[mm];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0 && mm < m) store_out<F16, EP, ACT>(y, mm, row, n, epi, s);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core GEMV for 3 <= M <= 16 activation rows.  With more than two rows
// the dot2 path spends M v_dot2 per pair of weights; here each weight is
// decoded once to float16 (its exact value rounded once) and the products go
// to v_mfma_f32_16x16x32_f16.  B operand: 16 weight rows x 32 K values, lane
// l holding row (l & 15) and 8 consecutive values of unit 4g + (l >> 4) of
// that row, so each lane still decodes whole units from their wire bytes.
// The contraction only needs A and B to agree on K, so the 32 K values of an
// MFMA come from four different units.  A operand: the same K positions of
// activation row (l & 15); rows past M repeat row M - 1 and their outputs are
// dropped.  A wave owns 16 weight rows and a part of K (KS waves of a
// workgroup share a row group: MMA_KSPLIT, or four for a matrix with few
// rows); the parts meet in LDS at the end.
// ---------------------------------------------------------------------------

constexpr int MMA_THREADS = 256;
constexpr int MMA_KSPLIT = 2;  // waves of a workgroup sharing one 16-row group, each a part of K
constexpr int MMA_PD = 4;      // units of a lane in flight ahead of the one decoded
// K values per LDS chunk: at most 64 KiB of activations.
__host__ __device__ constexpr int mma_kchunk(int m) { return (32768 / m) & ~255; }
__host__ __device__ constexpr int mma_xstride(int kc) { return xpad(kc) + 8; }  // +16 B: rows start on different banks

template <int C, int M, bool F16, int EP = EP_PLAIN, int KS = MMA_KSPLIT>
__global__ __launch_bounds__(MMA_THREADS) void qmv_mma_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                              int64_t row_bytes, const half_t* __restrict__ x,
                                                              void* __restrict__ y, Epi epi, int act) {
  typedef typename UnitOf<C>::T Unit;
  static_assert(M >= 1 && M <= 16, "activation rows");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int KC = mma_kchunk(M);
  const int kc_alloc = k < KC ? k : KC;
  half_t* xs = (half_t*)smem;
  const int xstride = mma_xstride(kc_alloc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rgroup = blockIdx.x * (4 / KS) + wave / KS, kpart = wave % KS;
  const int r = lane & 15, cu = lane >> 4;
  const int row = rgroup * 16 + r;
  const uint8_t* wrow = w + (int64_t)min(row, n - 1) * row_bytes;
  const int xm = min(r, M - 1);

  float4_t acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};  // even / odd slices
  for (int c0 = 0; c0 < k; c0 += KC) {
    const int kc = (k - c0) < KC ? (k - c0) : KC;
    const int ub = c0 / 64, ue = (c0 + kc) / 64;
    // this wave's groups (4 units each): [g0, g1) of the chunk's groups
    const int ngroups = (ue - ub + 3) / 4, gper = (ngroups + KS - 1) / KS;
    const int g0 = min(kpart * gper, ngroups), g1 = min(g0 + gper, ngroups);
    const int last = ue - 1;
    // Activation loads first (all of this thread's pieces at once, so their
    // latencies overlap), then the first units' weight loads.
    constexpr int XPT = (M * KC / 8 + MMA_THREADS - 1) / MMA_THREADS;
    const int xpieces = M * (kc / 8);
    u32x4 xr[XPT];
    {
      PieceWalk pw(tid, kc / 8, MMA_THREADS);  // pieces past the block re-read its last one
#pragma unroll
      for (int i = 0; i < XPT; ++i, pw.next()) {
        const bool in = tid + i * MMA_THREADS < xpieces;
        const int m = in ? pw.m : M - 1, v = (in ? pw.r : kc / 8 - 1) * 8;
        xr[i] = *(const u32x4*)(x + (int64_t)m * k + c0 + v);
      }
    }
    Unit ring[MMA_PD];
#pragma unroll
    for (int p = 0; p < MMA_PD; ++p) ring[p].load(wrow, min(ub + 4 * (g0 + p) + cu, last));
    if (c0) __syncthreads();  // previous chunk done with LDS
    {
      PieceWalk pw(tid, kc / 8, MMA_THREADS);
#pragma unroll
      for (int i = 0; i < XPT; ++i, pw.next()) {
        if (tid + i * MMA_THREADS < xpieces) *(u32x4*)(xs + pw.m * xstride + xpad(pw.r * 8)) = xr[i];
      }
    }
    __syncthreads();
    const half_t* xrow = xs + xm * xstride;
    // Slot j of the ring always holds group g + j: the loop is unrolled by
    // the ring depth so no register is copied while its load is in flight.
    // Groups past g1 (the last pass) are masked, not branched around.
    for (int g = g0; g < g1; g += MMA_PD) {
#pragma unroll
      for (int j = 0; j < MMA_PD; ++j) {
        const int u = ub + 4 * (g + j) + cu;
        const bool valid = g + j < g1 && u < ue;  // else this lane adds zeros
        const int uc = valid ? u : last;           // (and reads in-range x)
        // Activation fragments and the unit's eight weight fragments first,
        // so the slot's bytes are dead before its next load is issued (the
        // load then reuses the slot's registers: nothing is copied, nothing
        // waits at the loop edge).
        half8_t a[8];
        u32x4 fw[8];
        const MmaSlices<C> sl(ring[j], uc, valid);
        const half_t* xb = xrow + xpad(MmaSlices<C>::koff(uc) - c0);
        auto prep = [&](auto sc) __attribute__((always_inline)) {
          constexpr int S = decltype(sc)::value;
          a[S] = *(const half8_t*)(xb + MmaSlices<C>::template xstep<S>());
          uint32_t f[4];
          sl.template get<S>(f);
          fw[S] = u32x4{f[0], f[1], f[2], f[3]};
        };
        prep(std::integral_constant<int, 0>{});
        prep(std::integral_constant<int, 1>{});
        prep(std::integral_constant<int, 2>{});
        prep(std::integral_constant<int, 3>{});
        prep(std::integral_constant<int, 4>{});
        prep(std::integral_constant<int, 5>{});
        prep(std::integral_constant<int, 6>{});
        prep(std::integral_constant<int, 7>{});
        __builtin_amdgcn_sched_barrier(0);
        ring[j].load(wrow, min(u + 4 * MMA_PD, last));
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], __builtin_bit_cast(half8_t, fw[t]), acc, 0, 0, 0);
          acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t + 1], __builtin_bit_cast(half8_t, fw[t + 1]), acc2, 0, 0, 0);
        }
      }
    }
  }

  // Combine the K parts: lane l holds activation rows 4 (l >> 4) + i of
  // weight row 16 rgroup + (l & 15).
  acc += acc2;
  __syncthreads();
  float4_t* part = (float4_t*)smem;
  const int pbase = (wave / KS) * (KS - 1) * 64;
  if (kpart) part[pbase + (kpart - 1) * 64 + lane] = acc;
  __syncthreads();
  if (kpart == 0) {
#pragma unroll
    for (int p = 0; p + 1 < KS; ++p) acc += part[pbase + p * 64 + lane];
    const int col = rgroup * 16 + (lane & 15);
    if (col < n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * (lane >> 4) + i;
        if (m < M) {
          if constexpr (EP == EP_GLU_ACT) {
            if (act == GLU_SILU)
              store_out<F16, EP, GLU_SILU>(y, m, col, n, epi, acc[i]);
            else
              store_out<F16, EP, GLU_GELU_TANH>(y, m, col, n, epi, acc[i]);
          } else {
            store_out<F16, EP, 0>(y, m, col, n, epi, acc[i]);
          }
        }
      }
    }
  }
}

// The same kernel with a store mode (kq_internal.h; act: the GLU gate pass's
// activation).
template <int C, int M, int EP, int KS>
hipError_t launch_mma_ks(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, const Epi& epi, int act,
                         void* y, int f16, hipStream_t s) {
  const int kc = (int)(k < mma_kchunk(M) ? k : mma_kchunk(M));
  size_t lds = (size_t)M * mma_xstride(kc) * 2;
  const size_t part_bytes = (size_t)(4 / KS) * (KS - 1) * 64 * sizeof(float4_t);
  if (lds < part_bytes) lds = part_bytes;
  constexpr int rows_per_block = 16 * (4 / KS);
  const dim3 grid((unsigned)((n + rows_per_block - 1) / rows_per_block));
  if (f16)
    hipLaunchKernelGGL((qmv_mma_kernel<C, M, true, EP, KS>), grid, dim3(MMA_THREADS), lds, s, w, (int)n, (int)k, rb, x, y,
                       epi, act);
  else
    hipLaunchKernelGGL((qmv_mma_kernel<C, M, false, EP, KS>), grid, dim3(MMA_THREADS), lds, s, w, (int)n, (int)k, rb, x,
                       y, epi, act);
  return hipGetLastError();
}

// Four waves per row group for a matrix so narrow that two leave CUs without
// a workgroup (wide_narrow), else two.
template <int C, int M, int EP>
hipError_t launch_mma_ep(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, const Epi& epi, int act,
                         void* y, int f16, hipStream_t s) {
  if (wide_narrow(n)) return launch_mma_ks<C, M, EP, 4>(w, n, k, rb, x, epi, act, y, f16, s);
  return launch_mma_ks<C, M, EP, 2>(w, n, k, rb, x, epi, act, y, f16, s);
}

template <int C, int M>
hipError_t launch_mma(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, void* y, int f16,
                      hipStream_t s) {
  return launch_mma_ep<C, M, EP_PLAIN>(w, n, k, rb, x, Epi{nullptr, nullptr, nullptr, 1}, 0, y, f16, s);
}

template <int C, int M, int LPR>
hipError_t launch_ml(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, void* y, int f16,
                     hipStream_t s) {
  const int kc = (int)(k < kchunk_max(M) ? k : kchunk_max(M));
  const size_t lds = (size_t)M * xpad(kc) * 2 + (size_t)M * (kc / 16) * 4;
  const dim3 grid((unsigned)((n + rows_per_block(LPR) - 1) / rows_per_block(LPR)));
  if (f16)
    hipLaunchKernelGGL((qmv_kernel<C, M, LPR, true>), grid, dim3(QMV_THREADS), lds, s, w, (int)n, (int)k, rb, x, y);
  else
    hipLaunchKernelGGL((qmv_kernel<C, M, LPR, false>), grid, dim3(QMV_THREADS), lds, s, w, (int)n, (int)k, rb, x, y);
  return hipGetLastError();
}

// The streaming GEMV: one or two activation rows, K <= 4096 and at least
// 8192 weight rows (the q6_K 128256 x 4096 lm-head: 119 -> 89 us; q4_0
// 14336 x 4096, one row: 9.4 -> 8.5 us; at 4096 rows the one-pass kernel
// stays ahead).  One row: a wave per row and about four row blocks per
// workgroup (1024 to 8192 workgroups); two rows: 16 lanes per row and one
// block per workgroup (5% ahead of the one-pass kernel at 14336 rows).
__host__ inline bool qmv_stream_ok(int m, int64_t n, int64_t k) { return m <= 2 && k <= 4096 && n >= 8192; }
__host__ inline int64_t qmv_stream_grid(int m, int64_t nblocks) {
  if (m > 1) return nblocks;
  return std::max<int64_t>(1, std::min<int64_t>(nblocks, std::max<int64_t>(1024, std::min<int64_t>(8192, nblocks / 4))));
}

template <int C, int M, int LPR, int PD>
hipError_t launch_stream_pd(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, void* y, int f16,
                            hipStream_t s) {
  const size_t lds = (size_t)M * xpad((int)k) * 2 + (size_t)M * (k / 16) * 4;
  const int64_t nblocks = (n + rows_per_block(LPR) - 1) / rows_per_block(LPR);
  const dim3 grid((unsigned)qmv_stream_grid(M, nblocks));
  if (f16)
    hipLaunchKernelGGL((qmv_stream_kernel<C, M, LPR, true, PD>), grid, dim3(QMV_THREADS), lds, s, w, (int)n, (int)k, rb,
                       x, y, (int)nblocks);
  else
    hipLaunchKernelGGL((qmv_stream_kernel<C, M, LPR, false, PD>), grid, dim3(QMV_THREADS), lds, s, w, (int)n, (int)k,
                       rb, x, y, (int)nblocks);
  return hipGetLastError();
}
template <int C, int M, int LPR>
hipError_t launch_stream(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, void* y, int f16,
                         hipStream_t s) {
  return launch_stream_pd<C, M, LPR, 1>(w, n, k, rb, x, y, f16, s);
}

template <int C, int M>
hipError_t launch_stage(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, void* y, int f16,
                        hipStream_t s) {
  const int64_t nblocks = (n + QMV_THREADS / 64 - 1) / (QMV_THREADS / 64);
  const size_t lds = (size_t)qmv_stage_xbytes(M, k) + (size_t)(QMV_THREADS / 64) * rb;
  const dim3 grid((unsigned)qmv_stream_grid(1, nblocks));
  if (f16)
    hipLaunchKernelGGL((qmv_stage_kernel<C, M, true>), grid, dim3(QMV_THREADS), lds, s, w, (int)n, (int)k, rb, x, y,
                       (int)nblocks);
  else
    hipLaunchKernelGGL((qmv_stage_kernel<C, M, false>), grid, dim3(QMV_THREADS), lds, s, w, (int)n, (int)k, rb, x, y,
                       (int)nblocks);
  return hipGetLastError();
}

// Three or more activation rows (five or more for q8_0) go to the matrix
// cores.  Fewer take the dot2 kernel: one wave per row (64 lanes, one 64-value unit each at
// K = 4096) for one activation row and a matrix with few rows (four times
// the workgroups and a quarter of the serial work per lane), otherwise 16
// lanes per row, so the activation staging is shared by 16 rows per
// workgroup.
template <int C, int M>
hipError_t launch_m(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, void* y, int f16,
                    hipStream_t s) {
  // q8_0's decode costs the matrix path more per byte: its dot2 kernel is
  // still the faster one at four rows.
  constexpr int mma_from = C == Q8_0 ? 5 : 3;
  if constexpr (M <= qmv_stage_max_m<C>())
    if (qmv_stage_use(n, k) && qmv_stage_ok<C>(w, rb)) return launch_stage<C, M>(w, n, k, rb, x, y, f16, s);
  if constexpr (M >= mma_from) {
    return launch_mma<C, M>(w, n, k, rb, x, y, f16, s);
  } else {
    if (qmv_stream_ok(M, n, k)) return launch_stream<C, M, (M == 1 ? 64 : 16)>(w, n, k, rb, x, y, f16, s);
    if (M == 1 && n <= 32768) return launch_ml<C, M, 64>(w, n, k, rb, x, y, f16, s);
    return launch_ml<C, M, 16>(w, n, k, rb, x, y, f16, s);
  }
}

template <int C, int EP, int ACT>
hipError_t launch_generic(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int m, void* y,
                          int f16, const Epi& epi, hipStream_t s) {
  const dim3 grid((unsigned)((n + 3) / 4));
  if (f16)
    hipLaunchKernelGGL((qmv_generic_kernel<C, true, EP, ACT>), grid, dim3(256), 0, s, w, (int)n, (int)k, rb, x, m, y,
                       epi);
  else
    hipLaunchKernelGGL((qmv_generic_kernel<C, false, EP, ACT>), grid, dim3(256), 0, s, w, (int)n, (int)k, rb, x, m, y,
                       epi);
  return hipGetLastError();
}

template <int C>
hipError_t launch_c(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int m, void* y, int f16,
                    hipStream_t s) {
  // The unit kernels need whole 64-value units per row (q8_0 / q4_0: an even block count).
  if (k % 64 != 0) return launch_generic<C, EP_PLAIN, 0>(w, n, k, rb, x, m, y, f16, Epi{nullptr, nullptr, nullptr, 1}, s);
  switch (m) {
    case 1: return launch_m<C, 1>(w, n, k, rb, x, y, f16, s);
    case 2: return launch_m<C, 2>(w, n, k, rb, x, y, f16, s);
    case 3: return launch_m<C, 3>(w, n, k, rb, x, y, f16, s);
    case 4: return launch_m<C, 4>(w, n, k, rb, x, y, f16, s);
    case 5: return launch_m<C, 5>(w, n, k, rb, x, y, f16, s);
    case 6: return launch_m<C, 6>(w, n, k, rb, x, y, f16, s);
    case 7: return launch_m<C, 7>(w, n, k, rb, x, y, f16, s);
    case 8: return launch_m<C, 8>(w, n, k, rb, x, y, f16, s);
  }
  // 9..16 rows: the wide matrix-core GEMV on one 16-row A operand, whose
  // next chunk's weights load while the current chunk is consumed
  if (m >= 9 && m <= QMV_MAX_M) return launch_qmv_wide(C, w, n, k, rb, x, m, y, f16, s);
  return hipErrorInvalidValue;
}

// mode 0: epilogue; 1..3: GLU with act = mode - 1 (GLU_SILU, GLU_GELU_TANH)
template <int C, int M, int LPR>
hipError_t launch_fused_ml(const uint8_t* w, const uint8_t* w2, int64_t n, int64_t k, int64_t rb, const half_t* x,
                           const Epi& epi, int act, bool glu, void* y, int f16, hipStream_t s) {
  const int kc = (int)(k < kchunk_max(M) ? k : kchunk_max(M));
  const size_t lds = (size_t)M * xpad(kc) * 2 + (size_t)M * (kc / 16) * 4;
  const dim3 grid((unsigned)((n + rows_per_block(LPR) - 1) / rows_per_block(LPR)));
  if (!glu) {
    if (f16)
      hipLaunchKernelGGL((qmv_epi_kernel<C, M, LPR, true>), grid, dim3(QMV_THREADS), lds, s, w, (int)n, (int)k, rb, x,
                         epi, y);
    else
      hipLaunchKernelGGL((qmv_epi_kernel<C, M, LPR, false>), grid, dim3(QMV_THREADS), lds, s, w, (int)n, (int)k, rb,
                         x, epi, y);
  } else if constexpr (M > qmv_glu_max_m(C)) {
    return hipErrorInvalidValue;
  } else if (act == GLU_SILU) {
    if (f16)
      hipLaunchKernelGGL((qmv_glu_kernel<C, M, LPR, true, GLU_SILU>), grid, dim3(QMV_THREADS), lds, s, w, w2, (int)n,
                         (int)k, rb, x, y);
    else
      hipLaunchKernelGGL((qmv_glu_kernel<C, M, LPR, false, GLU_SILU>), grid, dim3(QMV_THREADS), lds, s, w, w2, (int)n,
                         (int)k, rb, x, y);
  } else {
    if (f16)
      hipLaunchKernelGGL((qmv_glu_kernel<C, M, LPR, true, GLU_GELU_TANH>), grid, dim3(QMV_THREADS), lds, s, w, w2,
                         (int)n, (int)k, rb, x, y);
    else
      hipLaunchKernelGGL((qmv_glu_kernel<C, M, LPR, false, GLU_GELU_TANH>), grid, dim3(QMV_THREADS), lds, s, w, w2,
                         (int)n, (int)k, rb, x, y);
  }
  return hipGetLastError();
}

template <int C, int M>
hipError_t launch_fused_m(const uint8_t* w, const uint8_t* w2, int64_t n, int64_t k, int64_t rb, const half_t* x,
                          const Epi& epi, int act, bool glu, void* y, int f16, hipStream_t s) {
  if (M == 1 && n <= 32768) return launch_fused_ml<C, M, 64>(w, w2, n, k, rb, x, epi, act, glu, y, f16, s);
  return launch_fused_ml<C, M, 16>(w, w2, n, k, rb, x, epi, act, glu, y, f16, s);
}

template <int C>
hipError_t launch_fused_c(const uint8_t* w, const uint8_t* w2, int64_t n, int64_t k, int64_t rb, const half_t* x,
                          int m, const Epi& epi, int act, bool glu, void* y, int f16, hipStream_t s) {
  if (k % 64 != 0) {  // odd block count (32-value codecs): the generic kernel; the GLU in two passes
    if constexpr (is_block32<C>()) {
      if (!glu) return launch_generic<C, EP_EPI, 0>(w, n, k, rb, x, m, y, f16, epi, s);
      const hipError_t e =
          act == GLU_SILU ? launch_generic<C, EP_GLU_ACT, GLU_SILU>(w, n, k, rb, x, m, y, f16, epi, s)
                          : launch_generic<C, EP_GLU_ACT, GLU_GELU_TANH>(w, n, k, rb, x, m, y, f16, epi, s);
      if (e != hipSuccess) return e;
      return launch_generic<C, EP_GLU_MUL, 0>(w2, n, k, rb, x, m, y, f16, epi, s);
    }
    return hipErrorInvalidValue;
  }
  switch (m) {
    case 1: return launch_fused_m<C, 1>(w, w2, n, k, rb, x, epi, act, glu, y, f16, s);
    case 2: return launch_fused_m<C, 2>(w, w2, n, k, rb, x, epi, act, glu, y, f16, s);
    case 3: return launch_fused_m<C, 3>(w, w2, n, k, rb, x, epi, act, glu, y, f16, s);
    case 4: return launch_fused_m<C, 4>(w, w2, n, k, rb, x, epi, act, glu, y, f16, s);
    case 5: return launch_fused_m<C, 5>(w, w2, n, k, rb, x, epi, act, glu, y, f16, s);
    case 6: return launch_fused_m<C, 6>(w, w2, n, k, rb, x, epi, act, glu, y, f16, s);
    case 7: return launch_fused_m<C, 7>(w, w2, n, k, rb, x, epi, act, glu, y, f16, s);
    case 8: return launch_fused_m<C, 8>(w, w2, n, k, rb, x, epi, act, glu, y, f16, s);
  }
  return hipErrorInvalidValue;
}


template <int C, int LPR>
hipError_t launch_gather_l(const uint8_t* w, int64_t ne, int64_t n, int64_t k, int64_t rb, const half_t* x,
                           const uint32_t* ids, int64_t rows, void* y, int f16, hipStream_t s) {
  const int kc = (int)(k < kchunk_max(1) ? k : kchunk_max(1));
  const size_t lds = (size_t)xpad(kc) * 2 + (size_t)(kc / 16) * 4;
  const unsigned gx = (unsigned)((n + rows_per_block(LPR) - 1) / rows_per_block(LPR));
  for (int64_t r0 = 0; r0 < rows; r0 += 65535) {  // grid y holds at most 65535 rows per launch
    const dim3 grid(gx, (unsigned)(rows - r0 < 65535 ? rows - r0 : 65535));
    if (f16)
      hipLaunchKernelGGL((gather_qmv_kernel<C, LPR, true>), grid, dim3(QMV_THREADS), lds, s, w, (int)ne, n * rb,
                         (int)n, (int)k, rb, x, ids, (int)r0, y);
    else
      hipLaunchKernelGGL((gather_qmv_kernel<C, LPR, false>), grid, dim3(QMV_THREADS), lds, s, w, (int)ne, n * rb,
                         (int)n, (int)k, rb, x, ids, (int)r0, y);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int C, int LPR, int ACT>
hipError_t launch_glu_l(const uint8_t* gw, const uint8_t* uw, int64_t ne, int64_t n, int64_t k, int64_t rb,
                        const half_t* x, const uint32_t* ids, int64_t rows, int64_t top_k, float limit, void* y,
                        int f16, hipStream_t s) {
  const int kc = (int)(k < kchunk_max(1) ? k : kchunk_max(1));
  const size_t lds = (size_t)xpad(kc) * 2 + (size_t)(kc / 16) * 4;
  const unsigned gx = (unsigned)((n + rows_per_block(LPR) - 1) / rows_per_block(LPR));
  for (int64_t r0 = 0; r0 < rows; r0 += 65535) {  // grid y holds at most 65535 rows per launch
    const dim3 grid(gx, (unsigned)(rows - r0 < 65535 ? rows - r0 : 65535));
    if (f16)
      hipLaunchKernelGGL((moe_glu_gather_kernel<C, LPR, true, ACT>), grid, dim3(QMV_THREADS), lds, s, gw, uw, (int)ne,
                         n * rb, (int)n, (int)k, rb, x, ids, (int)top_k, (int)r0, limit, y);
    else
      hipLaunchKernelGGL((moe_glu_gather_kernel<C, LPR, false, ACT>), grid, dim3(QMV_THREADS), lds, s, gw, uw, (int)ne,
                         n * rb, (int)n, (int)k, rb, x, ids, (int)top_k, (int)r0, limit, y);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int C, int ACT>
hipError_t launch_glu_a(const uint8_t* gw, const uint8_t* uw, int64_t ne, int64_t n, int64_t k, int64_t rb,
                        const half_t* x, const uint32_t* ids, int64_t rows, int64_t top_k, float limit, void* y,
                        int f16, hipStream_t s) {
  if (n <= 32768) return launch_glu_l<C, 64, ACT>(gw, uw, ne, n, k, rb, x, ids, rows, top_k, limit, y, f16, s);
  return launch_glu_l<C, 16, ACT>(gw, uw, ne, n, k, rb, x, ids, rows, top_k, limit, y, f16, s);
}

template <int C>
hipError_t launch_glu_c(const uint8_t* gw, const uint8_t* uw, int64_t ne, int64_t n, int64_t k, int64_t rb,
                        const half_t* x, const uint32_t* ids, int64_t rows, int64_t top_k, int act, float limit,
                        void* y, int f16, hipStream_t s) {
  switch (act) {
    case GLU_SILU: return launch_glu_a<C, GLU_SILU>(gw, uw, ne, n, k, rb, x, ids, rows, top_k, limit, y, f16, s);
    case GLU_GELU_TANH:
      return launch_glu_a<C, GLU_GELU_TANH>(gw, uw, ne, n, k, rb, x, ids, rows, top_k, limit, y, f16, s);
    case GLU_SILU_LIMIT:
      return launch_glu_a<C, GLU_SILU_LIMIT>(gw, uw, ne, n, k, rb, x, ids, rows, top_k, limit, y, f16, s);
  }
  return hipErrorInvalidValue;
}

template <int C>
hipError_t launch_gather_c(const uint8_t* w, int64_t ne, int64_t n, int64_t k, int64_t rb, const half_t* x,
                           const uint32_t* ids, int64_t rows, void* y, int f16, hipStream_t s) {
  if (n <= 32768) return launch_gather_l<C, 64>(w, ne, n, k, rb, x, ids, rows, y, f16, s);
  return launch_gather_l<C, 16>(w, ne, n, k, rb, x, ids, rows, y, f16, s);
}

}  // namespace
}  // namespace kq
