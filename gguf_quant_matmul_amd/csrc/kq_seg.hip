// kq_gather_qmm_seg on the matrix cores with the weights decoded straight
// into MFMA operands.
//
// mlx-kquant bindings.cpp page, gather_qmm_seg docstring: expert-sorted rows
// walked tile by tile from a (expert, row_start, num_rows) map of at most 64
// rows per tile; rows no tile covers stay unwritten.
//
// A tile holds at most 64 activation rows, so a weight decoded into shared
// LDS (as the prefill GEMM does) serves few MFMAs.  Here no weight goes
// through LDS:
//  * a workgroup takes one tile and 192 weight rows of its expert; each of
//    its four waves owns 48 rows (three groups of 16) and decodes them from
//    their wire bytes into v_mfma_f32_16x16x32_f16 B operands, lane l taking
//    row (l & 15) of a group and 8 values of unit 4g + (l >> 4) per MFMA (the
//    contraction only needs A and B to agree on K, so one MFMA's 32 K values
//    come from four units);
//  * the tile's activation rows are staged in LDS, double-buffered, in
//    chunks of 256 K values (the next chunk's loads go out before the current
//    chunk's products); every decoded B operand meets up to four 16-row
//    groups of activations, and groups past the tile's row count are not
//    computed (one code path per live group count, so the K loop has no
//    branches);
//  * each lane keeps the next unit group in flight while it decodes the
//    current one; a unit is fully decoded before its registers are reloaded;
//  * weights and activations are read with buffer loads whose moving part is
//    a wave-uniform scalar offset (no per-load address arithmetic), and every
//    load in the K loop is unconditional so the compiler's count of loads in
//    flight stays exact;
//  * the kernel fits in 256 registers and 74 KB of LDS, so two workgroups
//    share a CU and each SIMD holds two waves: one wave's decode and waits
//    overlap the other's matrix work.
#include <type_traits>

#include "kq_units.h"

namespace kq {
namespace {

constexpr int SEG_THREADS = 256;                     // four waves
constexpr int SEG_RG = 3;                            // 16-row weight groups per wave
constexpr int SEG_BN = 4 * 16 * SEG_RG;              // weight rows per workgroup (192)
constexpr int SEG_KC = 256;                          // K values per LDS chunk
constexpr int SEG_GPC = SEG_KC / 256;                // unit groups (four units per 16-lane quarter) per chunk
constexpr int SEG_XSTRIDE = xpad(SEG_KC) + 8;        // halves per staged row: rows start on different banks
constexpr int SEG_XBUF = 64 * SEG_XSTRIDE;           // halves per chunk buffer (64 rows)
constexpr int SEG_PPR = SEG_KC / 8;                  // 16-byte activation pieces per row per chunk
constexpr int SEG_RPI = SEG_THREADS / SEG_PPR;       // rows one staging pass of the workgroup covers
constexpr int SEG_NXCD = 8;

// Unit groups in flight per weight group and lane.  Two workgroups share a
// CU (two waves per SIMD), so the other one covers what latency two slots
// leave open.
template <int C> struct SegSlots { static constexpr int value = 2; };
// Workgroups per CU the register budget is sized for.  q5_K's units carry
// the 32 qh bytes as well (20 registers a unit against q4_K's 12), q3_K's
// five 2-byte-aligned spans (27): at two waves per SIMD their rings spill,
// so they take one wave per SIMD and the whole register file (the 2-slot
// ring at one wave per SIMD measured within a few percent of two waves for
// q4_K).
template <int C> struct SegOcc { static constexpr int value = (C == Q5_K || C == Q3_K) ? 1 : 2; };

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// One tile of XG live 16-row activation groups against SEG_BN weight rows.
template <int C, bool F16, int XG>
__device__ __forceinline__ void seg_tile(const uint8_t* __restrict__ wbase, int n, int k, int64_t row_bytes,
                                         const half_t* __restrict__ xtile, int64_t x_bytes, int nr, int64_t yrow0,
                                         int n0, half_t* xs, void* __restrict__ y) {
  typedef typename UnitOf<C>::T Unit;
  constexpr int NS = SegSlots<C>::value;  // ring slots, one unit group each
  constexpr int XPT = XG * 16 * SEG_PPR / SEG_THREADS;  // activation pieces per thread per chunk
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, cu = lane >> 4;
  // the wave's 48 weight rows from a dword-aligned base; rows past N read
  // as zeros
  const uintptr_t wwave = (uintptr_t)(wbase + (int64_t)(n0 + wave * 16 * SEG_RG) * row_bytes);
  const int wdelta = (int)(wwave & 3);
  const rsrc_t wrs = make_rsrc((const void*)(wwave - wdelta), (int64_t)(n - n0 - wave * 16 * SEG_RG) * row_bytes + wdelta);
  int rowoff[SEG_RG];
#pragma unroll
  for (int j = 0; j < SEG_RG; ++j) rowoff[j] = wdelta + (16 * j + r) * (int)row_bytes;
  const int units = k / 64, last4 = (units - 1) & ~3;
  // group u4 (a multiple of 4) of the three rows: unit u4 + cu in each lane;
  // groups past K re-read the last one
  auto refill = [&](Unit* slot, int u4) __attribute__((always_inline)) {
    const int g = min(u4, last4);
#pragma unroll
    for (int j = 0; j < SEG_RG; ++j) {
      slot[j].bload(wrs, rowoff[j], cu, g);
    }
  };

  float4_t acc[SEG_RG][XG];
#pragma unroll
  for (int j = 0; j < SEG_RG; ++j)
#pragma unroll
    for (int i = 0; i < XG; ++i) acc[j][i] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Piece i of a thread is row tid / SEG_PPR + SEG_RPI i, values
  // 8 (tid % SEG_PPR) .. of the chunk.  Rows past the tile and values past K hold whatever follows
  // in x, and offsets past its end read as zeros (the whole offset is the
  // per-lane operand, which the descriptor's byte count bounds); neither is
  // read for a stored output.  Every load in the K loop is unconditional, so
  // the compiler can count the loads still in flight exactly and wait only
  // for the oldest.
  const rsrc_t xrs = make_rsrc(xtile, x_bytes);
  const int xvoff = (tid / SEG_PPR) * k * 2 + (tid % SEG_PPR) * 16;
  u32x4 xr[XPT];
  auto load_x = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) xr[i] = bld16(xrs, xvoff + 2 * c0 + i * SEG_RPI * 2 * k, 0);
  };
  half_t* xst = xs + (tid / SEG_PPR) * SEG_XSTRIDE + xpad((tid % SEG_PPR) * 8);
  auto store_x = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) *(u32x4*)(xst + buf * SEG_XBUF + SEG_RPI * i * SEG_XSTRIDE) = xr[i];
  };

  // The loads keep program order (scheduling fences): slot p's loads all go
  // out before slot p + 1's, as they do in the K loop, so the wait for a
  // slot is the same on entry as on every iteration.
  load_x(0);
  Unit ring[NS][SEG_RG];
#pragma unroll
  for (int p = 0; p < NS; ++p) {
    __builtin_amdgcn_sched_barrier(0);
    refill(ring[p], 4 * p);
  }
  __builtin_amdgcn_sched_barrier(0);
  store_x(0);
  __syncthreads();

  // One chunk: SEG_GPC groups of four units (one per 16-lane quarter); ring
  // slot (SEG_GPC H + gg) % NS holds group gg of the chunk and is refilled NS
  // groups ahead.  A chunk that starts at or past K (the second of a pair)
  // adds zeros.
  auto chunk = [&](auto hc, int c0) __attribute__((always_inline)) {
    constexpr int H = decltype(hc)::value;
    const int ub = c0 / 64, ue = ub + max(min(k - c0, SEG_KC), 0) / 64;
    const int cb = (c0 / SEG_KC) & 1;
    const half_t* cur = xs + cb * SEG_XBUF;
    load_x(c0 + SEG_KC);  // stored after this chunk's products
#pragma unroll
    for (int gg = 0; gg < SEG_GPC; ++gg) {
      const int u = ub + 4 * gg + cu;
      const bool valid = u < ue;                    // else this lane adds zeros
      const int uc = valid ? u : max(ue - 1, ub);  // (and reads in-chunk activations)
      // q4_K and q5_K read only u & 3 (lane-uniform): spelled out, their
      // scale fields' offsets are computed once outside the loop
      const int us = (C == Q4_K || C == Q5_K) ? 4 * (u >> 2) + cu : uc;
      const half_t* xb = cur + r * SEG_XSTRIDE + xpad(MmaSlices<C>::koff(uc) - c0);
      const MmaSlices<C> sl0(ring[(SEG_GPC * H + gg) % NS][0], us, valid);
      const MmaSlices<C> sl1(ring[(SEG_GPC * H + gg) % NS][1], us, valid);
      const MmaSlices<C> sl2(ring[(SEG_GPC * H + gg) % NS][2], us, valid);
      auto step = [&](auto sc) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        uint32_t f0[4], f1[4], f2[4];
        sl0.template get<S>(f0);
        sl1.template get<S>(f1);
        sl2.template get<S>(f2);
        if constexpr (S == 7) {
          // every slice of the three units is decoded: refill their registers
          __builtin_amdgcn_sched_barrier(0);
          refill(ring[(SEG_GPC * H + gg) % NS], ub + 4 * gg + 4 * NS);
        }
        const half8_t b0 = __builtin_bit_cast(half8_t, u32x4{f0[0], f0[1], f0[2], f0[3]});
        const half8_t b1 = __builtin_bit_cast(half8_t, u32x4{f1[0], f1[1], f1[2], f1[3]});
        const half8_t b2 = __builtin_bit_cast(half8_t, u32x4{f2[0], f2[1], f2[2], f2[3]});
#pragma unroll
        for (int i = 0; i < XG; ++i) {
          const half8_t a = *(const half8_t*)(xb + 16 * i * SEG_XSTRIDE + MmaSlices<C>::template xstep<S>());
          acc[0][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b0, acc[0][i], 0, 0, 0);
          acc[1][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b1, acc[1][i], 0, 0, 0);
          acc[2][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b2, acc[2][i], 0, 0, 0);
        }
      };
      static_for<8>(step);
    }
    store_x(cb ^ 1);  // the other buffer was last read before the previous barrier
    __syncthreads();
  };
  for (int c0 = 0; c0 < k; c0 += 2 * SEG_KC) {
    chunk(std::integral_constant<int, 0>{}, c0);
    chunk(std::integral_constant<int, 1>{}, c0 + SEG_KC);
  }

  // lane l holds activation rows 16 i + 4 (l >> 4) + q of weight row
  // n0 + 48 wave + 16 j + (l & 15)
#pragma unroll
  for (int j = 0; j < SEG_RG; ++j) {
    const int col = n0 + wave * 16 * SEG_RG + 16 * j + (lane & 15);
    if (col >= n) continue;
#pragma unroll
    for (int i = 0; i < XG; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 16 * i + 4 * (lane >> 4) + q;
        if (row < nr) {
          const int64_t o = (yrow0 + row) * n + col;
          if (F16)
            ((half_t*)y)[o] = (half_t)acc[j][i][q];
          else
            ((float*)y)[o] = acc[j][i][q];
        }
      }
    }
  }
}

template <int C, bool F16>
__global__ __launch_bounds__(SEG_THREADS, SegOcc<C>::value) void seg_mma_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                              int64_t row_bytes, int64_t expert_stride, int n_experts,
                                                              const half_t* __restrict__ x, int m_total,
                                                              const uint32_t* __restrict__ map,
                                                              const uint32_t* __restrict__ counts, int cap,
                                                              void* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) half_t xs[2 * SEG_XBUF];

  // Workgroup b runs on XCD b % 8.  The map's live (tile, column block)
  // pairs are split into eight contiguous ranges, one per XCD, so the blocks
  // of one tile share its activations, and consecutive tiles of one expert
  // its weights, in that XCD's L2; the grid covers the map's capacity and
  // workgroups past the live count leave at once.
  const int nb = (n + SEG_BN - 1) / SEG_BN;
  const int64_t live = (int64_t)min(counts[0], (uint32_t)cap) * nb;
  const int64_t per_xcd = (live + SEG_NXCD - 1) / SEG_NXCD;
  const int64_t idx = blockIdx.x / SEG_NXCD;
  if (idx >= per_xcd) return;
  const int64_t t = (int64_t)(blockIdx.x % SEG_NXCD) * per_xcd + idx;
  if (t >= live) return;
  const int by = (int)(t / nb), n0 = (int)(t - (int64_t)by * nb) * SEG_BN;
  const uint32_t* mt = map + 3 * (size_t)by;
  const uint32_t e = mt[0], rs = mt[1], nr = mt[2];
  if (e >= (uint32_t)n_experts || nr == 0 || nr > 64 || rs >= (uint32_t)m_total || nr > (uint32_t)m_total - rs)
    return;
  const uint8_t* wbase = w + (int64_t)e * expert_stride;
  const half_t* xtile = x + (int64_t)rs * k;
  const int64_t x_bytes = (int64_t)(m_total - rs) * k * 2;
  switch ((nr + 15) >> 4) {  // 16-row activation groups holding live rows
    case 1: seg_tile<C, F16, 1>(wbase, n, k, row_bytes, xtile, x_bytes, (int)nr, rs, n0, xs, y); break;
    case 2: seg_tile<C, F16, 2>(wbase, n, k, row_bytes, xtile, x_bytes, (int)nr, rs, n0, xs, y); break;
    case 3: seg_tile<C, F16, 3>(wbase, n, k, row_bytes, xtile, x_bytes, (int)nr, rs, n0, xs, y); break;
    default: seg_tile<C, F16, 4>(wbase, n, k, row_bytes, xtile, x_bytes, (int)nr, rs, n0, xs, y); break;
  }
}

template <int C>
hipError_t launch_seg_mma_c(const uint8_t* w, int64_t ne, int64_t n, int64_t k, int64_t rb, const half_t* x,
                            int64_t rows, const uint32_t* map, const uint32_t* counts, int64_t cap, void* y, int f16,
                            hipStream_t s) {
  const int64_t pairs = cap * ((n + SEG_BN - 1) / SEG_BN);  // (tile, column block) pairs the map can hold
  const dim3 grid((unsigned)((pairs + SEG_NXCD - 1) / SEG_NXCD * SEG_NXCD));
  if (f16)
    hipLaunchKernelGGL((seg_mma_kernel<C, true>), grid, dim3(SEG_THREADS), 0, s, w, (int)n, (int)k, rb, n * rb,
                       (int)ne, x, (int)rows, map, counts, (int)cap, y);
  else
    hipLaunchKernelGGL((seg_mma_kernel<C, false>), grid, dim3(SEG_THREADS), 0, s, w, (int)n, (int)k, rb, n * rb,
                       (int)ne, x, (int)rows, map, counts, (int)cap, y);
  return hipGetLastError();
}

}  // namespace

// K must be a multiple of 64 (whole units); other K take the GEMM kernel.
hipError_t launch_seg_mma(int codec, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k, int64_t row_bytes,
                          const half_t* x, int64_t rows, const uint32_t* map, const uint32_t* counts, int64_t cap,
                          void* y, int f16out, hipStream_t s) {
  switch (codec) {
    case Q4_0: return launch_seg_mma_c<Q4_0>(w, n_experts, n, k, row_bytes, x, rows, map, counts, cap, y, f16out, s);
    case Q8_0: return launch_seg_mma_c<Q8_0>(w, n_experts, n, k, row_bytes, x, rows, map, counts, cap, y, f16out, s);
    case Q2_K: return launch_seg_mma_c<Q2_K>(w, n_experts, n, k, row_bytes, x, rows, map, counts, cap, y, f16out, s);
    case Q3_K: return launch_seg_mma_c<Q3_K>(w, n_experts, n, k, row_bytes, x, rows, map, counts, cap, y, f16out, s);
    case Q4_K: return launch_seg_mma_c<Q4_K>(w, n_experts, n, k, row_bytes, x, rows, map, counts, cap, y, f16out, s);
    case Q5_K: return launch_seg_mma_c<Q5_K>(w, n_experts, n, k, row_bytes, x, rows, map, counts, cap, y, f16out, s);
    case Q4_1: return launch_seg_mma_c<Q4_1>(w, n_experts, n, k, row_bytes, x, rows, map, counts, cap, y, f16out, s);
    case Q5_0: return launch_seg_mma_c<Q5_0>(w, n_experts, n, k, row_bytes, x, rows, map, counts, cap, y, f16out, s);
    case Q5_1: return launch_seg_mma_c<Q5_1>(w, n_experts, n, k, row_bytes, x, rows, map, counts, cap, y, f16out, s);
    case Q6_K: return launch_seg_mma_c<Q6_K>(w, n_experts, n, k, row_bytes, x, rows, map, counts, cap, y, f16out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kq
