// kq_qmm and kq_gather_qmm_seg: quantized GEMM on gfx950 float16 matrix cores.
//
// mlx-kquant bindings.cpp page: quantized_matmul docstring (y = x @ dequant(w)
// transposed, w [N, K]); gather_qmm_seg docstring (expert-sorted rows walked
// tile by tile from a (expert, row_start, num_rows) map with <= 64 rows per
// tile, dead rows of a partial tile skipped, uncovered rows unwritten).
//
// Design.
//  * Workgroup tile BM x BN of the output, K walked 64 values (one "unit") at
//    a time.  Per step the workgroup stages the x tile (BM x 64 float16) and
//    DECODES the weight tile (BN rows x 64 values) straight from wire bytes
//    into LDS as float16 -- each thread decodes half a unit (32 values) with
//    packed float16 math -- then 4 waves run v_mfma_f32_32x32x16_f16 on it
//    with float32 accumulators.
//  * Within a 64-value step the order of k does not matter to the
//    contraction, only that x and W agree: a q6_K unit's four 16-value
//    segments are not contiguous in K, so x is gathered with the same
//    segment map the decode writes with.
//  * Weights are decoded once per BM rows of x; activations once per BN
//    weight rows.
//  * The segment variant takes one tile per workgroup row of the grid: it
//    reads (expert, row_start, num_rows) and the valid-tile count on the
//    device, so no host sync sits between the tile map and this kernel.
#include "kq_decode.h"

namespace kq {
namespace {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // halves; 144-byte rows spread 16-byte reads over the banks

// Row offset of segment t (16 values) of unit u.
template <int C>
__device__ __forceinline__ int seg_off(int u, int t) {
  if (C == Q6_K) return 256 * (u >> 2) + 128 * ((u >> 1) & 1) + 32 * t + 16 * (u & 1);
  return 64 * u + 16 * t;
}

__device__ __forceinline__ half2_t h2(half_t a) { return half2_t{a, a}; }

// Decode half of unit u of one weight row into 32 float16 values.  Writes
// values to dst[16 * t + i] for its two segments t.
template <int C> struct HalfUnit;

template <> struct HalfUnit<Q4_K> {
  // half hh: qs bytes 16*hh..16*hh+15 of the pair = positions l in [16hh, 16hh+16)
  // of sub-blocks j0 = 2P (low nibbles, segment hh) and j1 = 2P+1 (high, segment 2+hh).
  // Each weight is the exact float32 value (d*sc)*q - dmin*m (one FMA, inputs
  // exact) rounded once to float16: rounding d*sc or dmin*m to float16 first
  // would put one correlated error on all 32 weights of a sub-block.
  __device__ __forceinline__ static void run(const uint8_t* row, int u, int hh, half_t* dst) {
    const uint8_t* blk = row + (u >> 2) * 144;
    const u32x4 h = ld_16B(blk);
    const u32x4 q = ld_16B(blk + 16 + 32 * (u & 3) + 16 * hh);
    const float d = f16_to_f32(h.x), dmin = f16_to_f32(h.x >> 16);
    uint32_t sc0, m0, sc1, m1;
    q4k_scale_min(h.y, h.z, h.w, 2 * (u & 3), sc0, m0);
    q4k_scale_min(h.y, h.z, h.w, 2 * (u & 3) + 1, sc1, m1);
    const float s0 = d * (float)sc0, n0 = -(dmin * (float)m0);
    const float s1 = d * (float)sc1, n1 = -(dmin * (float)m1);
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t l = qw[i] & 0x0F0F0F0Fu, t = (qw[i] >> 4) & 0x0F0F0F0Fu;
      lo[2 * i] = pack_h2(fmaf(s0, byte_f32<0>(l), n0), fmaf(s0, byte_f32<1>(l), n0));
      lo[2 * i + 1] = pack_h2(fmaf(s0, byte_f32<2>(l), n0), fmaf(s0, byte_f32<3>(l), n0));
      hi[2 * i] = pack_h2(fmaf(s1, byte_f32<0>(t), n1), fmaf(s1, byte_f32<1>(t), n1));
      hi[2 * i + 1] = pack_h2(fmaf(s1, byte_f32<2>(t), n1), fmaf(s1, byte_f32<3>(t), n1));
    }
    *(u32x4*)(dst + 16 * hh) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    *(u32x4*)(dst + 16 * hh + 8) = u32x4{lo[4], lo[5], lo[6], lo[7]};
    *(u32x4*)(dst + 16 * (2 + hh)) = u32x4{hi[0], hi[1], hi[2], hi[3]};
    *(u32x4*)(dst + 16 * (2 + hh) + 8) = u32x4{hi[4], hi[5], hi[6], hi[7]};
  }
};

// 16 bytes at a 2-byte-aligned address (see kq_qmv.hip: never reads past them).
__device__ __forceinline__ void ld16_a2(const uint8_t* p, uint32_t sh, uint32_t o[4]) {
  const uint8_t* q = p - sh;
  const u32x4 a = ld_16B_a4(q);
  const uint32_t b = ld_u32(q + 16 - (sh ? 0 : 4));
  o[0] = alignbyte(a.y, a.x, sh);
  o[1] = alignbyte(a.z, a.y, sh);
  o[2] = alignbyte(a.w, a.z, sh);
  o[3] = alignbyte(b, a.w, sh);
}

template <> struct HalfUnit<Q6_K> {
  // unit u = (superblock s, h, half); half hh takes c = hh (low nibbles) and
  // c = hh + 2 (high nibbles) of ql[64h + 32hh + 16half + i].
  __device__ __forceinline__ static void run(const uint8_t* row, int u, int hh, half_t* dst) {
    const uint8_t* blk = row + (u >> 2) * 210;
    const int h = (u >> 1) & 1, half = u & 1;
    const uint32_t sh = (uint32_t)((uintptr_t)blk & 3);
    uint32_t Q[4], H[4], S[4];
    ld16_a2(blk + 64 * h + 32 * hh + 16 * half, sh, Q);
    ld16_a2(blk + 128 + 32 * h + 16 * half, sh, H);
    ld16_a2(blk + 192, sh, S);
    const float d = f16_to_f32(ld_u16(blk + 208));  // exact in float16 again below
    // scales[8h + 2c + half]: c = hh in dword 2h (byte half + 2hh), c = hh+2 in dword 2h+1
    const uint32_t slo = h ? S[2] : S[0], shi = h ? S[3] : S[1];
    const int bsh = 8 * (half + 2 * hh);
    // value = ((q - 32) * sc) * d: (q - 32) * sc is an integer of magnitude <= 4096
    // (exact in float16 up to 2048), so each weight is rounded once, by itself.
    const half2_t sa = h2((half_t)(float)(int)(int8_t)(slo >> bsh));
    const half2_t sb = h2((half_t)(float)(int)(int8_t)(shi >> bsh));
    const half2_t dd = h2((half_t)d);
    const half2_t k1056 = h2((half_t)1056.f);
    const int hs = 2 * hh;
    uint32_t a[8], b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ca = (Q[i] & 0x0F0F0F0Fu) | (((H[i] >> hs) << 4) & 0x30303030u);
      const uint32_t cb = ((Q[i] >> 4) & 0x0F0F0F0Fu) | (((H[i] >> (hs + 4)) << 4) & 0x30303030u);
      a[2 * i] = as_u32(((as_h2(pair01(ca)) - k1056) * sa) * dd);
      a[2 * i + 1] = as_u32(((as_h2(pair23(ca)) - k1056) * sa) * dd);
      b[2 * i] = as_u32(((as_h2(pair01(cb)) - k1056) * sb) * dd);
      b[2 * i + 1] = as_u32(((as_h2(pair23(cb)) - k1056) * sb) * dd);
    }
    *(u32x4*)(dst + 16 * hh) = u32x4{a[0], a[1], a[2], a[3]};
    *(u32x4*)(dst + 16 * hh + 8) = u32x4{a[4], a[5], a[6], a[7]};
    *(u32x4*)(dst + 16 * (hh + 2)) = u32x4{b[0], b[1], b[2], b[3]};
    *(u32x4*)(dst + 16 * (hh + 2) + 8) = u32x4{b[4], b[5], b[6], b[7]};
  }
};

template <> struct HalfUnit<Q8_0> {
  // unit u = two blocks at 68u; half hh = block hh (34 bytes) -> segments 2hh, 2hh+1.
  __device__ __forceinline__ static void run(const uint8_t* row, int u, int hh, half_t* dst) {
    const uint8_t* p = row + 68 * u + 34 * hh;
    const uint32_t sh = (uint32_t)((uintptr_t)p & 3);
    const uint8_t* a = p - sh;
    const u32x4 r0 = ld_16B_a4(a), r1 = ld_16B_a4(a + 16);
    const uint32_t r8 = ld_u32(a + 32);
    const uint32_t R[9] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w, r8};
    const half2_t d = h2(__builtin_bit_cast(half_t, (uint16_t)(sh ? (R[0] >> 16) : (R[0] & 0xFFFFu))));
    const half2_t k1152 = h2((half_t)1152.f);
    uint32_t o[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = (sh ? R[i + 1] : alignbyte(R[i + 1], R[i], 2)) ^ 0x80808080u;
      o[2 * i] = as_u32((as_h2(pair01(c)) - k1152) * d);
      o[2 * i + 1] = as_u32((as_h2(pair23(c)) - k1152) * d);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(dst + 32 * hh + 8 * i) = u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
  }
};

template <> struct HalfUnit<Q4_0> {
  // unit u = two blocks at 36u; half hh = block hh (18 bytes): low nibbles are
  // values 0..15 (segment 2hh), high nibbles 16..31 (segment 2hh+1).
  __device__ __forceinline__ static void run(const uint8_t* row, int u, int hh, half_t* dst) {
    const uint8_t* p = row + 36 * u + 18 * hh;
    const uint32_t sh = (uint32_t)((uintptr_t)p & 3);
    const uint8_t* a = p - sh;
    const u32x4 r0 = ld_16B_a4(a);
    const uint32_t r4 = ld_u32(a + 16);
    const uint32_t R[5] = {r0.x, r0.y, r0.z, r0.w, r4};
    const half2_t d = h2(__builtin_bit_cast(half_t, (uint16_t)(sh ? (R[0] >> 16) : (R[0] & 0xFFFFu))));
    const half2_t k1032 = h2((half_t)1032.f);
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t q = sh ? R[i + 1] : alignbyte(R[i + 1], R[i], 2);
      const uint32_t l = q & 0x0F0F0F0Fu, t = (q >> 4) & 0x0F0F0F0Fu;
      lo[2 * i] = as_u32((as_h2(pair01(l)) - k1032) * d);
      lo[2 * i + 1] = as_u32((as_h2(pair23(l)) - k1032) * d);
      hi[2 * i] = as_u32((as_h2(pair01(t)) - k1032) * d);
      hi[2 * i + 1] = as_u32((as_h2(pair23(t)) - k1032) * d);
    }
    *(u32x4*)(dst + 32 * hh) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    *(u32x4*)(dst + 32 * hh + 8) = u32x4{lo[4], lo[5], lo[6], lo[7]};
    *(u32x4*)(dst + 32 * hh + 16) = u32x4{hi[0], hi[1], hi[2], hi[3]};
    *(u32x4*)(dst + 32 * hh + 24) = u32x4{hi[4], hi[5], hi[6], hi[7]};
  }
};

template <int C, int BM, int BN, int WM, int WN, bool SEG, bool F16>
__global__ __launch_bounds__(256) void qmm_kernel(const uint8_t* __restrict__ w, int n, int k, int64_t row_bytes,
                                                  int64_t expert_stride, int n_experts,
                                                  const half_t* __restrict__ x, int m_total,
                                                  const uint32_t* __restrict__ map, const uint32_t* __restrict__ counts,
                                                  void* __restrict__ y) {
  static_assert(WM * WN == 4, "4 waves");
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  __shared__ __attribute__((aligned(16))) half_t As[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) half_t Bs[BN * LDS_STRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = (n + BN - 1) / BN;
  const int by = (int)(blockIdx.x / nb);
  const int n0 = (int)(blockIdx.x % nb) * BN;
  int m0, mrows;
  const uint8_t* wbase = w;
  if (SEG) {
    const int tile = by;
    if (tile >= (int)counts[0]) return;
    const uint32_t* mt = map + 3 * (size_t)tile;
    const uint32_t e = mt[0], rs = mt[1], nr = mt[2];
    if (e >= (uint32_t)n_experts || nr == 0 || nr > 64 || rs >= (uint32_t)m_total || nr > (uint32_t)m_total - rs)
      return;
    m0 = (int)rs;
    mrows = (int)nr;
    wbase = w + (int64_t)e * expert_stride;
  } else {
    m0 = by * BM;
    mrows = min(BM, m_total - m0);
  }

  const int wm = wave / WN, wn = wave % WN;
  const int wr0 = wm * (BM / WM), wc0 = wn * (BN / WN);
  const bool wave_live = wr0 < mrows;  // dead row fragments of a partial tile skip the MFMAs

  float16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int units = k / BK;
  for (int u = 0; u < units; ++u) {
    // x tile: BM rows x 4 segments x 2 halves of 8 values
    for (int c = tid; c < BM * 8; c += 256) {
      const int r = c >> 3, part = c & 7, t = part >> 1, hf = part & 1;
      u32x4 v = {0, 0, 0, 0};
      if (r < mrows) v = *(const u32x4*)(x + (int64_t)(m0 + r) * k + seg_off<C>(u, t) + 8 * hf);
      *(u32x4*)(As + r * LDS_STRIDE + 16 * t + 8 * hf) = v;
    }
    // weight tile: BN rows x 2 half-units
    for (int c = tid; c < BN * 2; c += 256) {
      const int r = c >> 1, hh = c & 1;
      half_t* dst = Bs + r * LDS_STRIDE;
      if (n0 + r < n) {
        HalfUnit<C>::run(wbase + (int64_t)(n0 + r) * row_bytes, u, hh, dst);
      } else {
        const u32x4 z = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4*)(dst + 32 * hh + 8 * i) = z;
      }
    }
    __syncthreads();
    if (wave_live) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        half8_t a[TM], b[TN];
        const int kk = 16 * ks + 8 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = *(const half8_t*)(As + (wr0 + 32 * i + (lane & 31)) * LDS_STRIDE + kk);
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = *(const half8_t*)(Bs + (wc0 + 32 * j + (lane & 31)) * LDS_STRIDE + kk);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  if (!wave_live) return;
  // 32x32 accumulator layout: lane holds column (lane & 31); register r holds
  // row 8*(r/4) + 4*(lane/32) + (r%4).
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wc0 + 32 * j + (lane & 31);
      if (col >= n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wr0 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < mrows) {
          const int64_t o = (int64_t)(m0 + row) * n + col;
          if (F16)
            ((half_t*)y)[o] = (half_t)acc[i][j][r];
          else
            ((float*)y)[o] = acc[i][j][r];
        }
      }
    }
}

template <int C, bool SEG, int BM, int BN, int WM, int WN>
hipError_t launch_t(const uint8_t* w, int64_t n, int64_t k, int64_t rb, int64_t estride, int64_t ne, const half_t* x,
                    int64_t m, const uint32_t* map, const uint32_t* counts, int64_t gy, void* y, int f16, hipStream_t s) {
  const dim3 grid((unsigned)(((n + BN - 1) / BN) * gy));
  if (f16)
    hipLaunchKernelGGL((qmm_kernel<C, BM, BN, WM, WN, SEG, true>), grid, dim3(256), 0, s, w, (int)n, (int)k, rb,
                       estride, (int)ne, x, (int)m, map, counts, y);
  else
    hipLaunchKernelGGL((qmm_kernel<C, BM, BN, WM, WN, SEG, false>), grid, dim3(256), 0, s, w, (int)n, (int)k, rb,
                       estride, (int)ne, x, (int)m, map, counts, y);
  return hipGetLastError();
}

template <int C>
hipError_t launch_dense(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int64_t m, void* y,
                        int f16, hipStream_t s) {
  return launch_t<C, false, 128, 128, 2, 2>(w, n, k, rb, 0, 1, x, m, nullptr, nullptr, (m + 127) / 128, y, f16, s);
}

template <int C>
hipError_t launch_seg(const uint8_t* w, int64_t ne, int64_t n, int64_t k, int64_t rb, const half_t* x, int64_t rows,
                      const uint32_t* map, const uint32_t* counts, int64_t cap, void* y, int f16, hipStream_t s) {
  return launch_t<C, true, 64, 128, 2, 2>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
}

// Generic fallback for K with an odd number of 32-value blocks (q8_0 / q4_0):
// one float32 dot per output, 64 lanes over K.  Correct, not fast.
template <int C, bool SEG, bool F16>
__global__ __launch_bounds__(256) void qmm_generic_kernel(const uint8_t* __restrict__ w, int n, int k, int64_t rb,
                                                          int64_t estride, int n_experts, const half_t* __restrict__ x,
                                                          int m_total, const uint32_t* __restrict__ map,
                                                          const uint32_t* __restrict__ counts, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int nb = (n + 3) / 4;
  const int by = (int)(blockIdx.x / nb);
  const int col = (int)(blockIdx.x % nb) * 4 + (threadIdx.x >> 6);
  if (col >= n) return;
  int r0, r1;
  const uint8_t* wb = w;
  if (SEG) {
    const int tile = by;
    if (tile >= (int)counts[0]) return;
    const uint32_t* mt = map + 3 * (size_t)tile;
    const uint32_t e = mt[0], rs = mt[1], nr = mt[2];
    if (e >= (uint32_t)n_experts || nr == 0 || nr > 64 || rs >= (uint32_t)m_total || nr > (uint32_t)m_total - rs)
      return;
    r0 = (int)rs; r1 = (int)(rs + nr);
    wb = w + (int64_t)e * estride;
  } else {
    r0 = by * 64;
    r1 = min(m_total, r0 + 64);
  }
  const uint8_t* wrow = wb + (int64_t)col * rb;
  for (int r = r0; r < r1; ++r) {
    float acc = 0.f;
    for (int g = lane; g < k / 8; g += 64) {
      float v[8];
      decode8<C>(wrow, (int64_t)g * 8, v);
      const half8_t xv = *(const half8_t*)(x + (int64_t)r * k + 8 * g);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += v[i] * (float)xv[i];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) {
      if (F16)
        ((half_t*)y)[(int64_t)r * n + col] = (half_t)acc;
      else
        ((float*)y)[(int64_t)r * n + col] = acc;
    }
  }
}

template <int C, bool SEG>
hipError_t launch_generic(const uint8_t* w, int64_t n, int64_t k, int64_t rb, int64_t estride, int64_t ne,
                          const half_t* x, int64_t m, const uint32_t* map, const uint32_t* counts, int64_t gy, void* y,
                          int f16, hipStream_t s) {
  const dim3 grid((unsigned)(((n + 3) / 4) * gy));
  if (f16)
    hipLaunchKernelGGL((qmm_generic_kernel<C, SEG, true>), grid, dim3(256), 0, s, w, (int)n, (int)k, rb, estride,
                       (int)ne, x, (int)m, map, counts, y);
  else
    hipLaunchKernelGGL((qmm_generic_kernel<C, SEG, false>), grid, dim3(256), 0, s, w, (int)n, (int)k, rb, estride,
                       (int)ne, x, (int)m, map, counts, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qmm(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int64_t m,
                      void* y, int f16, hipStream_t s) {
  if (k % 64 != 0) {
    const int64_t gy = (m + 63) / 64;
    switch (codec) {
      case Q4_0: return launch_generic<Q4_0, false>(w, n, k, rb, 0, 1, x, m, nullptr, nullptr, gy, y, f16, s);
      case Q8_0: return launch_generic<Q8_0, false>(w, n, k, rb, 0, 1, x, m, nullptr, nullptr, gy, y, f16, s);
    }
    return hipErrorInvalidValue;
  }
  switch (codec) {
    case Q4_0: return launch_dense<Q4_0>(w, n, k, rb, x, m, y, f16, s);
    case Q8_0: return launch_dense<Q8_0>(w, n, k, rb, x, m, y, f16, s);
    case Q4_K: return launch_dense<Q4_K>(w, n, k, rb, x, m, y, f16, s);
    case Q6_K: return launch_dense<Q6_K>(w, n, k, rb, x, m, y, f16, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gather_qmm_seg(int codec, const uint8_t* w, int64_t ne, int64_t n, int64_t k, int64_t rb,
                                 const half_t* x, int64_t rows, const uint32_t* map, const uint32_t* counts,
                                 int64_t cap, void* y, int f16, hipStream_t s) {
  if (k % 64 != 0) {
    switch (codec) {
      case Q4_0: return launch_generic<Q4_0, true>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
      case Q8_0: return launch_generic<Q8_0, true>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
    }
    return hipErrorInvalidValue;
  }
  switch (codec) {
    case Q4_0: return launch_seg<Q4_0>(w, ne, n, k, rb, x, rows, map, counts, cap, y, f16, s);
    case Q8_0: return launch_seg<Q8_0>(w, ne, n, k, rb, x, rows, map, counts, cap, y, f16, s);
    case Q4_K: return launch_seg<Q4_K>(w, ne, n, k, rb, x, rows, map, counts, cap, y, f16, s);
    case Q6_K: return launch_seg<Q6_K>(w, ne, n, k, rb, x, rows, map, counts, cap, y, f16, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kq
