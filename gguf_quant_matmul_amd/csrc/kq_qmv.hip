// kq_qmv: decode-shaped quantized GEMV, y[m][n] = sum_k x[m][k] * W[n][k],
// 1 <= M <= 8 activation rows, float32 accumulation.
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
#include "kq_decode.h"

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
__host__ __device__ constexpr int xpad(int v) { return v + (v >> 6) * 8; }  // padded LDS offset (halves)

// ---------------------------------------------------------------------------
// Units.  load(row, u): issue the loads of unit u of a row.
// seg(u, t): row offset of the t-th 16-value segment of unit u.
// dot<M>(...): accumulate the unit's contribution into acc[0..M).
// ---------------------------------------------------------------------------

struct Xv {  // activation views for one chunk
  const half_t* xs;  // LDS [M][xpad(kc)]
  const float* xsum; // LDS [M][kc/16]
  int xstride, sstride, c0;
  __device__ __forceinline__ const uint32_t* pairs(int m, int off) const {  // off: row offset, multiple of 16
    return (const uint32_t*)(xs + m * xstride + xpad(off - c0));
  }
  __device__ __forceinline__ float sum16(int m, int off) const { return xsum[m * sstride + ((off - c0) >> 4)]; }
};

// sum over 16 values: (float16 pairs of codes) . (x pairs), 4 code dwords (p01, p23 per dword)
__device__ __forceinline__ float dot16(const uint32_t* cp /*8 pairs*/, const uint32_t* xp, float s) {
  const u32x4 a = *(const u32x4*)xp, b = *(const u32x4*)(xp + 4);
  s = dot2(cp[0], a.x, s); s = dot2(cp[1], a.y, s); s = dot2(cp[2], a.z, s); s = dot2(cp[3], a.w, s);
  s = dot2(cp[4], b.x, s); s = dot2(cp[5], b.y, s); s = dot2(cp[6], b.z, s); s = dot2(cp[7], b.w, s);
  return s;
}

// 4 code-byte dwords (16 codes) -> 8 float16 pairs (1024 + code)
__device__ __forceinline__ void pairs16(const uint32_t c[4], uint32_t p[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { p[2 * i] = pair01(c[i]); p[2 * i + 1] = pair23(c[i]); }
}

struct UnitQ4K {
  u32x4 h, q0, q1;
  __device__ __forceinline__ void load(const uint8_t* row, int u) {
    const uint8_t* blk = row + (u >> 2) * 144;
    h = ld_16B(blk);
    const uint8_t* qs = blk + 16 + 32 * (u & 3);
    q0 = ld_16B(qs);
    q1 = ld_16B(qs + 16);
  }
  template <int M>
  __device__ __forceinline__ void dot(int u, const Xv& xv, float acc[M]) const {
    const float d = f16_to_f32(h.x), dmin = f16_to_f32(h.x >> 16);
    const int j0 = 2 * (u & 3);
    uint32_t sc0, m0, sc1, m1;
    q4k_scale_min(h.y, h.z, h.w, j0, sc0, m0);
    q4k_scale_min(h.y, h.z, h.w, j0 + 1, sc1, m1);
    const float dsc0 = d * (float)sc0, dm0 = dmin * (float)m0;
    const float dsc1 = d * (float)sc1, dm1 = dmin * (float)m1;
    const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    uint32_t lo[16], hi[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t l = qw[i] & 0x0F0F0F0Fu, hh = (qw[i] >> 4) & 0x0F0F0F0Fu;
      lo[2 * i] = pair01(l); lo[2 * i + 1] = pair23(l);
      hi[2 * i] = pair01(hh); hi[2 * i + 1] = pair23(hh);
    }
    const int base = 64 * u;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float s0 = 0.f, s1 = 0.f;
      s0 = dot16(lo, xv.pairs(m, base), s0);
      s0 = dot16(lo + 8, xv.pairs(m, base + 16), s0);
      s1 = dot16(hi, xv.pairs(m, base + 32), s1);
      s1 = dot16(hi + 8, xv.pairs(m, base + 48), s1);
      const float4_t xs = *(const float4_t*)&xv.xsum[m * xv.sstride + ((base - xv.c0) >> 4)];
      const float x0 = xs.x + xs.y, x1 = xs.z + xs.w;
      acc[m] += dsc0 * (s0 - 1024.f * x0) - dm0 * x0 + dsc1 * (s1 - 1024.f * x1) - dm1 * x1;
    }
  }
};

// 16 bytes at a 2-byte aligned address: dwords loaded from the dword-aligned
// address below it, then shifted by (addr & 3) bytes.
struct Shift16 {
  u32x4 a;
  uint32_t b;
  __device__ __forceinline__ void load(const uint8_t* p, uint32_t sh) {
    const uint8_t* q = p - sh;
    a = ld_16B_a4(q);
    b = ld_u32(q + 16 - (sh ? 0 : 4));  // sh == 0: re-read the 4th dword, never past the 16 bytes
  }
  __device__ __forceinline__ void get(uint32_t sh, uint32_t o[4]) const {
    o[0] = alignbyte(a.y, a.x, sh);
    o[1] = alignbyte(a.z, a.y, sh);
    o[2] = alignbyte(a.w, a.z, sh);
    o[3] = alignbyte(b, a.w, sh);
  }
};

struct UnitQ6K {
  Shift16 qa, qb, qhh, scl;
  uint32_t dbits, sh;
  __device__ __forceinline__ void load(const uint8_t* row, int u) {
    const uint8_t* blk = row + (u >> 2) * 210;
    const int h = (u >> 1) & 1, half = u & 1;
    sh = (uint32_t)((uintptr_t)blk & 3);
    qa.load(blk + 64 * h + 16 * half, sh);
    qb.load(blk + 64 * h + 32 + 16 * half, sh);
    qhh.load(blk + 128 + 32 * h + 16 * half, sh);
    scl.load(blk + 192, sh);
    dbits = ld_u16(blk + 208);
  }
  template <int M>
  __device__ __forceinline__ void dot(int u, const Xv& xv, float acc[M]) const {
    const int h = (u >> 1) & 1, half = u & 1;
    uint32_t A[4], B[4], H[4], S[4];
    qa.get(sh, A); qb.get(sh, B); qhh.get(sh, H); scl.get(sh, S);
    const float d = f16_to_f32(dbits);
    const uint32_t slo = h ? S[2] : S[0], shi = h ? S[3] : S[1];
    float dsc[4];
    dsc[0] = d * (float)(int)(int8_t)(slo >> (8 * half));
    dsc[1] = d * (float)(int)(int8_t)(slo >> (8 * (half + 2)));
    dsc[2] = d * (float)(int)(int8_t)(shi >> (8 * half));
    dsc[3] = d * (float)(int)(int8_t)(shi >> (8 * (half + 2)));
    uint32_t c[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[0][i] = (A[i] & 0x0F0F0F0Fu) | ((H[i] << 4) & 0x30303030u);
      c[1][i] = (B[i] & 0x0F0F0F0Fu) | ((H[i] << 2) & 0x30303030u);
      c[2][i] = ((A[i] >> 4) & 0x0F0F0F0Fu) | (H[i] & 0x30303030u);
      c[3][i] = ((B[i] >> 4) & 0x0F0F0F0Fu) | ((H[i] >> 2) & 0x30303030u);
    }
    uint32_t p[4][8];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) pairs16(c[cc], p[cc]);
    const int base = 256 * (u >> 2) + 128 * h + 16 * half;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float t = 0.f;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int off = base + 32 * cc;
        const float s = dot16(p[cc], xv.pairs(m, off), 0.f);
        const float xs = xv.sum16(m, off);
        t += dsc[cc] * (s - 1056.f * xs);
      }
      acc[m] += t;
    }
  }
};

struct UnitQ8_0 {  // two 34-byte blocks, 68 bytes, dword aligned
  u32x4 r0, r1, r2, r3;
  uint32_t r4;
  __device__ __forceinline__ void load(const uint8_t* row, int u) {
    const uint8_t* p = row + 68 * u;
    r0 = ld_16B_a4(p); r1 = ld_16B_a4(p + 16); r2 = ld_16B_a4(p + 32); r3 = ld_16B_a4(p + 48);
    r4 = ld_u32(p + 64);
  }
  template <int M>
  __device__ __forceinline__ void dot(int u, const Xv& xv, float acc[M]) const {
    const uint32_t R[17] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w,
                            r2.x, r2.y, r2.z, r2.w, r3.x, r3.y, r3.z, r3.w, r4};
    const float d0 = f16_to_f32(R[0]), d1 = f16_to_f32(R[8] >> 16);
    uint32_t c0[8], c1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      c0[i] = alignbyte(R[i + 1], R[i], 2) ^ 0x80808080u;  // code + 128
      c1[i] = R[9 + i] ^ 0x80808080u;
    }
    uint32_t p0[16], p1[16];
    pairs16(c0, p0); pairs16(c0 + 4, p0 + 8);
    pairs16(c1, p1); pairs16(c1 + 4, p1 + 8);
    const int base = 64 * u;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float s0 = dot16(p0, xv.pairs(m, base), 0.f);
      s0 = dot16(p0 + 8, xv.pairs(m, base + 16), s0);
      float s1 = dot16(p1, xv.pairs(m, base + 32), 0.f);
      s1 = dot16(p1 + 8, xv.pairs(m, base + 48), s1);
      const float4_t xs = *(const float4_t*)&xv.xsum[m * xv.sstride + ((base - xv.c0) >> 4)];
      const float x0 = xs.x + xs.y, x1 = xs.z + xs.w;
      acc[m] += d0 * (s0 - 1152.f * x0) + d1 * (s1 - 1152.f * x1);
    }
  }
};

struct UnitQ4_0 {  // two 18-byte blocks, 36 bytes, dword aligned
  u32x4 r0, r1;
  uint32_t r2;
  __device__ __forceinline__ void load(const uint8_t* row, int u) {
    const uint8_t* p = row + 36 * u;
    r0 = ld_16B_a4(p); r1 = ld_16B_a4(p + 16);
    r2 = ld_u32(p + 32);
  }
  template <int M>
  __device__ __forceinline__ void dot(int u, const Xv& xv, float acc[M]) const {
    const uint32_t R[9] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w, r2};
    const float d0 = f16_to_f32(R[0]), d1 = f16_to_f32(R[4] >> 16);
    uint32_t q0[4], q1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { q0[i] = alignbyte(R[i + 1], R[i], 2); q1[i] = R[5 + i]; }
    uint32_t l0[4], h0[4], l1[4], h1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      l0[i] = q0[i] & 0x0F0F0F0Fu; h0[i] = (q0[i] >> 4) & 0x0F0F0F0Fu;
      l1[i] = q1[i] & 0x0F0F0F0Fu; h1[i] = (q1[i] >> 4) & 0x0F0F0F0Fu;
    }
    uint32_t pl0[8], ph0[8], pl1[8], ph1[8];
    pairs16(l0, pl0); pairs16(h0, ph0); pairs16(l1, pl1); pairs16(h1, ph1);
    const int base = 64 * u;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float s0 = dot16(pl0, xv.pairs(m, base), 0.f);
      s0 = dot16(ph0, xv.pairs(m, base + 16), s0);
      float s1 = dot16(pl1, xv.pairs(m, base + 32), 0.f);
      s1 = dot16(ph1, xv.pairs(m, base + 48), s1);
      const float4_t xs = *(const float4_t*)&xv.xsum[m * xv.sstride + ((base - xv.c0) >> 4)];
      const float x0 = xs.x + xs.y, x1 = xs.z + xs.w;
      acc[m] += d0 * (s0 - 1032.f * x0) + d1 * (s1 - 1032.f * x1);
    }
  }
};

template <int C> struct UnitOf;
template <> struct UnitOf<Q4_K> { typedef UnitQ4K T; };
template <> struct UnitOf<Q6_K> { typedef UnitQ6K T; };
template <> struct UnitOf<Q8_0> { typedef UnitQ8_0 T; };
template <> struct UnitOf<Q4_0> { typedef UnitQ4_0 T; };

// Sum over the 16 lanes of a DPP row (every lane receives the total).
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));  // row_ror:8
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));  // row_ror:4
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));  // row_ror:2
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));  // row_ror:1
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

template <int C, int M, int LPR, bool F16>
__global__ __launch_bounds__(QMV_THREADS) void qmv_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                          int64_t row_bytes, const half_t* __restrict__ x,
                                                          void* __restrict__ y) {
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
  const int row = (blockIdx.x * (QMV_THREADS / 64) + wave) * ROWS_PER_WAVE + rslot;
  const bool row_ok = row < n;
  const uint8_t* wrow = w + (int64_t)(row_ok ? row : 0) * row_bytes;

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;

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
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      int c = tid + i * QMV_THREADS;
      c = c < xpieces ? c : xpieces - 1;
      const int m = c / (kc / 8), v = (c % (kc / 8)) * 8;
      xr[i] = *(const u32x4*)(x + (int64_t)m * k + c0 + v);
    }
    Unit cur[UNROLL];
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      const int u = ub + uslot + LANES_PER_ROW * j;
      cur[j].load(wrow, u < ue ? u : ue - 1);
    }
    if (c0) __syncthreads();  // previous chunk done with LDS
    // Stage x and its 16-value sums in one pass: pieces 2g and 2g + 1 (8
    // values each) sit in adjacent lanes, so each lane sums its own 8 values
    // and adds its neighbour's with a DPP quad permutation [1, 0, 3, 2].
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = tid + i * QMV_THREADS;
      const uint32_t one2 = 0x3C003C00u;  // (1.0, 1.0)
      float s = 0.f;
      s = dot2(xr[i].x, one2, s); s = dot2(xr[i].y, one2, s); s = dot2(xr[i].z, one2, s); s = dot2(xr[i].w, one2, s);
      s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, false));
      if (c < xpieces) {
        const int m = c / (kc / 8), v = (c % (kc / 8)) * 8;
        *(u32x4*)(xs + m * xstride + xpad(v)) = xr[i];
        if ((c & 1) == 0) xsum[m * sstride + (v >> 4)] = s;
      }
    }
    __syncthreads();
    const Xv xv{xs, xsum, xstride, sstride, c0};
    for (int g = 0; g < ngroups; ++g) {
      const int u0 = ub + uslot + LANES_PER_ROW * UNROLL * g;
      Unit nxt[UNROLL];
      if (g + 1 < ngroups) {  // uniform across the block
#pragma unroll
        for (int j = 0; j < UNROLL; ++j) {
          const int u = u0 + LANES_PER_ROW * (UNROLL + j);
          nxt[j].load(wrow, u < ue ? u : ue - 1);
        }
      }
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        const int u = u0 + LANES_PER_ROW * j;
        if (row_ok && u < ue) cur[j].template dot<M>(u, xv, acc);
      }
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) cur[j] = nxt[j];
    }
  }

#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = lanes_sum<LPR>(acc[m]);
  if (row_ok && uslot < M) {
    float v = acc[0];
#pragma unroll
    for (int m = 1; m < M; ++m)
      if (uslot == m) v = acc[m];
    if (F16)
      ((half_t*)y)[(int64_t)uslot * n + row] = (half_t)v;
    else
      ((float*)y)[(int64_t)uslot * n + row] = v;
  }
}

// Generic GEMV for shapes the unit kernels do not take (q8_0 / q4_0 with an
// odd number of blocks per row): one wave per row, 8 values per lane step.
template <int C, bool F16>
__global__ __launch_bounds__(256) void qmv_generic_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                          int64_t row_bytes, const half_t* __restrict__ x, int m,
                                                          void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint8_t* wrow = w + (int64_t)row * row_bytes;
  for (int g = lane; g < k / 8; g += 64) {
    float v[8];
    decode8<C>(wrow, (int64_t)g * 8, v);
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
      if (mm < m) {
        const half8_t xv = *(const half8_t*)(x + (int64_t)mm * k + 8 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[mm] += v[i] * (float)xv[i];
      }
    }
  }
#pragma unroll
  for (int mm = 0; mm < 8; ++mm) {
    float s = acc[mm];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0 && mm < m) {
      if (F16)
        ((half_t*)y)[(int64_t)mm * n + row] = (half_t)s;
      else
        ((float*)y)[(int64_t)mm * n + row] = s;
    }
  }
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

// One wave per row (64 lanes, one 64-value unit each at K = 4096) for one
// activation row and a matrix with few rows: four times the workgroups and a
// quarter of the serial work per lane.  Otherwise 16 lanes per row, so the
// activation staging is shared by 16 rows per workgroup.
template <int C, int M>
hipError_t launch_m(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, void* y, int f16,
                    hipStream_t s) {
  if (M == 1 && n <= 32768) return launch_ml<C, M, 64>(w, n, k, rb, x, y, f16, s);
  return launch_ml<C, M, 16>(w, n, k, rb, x, y, f16, s);
}

template <int C>
hipError_t launch_c(const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int m, void* y, int f16,
                    hipStream_t s) {
  // The unit kernels need whole 64-value units per row (q8_0 / q4_0: an even block count).
  if (k % 64 != 0) {
    const dim3 grid((unsigned)((n + 3) / 4));
    if (f16)
      hipLaunchKernelGGL((qmv_generic_kernel<C, true>), grid, dim3(256), 0, s, w, (int)n, (int)k, rb, x, m, y);
    else
      hipLaunchKernelGGL((qmv_generic_kernel<C, false>), grid, dim3(256), 0, s, w, (int)n, (int)k, rb, x, m, y);
    return hipGetLastError();
  }
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
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qmv(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int m, void* y,
                      int f16, hipStream_t s) {
  switch (codec) {
    case Q4_0: return launch_c<Q4_0>(w, n, k, rb, x, m, y, f16, s);
    case Q8_0: return launch_c<Q8_0>(w, n, k, rb, x, m, y, f16, s);
    case Q4_K: return launch_c<Q4_K>(w, n, k, rb, x, m, y, f16, s);
    case Q6_K: return launch_c<Q6_K>(w, n, k, rb, x, m, y, f16, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kq
