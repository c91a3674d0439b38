// kq_gather_qmm_seg for q4_K on the matrix cores with EXACT integer weight
// operands: no weight is rounded.
//
// mlx-kquant bindings.cpp page, gather_qmm_seg docstring: expert-sorted rows
// walked tile by tile from a (expert, row_start, num_rows) map of at most 64
// rows per tile; rows no tile covers stay unwritten.  q4_K geometry: the
// mlx-kquant README codec table (256-value superblocks, 8 sub-blocks of 32
// with 6-bit scale and min, float16 d and dmin); byte layout GGUF's.
//
// A q4_K weight is w = d sc_j q - dmin m_j (sub-block j of a superblock).  The
// product with x splits into
//   sum_k x_k w_k = d * sum_k x_k (sc_j q_k)  -  sum_j (dmin m_j) X_j,
// X_j the sum of x over sub-block j.  sc_j q_k is an integer below 946, so it
// is an exact float16: the main matrix-core product runs on these integers
// (one v_pk_fma_f16 per two weights turns the code's 1024 + q, built by a byte
// permute, into sc q exactly), accumulated in float32 over one superblock and
// then scaled by d.  That costs about 10 VALU per 8 weights against 18 for a
// float16 weight d sc q - dmin m rounded once.  The min term is a small
// product of the sub-block sums X with dmin m_j: one bfloat16 matrix-core
// product (K = 16) every two superblocks, each operand split into two
// bfloat16 terms (16 bits), which keeps float32's exponent range for any
// activation.
//
// Layout (as the float16-weight segment kernel in kq_seg.hip): a workgroup
// takes one tile and 128 weight rows of its expert; each of its four waves
// owns 32 rows (two groups of 16); lane l takes row l & 15 of a group and 8
// values of unit (superblock, sub-block pair l >> 4) per MFMA, so one MFMA's 32
// K values are the four sub-block pairs of one superblock at one offset, and
// all of them share the superblock's d.  Activations are staged in LDS one
// superblock (256 values) per chunk, double-buffered; the sub-block sums are
// formed while staging.
//
// LDS placement of the activation rows.  Measured on gfx950 with a probe of
// lane address patterns against SQ_LDS_BANK_CONFLICT: a 16-byte read of a
// wave is served in 32-lane halves over sixteen 16-byte bank slots
// (address / 16 mod 16); two lanes of a half that hit one slot at different
// addresses conflict unless they are exactly 16 lanes apart.  A fragment read
// has lane (r, cu) take 16-byte chunk 8 cu + S of row 16 i + r, so chunk c of
// row r is stored at swap34(c) ^ (r & 15) (bits 3 and 4 of c exchanged): lanes
// 16 apart then share a slot and each 16-lane group covers all sixteen.  The
// staging lane that writes physical chunk pc loads logical chunk
// swap34(pc ^ (r & 15)), so the writes are contiguous.
//
// A tile of 64 rows followed in the map by a tail of at most 16 rows of the
// same expert (contiguous rows) is worked as one 80-row tile: otherwise the
// tail's workgroups decode every weight of the expert again for a handful of
// rows.  The two tiles' workgroups then take 64-row weight blocks (one 16-row
// group per wave) against five activation groups, the activation chunk
// single-buffered so the kernel's LDS stays within two workgroups per CU.
#include <type_traits>

#include "kq_units.h"

namespace kq {
namespace {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));  // four bfloat16 bit patterns

constexpr int SX_THREADS = 256;            // four waves
constexpr int SX_RG = 2;                   // 16-row weight groups per wave
constexpr int SX_BN = 4 * 16 * SX_RG;      // weight rows per workgroup (128)
constexpr int SX_KC = 256;                 // K values per chunk: one superblock
constexpr int SX_XBUF = 64 * SX_KC;        // halves per activation chunk buffer (64 rows)
constexpr int SX_WROW = 16;                // sub-block sums per row per window: 8 sub-blocks x 2 superblocks
constexpr int SX_WBUF = 64 * 2 * SX_WROW;  // bfloat16 per window buffer: [row][hi, lo][16]
constexpr int SX_LDS = 2 * SX_XBUF * 2 + 2 * SX_WBUF * 2;  // bytes: both paths' buffers fit
constexpr int SX_MERGE_MAX = 16;           // largest tail merged into the full tile before it
constexpr int SX_NXCD = 8;

template <int N, typename F>
__device__ __forceinline__ void sx_for(F&& f) {
  if constexpr (N > 0) {
    sx_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// LDS (address space 3) views: a 32-bit LDS byte address and the 16-byte
// fragment it points at.
typedef __attribute__((address_space(3))) const half8_t lds_half8_t;
__device__ __forceinline__ uint32_t lds_addr(const half_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const half_t*)p;
}

// Bits 3 and 4 of a 16-byte chunk index exchanged.
__device__ __forceinline__ int sx_swap34(int c) { return (c & ~24) | ((c & 8) << 1) | ((c & 16) >> 1); }

// A window buffer row is eight 8-byte slots: the hi sums of sub-block pairs
// 0..3, then the lo sums.  Slot c of row r sits at c ^ ((r >> 1) & 7), so the
// 8-byte reads of rows 0..15 at one slot (16 lanes), or at two neighbouring
// slots (32 lanes), fall on distinct banks; unswizzled, rows r and r + 4
// share banks.  Returns the index of the slot's first bfloat16.  A lo slot
// (c + 4) is its hi slot's index with bit 4 flipped, and rows 8 apart differ
// by 256 and by that same flip, so the kernel forms every address from one
// base register and immediate offsets.
__device__ __forceinline__ int sx_wslot(int row, int c) { return 4 * (8 * row + (c ^ ((row >> 1) & 7))); }

// float32 v -> (hi, lo) bfloat16 bit patterns with v = hi + lo + O(2^-16 |v|):
// hi is v truncated to 8 significant bits, lo the (exact) remainder truncated.
__device__ __forceinline__ void bf16_split(float v, uint32_t& hi, uint32_t& lo) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const float r = v - __builtin_bit_cast(float, b & 0xFFFF0000u);
  hi = b;
  lo = __builtin_bit_cast(uint32_t, r);
}
// the high halves of two dwords as one dword: (a >> 16) | (b & 0xFFFF0000)
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) { return perm(b, a, 0x07060302u); }

// Per-superblock constants of one 16-row weight group for this lane (its row
// r, its sub-block pair cu): the float16 pairs that turn 1024 + q into sc q for
// the low-nibble (sub-block 2cu) and high-nibble (2cu + 1, codes used as 16 q)
// halves, the scale d, and -dmin m of both sub-blocks as bfloat16 hi / lo.
struct SxConst {
  half2_t k1, k2;  // (sc0, sc1 / 16), (-1024 sc0, -64 sc1): exact float16
  float d;
  uint32_t bh, bl;  // bfloat16 pairs (sub-block 2cu, 2cu + 1) of -dmin m
  SxConst() = default;
  __device__ __forceinline__ SxConst(const UnitQ4K& un, int cu) {
    uint32_t sc0, m0, sc1, m1;
    q4k_scale_min_pair(un.h.y, un.h.z, un.h.w, cu, sc0, m0, sc1, m1);
    const half2_t s = half2_t{(half_t)(float)sc0, (half_t)(float)sc1};
    k1 = s * half2_t{(half_t)1.0f, (half_t)0.0625f};
    k2 = s * half2_t{(half_t)-1024.0f, (half_t)-64.0f};
    d = f16_to_f32(un.h.x);
    const float dmin = f16_to_f32(un.h.x >> 16);
    uint32_t h0, l0, h1, l1;
    bf16_split(-(dmin * (float)m0), h0, l0);  // exact product: 11 x 6 bits
    bf16_split(-(dmin * (float)m1), h1, l1);
    bh = hi_halves(h0, h1);
    bl = hi_halves(l0, l1);
  }
};

// Step S (0..7) of a unit: 8 exact float16 integers sc q for K values
// 8 (S & 3) .. of the low (S < 4) or high (S >= 4) nibbles of its 32 code
// bytes, in K order.
template <int S>
__device__ __forceinline__ half8_t sx_slice(const UnitQ4K& un, const SxConst& c) {
  constexpr int t = S & 3;
  const uint32_t q0 = t < 2 ? (t == 0 ? un.q0.x : un.q0.z) : (t == 2 ? un.q1.x : un.q1.z);
  const uint32_t q1 = t < 2 ? (t == 0 ? un.q0.y : un.q0.w) : (t == 2 ? un.q1.y : un.q1.w);
  const uint32_t mask = S < 4 ? 0x0F0F0F0Fu : 0xF0F0F0F0u;
  const uint32_t w0 = q0 & mask, w1 = q1 & mask;
  const half2_t s = S < 4 ? half2_t{c.k1.x, c.k1.x} : half2_t{c.k1.y, c.k1.y};
  const half2_t a = S < 4 ? half2_t{c.k2.x, c.k2.x} : half2_t{c.k2.y, c.k2.y};
  const uint32_t p[4] = {pair01(w0), pair23(w0), pair01(w1), pair23(w1)};
  u32x4 f;
  f.x = as_u32(__builtin_elementwise_fma(as_h2(p[0]), s, a));
  f.y = as_u32(__builtin_elementwise_fma(as_h2(p[1]), s, a));
  f.z = as_u32(__builtin_elementwise_fma(as_h2(p[2]), s, a));
  f.w = as_u32(__builtin_elementwise_fma(as_h2(p[3]), s, a));
  return __builtin_bit_cast(half8_t, f);
}

// One tile of XG live 16-row activation groups against 4 * 16 * RG weight rows
// (RG 16-row groups per wave).  DB: activation chunks double-buffered (one
// barrier per superblock) or single-buffered (two).
template <bool F16, int XG, int RG, bool DB>
__device__ __forceinline__ void sx_tile(const uint8_t* __restrict__ wbase, int n, int k, int64_t row_bytes,
                                        const half_t* __restrict__ xtile, int64_t x_bytes, int nr, int64_t yrow0,
                                        int n0, uint8_t* lds, void* __restrict__ y) {
  constexpr int NS = 2;                        // ring slots, one superblock each
  constexpr int XPT = XG * 16 * 32 / SX_THREADS;  // 16-byte activation pieces per thread per chunk
  constexpr int ROWS = DB ? 64 : 16 * XG;      // activation rows a buffer holds
  constexpr int XBUF = ROWS * SX_KC, WBUF = ROWS * 2 * SX_WROW;
  static_assert((DB ? 2 : 1) * XBUF * 2 + 2 * WBUF * 2 <= SX_LDS, "LDS");
  half_t* xs = (half_t*)lds;
  uint16_t* xw = (uint16_t*)(lds + (DB ? 2 : 1) * XBUF * 2);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, cu = lane >> 4;
  const int nsb = k / 256;

  // the wave's 16 RG weight rows from their (16-byte aligned) base; rows past N read as zeros
  const int64_t wrow0 = (int64_t)(n0 + wave * 16 * RG);
  const rsrc_t wrs = make_rsrc(wbase + wrow0 * row_bytes, (int64_t)(n - wrow0) * row_bytes);
  int rowoff[RG];
#pragma unroll
  for (int j = 0; j < RG; ++j) rowoff[j] = (16 * j + r) * (int)row_bytes;
  auto refill = [&](UnitQ4K* slot, int sb) __attribute__((always_inline)) {
    const int g = 4 * min(sb, nsb - 1);
#pragma unroll
    for (int j = 0; j < RG; ++j) slot[j].bload(wrs, rowoff[j], cu, g);
  };

  float4_t acc[RG][XG], part[RG][XG];
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int i = 0; i < XG; ++i) acc[j][i] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Staging: piece i of a thread is row prow + 8 i (prow = tid >> 5), stored
  // at physical chunk pc = tid & 31 of the row: logical chunk lc = swap34(pc ^
  // prow) for even i, lc ^ 16 for odd i (row & 15 = prow + 8 (i & 1)).  A
  // quad of lanes holds the four chunks of one 32-value sub-block.  Rows past
  // the tile hold whatever follows in x (offsets past its end read as zeros);
  // no stored output reads them.
  const rsrc_t xrs = make_rsrc(xtile, x_bytes);
  const int pc = tid & 31, prow = tid >> 5;
  const int lc = sx_swap34(pc ^ prow);
  const int xvoff0 = prow * k * 2 + lc * 16, xvoff1 = prow * k * 2 + (lc ^ 16) * 16;
  // Double-buffered chunks stage the next superblock in two halves of the
  // pieces (loaded at the chunk start and mid-chunk, each stored a half chunk
  // later), so only half of them occupy registers at a time; single-buffered
  // chunks hold all of them until every wave has read the chunk.
  constexpr int XH = DB ? XPT / 2 : XPT;  // pieces per staging half
  static_assert(XPT % 2 == 0, "staging halves");
  u32x4 xr[XH];
  auto load_x = [&](int sb, auto hc) __attribute__((always_inline)) {
    constexpr int H = decltype(hc)::value;
    const int so = min(sb, nsb - 1) * 512;
#pragma unroll
    for (int h = 0; h < XH; ++h) {
      const int i = H * XH + h;
      // each piece's offset is formed here from an opaque base, so the
      // compiler does not keep all of them in registers across the chunk
      int vo = i & 1 ? xvoff1 : xvoff0;
      asm volatile("" : "+v"(vo));
      xr[h] = bld16(xrs, vo + i * 8 * 2 * k, so);
    }
  };
  // Store the staged pieces of superblock sb into buffer sb & 1 and their
  // sub-block sums (float32 over 32 values: four lanes' 8 each) into window
  // buffer (sb >> 1) & 1 at position cu * 4 + (sb & 1) * 2 + e of the row's
  // hi and lo halves for sub-block j = 2 cu + e.  An odd piece's sub-block is
  // j ^ 4, which moves its slots by 24 (hi) and 8 (lo) from the even pieces'.
  auto store_x = [&](int sb, auto hc) __attribute__((always_inline)) {
    constexpr int H = decltype(hc)::value;
    half_t* xb = xs + (DB ? (sb & 1) * XBUF : 0);
    uint16_t* wb = xw + ((sb >> 1) & 1) * WBUF;
    const int j = lc >> 2, pos = (j >> 1) * 4 + (sb & 1) * 2 + (j & 1);
    const int w0 = sx_wslot(prow, pos >> 2) + (pos & 3);  // even pieces' hi; lo is w0 ^ 16
#pragma unroll
    for (int h = 0; h < XH; ++h) {
      const int i = H * XH + h;
      const int row = prow + 8 * i;
      *(u32x4*)(xb + row * SX_KC + 8 * pc) = xr[h];
      float s = 0.f;
      s = dot2(xr[h].x, 0x3C003C00u, s);
      s = dot2(xr[h].y, 0x3C003C00u, s);
      s = dot2(xr[h].z, 0x3C003C00u, s);
      s = dot2(xr[h].w, 0x3C003C00u, s);
      s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, true));
      s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, true));
      if ((pc & 3) == 0) {
        uint32_t hi, lo;
        bf16_split(s, hi, lo);
        wb[(i & 1 ? w0 ^ 24 : w0) + 256 * i] = (uint16_t)(hi >> 16);
        wb[(i & 1 ? w0 ^ 8 : w0 ^ 16) + 256 * i] = (uint16_t)(lo >> 16);
      }
    }
  };
  const auto h0 = std::integral_constant<int, 0>{};
  const auto h1 = std::integral_constant<int, 1>{};

  // prologue: superblock 0's activations and the first NS superblocks' weights
  UnitQ4K ring[NS][RG];
  load_x(0, h0);
  __builtin_amdgcn_sched_barrier(0);
  refill(ring[0], 0);
  __builtin_amdgcn_sched_barrier(0);
  store_x(0, h0);
  if constexpr (DB) {
    load_x(0, h1);
    __builtin_amdgcn_sched_barrier(0);
    refill(ring[1], 1);
    __builtin_amdgcn_sched_barrier(0);
    store_x(0, h1);
  } else {
    refill(ring[1], 1);
  }
  __syncthreads();

  // physical chunk of this lane's fragment reads: swap34(8 cu + S) ^ r
  const int ca = sx_swap34(8 * cu) ^ r;

  // bfloat16 -dmin m of the window's two superblocks, per weight group:
  // dword L holds sub-blocks (2 cu, 2 cu + 1) of superblock L of the window
  u32x2 bh[RG], bl[RG];

  // Superblock sb (L = sb & 1 its place in the window and its ring slot).
  // The activation fragments of step S + 1 are read from LDS while step S is
  // decoded and multiplied, so each step waits on reads issued a step earlier.
  auto chunk = [&](auto lc, int sb) __attribute__((always_inline)) {
    constexpr int L = decltype(lc)::value;
    const half_t* cur = xs + (DB ? L * XBUF : 0);
    // x loads first, then the refill of the slot the previous chunk decoded
    // (superblock sb + 1; at sb = 0 the same bytes the prologue loaded), so a
    // wait for the x pieces does not wait for these weights
    load_x(sb + 1, h0);
    if constexpr (DB) {
      __builtin_amdgcn_sched_barrier(0);
      refill(ring[L ^ 1], sb + 1);
    }
    UnitQ4K* slot = ring[L];
    SxConst c[RG];
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      c[j] = SxConst(slot[j], cu);
      bh[j][L] = c[j].bh;
      bl[j][L] = c[j].bl;
    }
    // Activation fragments of step S + 1 are read into the other register set
    // before step S's products, so their LDS latency runs under step S.
    half8_t a[2][XG];
    // The byte address of chunk ca ^ S of row r is a0 ^ 16 S (the chunk bits
    // lie below the row and buffer bits); a0 is made opaque at every step so
    // the eight addresses are not all held in registers.
    const uint32_t a0 = lds_addr(cur + r * SX_KC + 8 * ca);
    auto read_a = [&](half8_t* dst, auto sc) __attribute__((always_inline)) {
      constexpr int S = decltype(sc)::value;
      uint32_t ab = a0;
      asm volatile("" : "+v"(ab));
      const lds_half8_t* p = (const lds_half8_t*)(uintptr_t)(ab ^ (16u * S));
#pragma unroll
      for (int i = 0; i < XG; ++i) dst[i] = p[i * SX_KC * 2];  // rows 16 i + r: 16 i * 512 bytes
    };
    read_a(a[0], std::integral_constant<int, 0>{});
    auto step = [&](auto sc) __attribute__((always_inline)) {
      constexpr int S = decltype(sc)::value;
      if constexpr (S < 7) {
        read_a(a[(S + 1) & 1], std::integral_constant<int, S + 1>{});
        __builtin_amdgcn_sched_barrier(0);
      }
      half8_t b[RG];
#pragma unroll
      for (int j = 0; j < RG; ++j) b[j] = sx_slice<S>(slot[j], c[j]);
      if constexpr (!DB && S == 7) {
        // every step of the superblock is decoded: refill its registers
        __builtin_amdgcn_sched_barrier(0);
        refill(slot, sb + NS);
      }
#pragma unroll
      for (int i = 0; i < XG; ++i) {
#pragma unroll
        for (int j = 0; j < RG; ++j)
          part[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[S & 1][i], b[j],
                                                              S == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : part[j][i], 0, 0, 0);
      }
      if constexpr (DB && S == 3) {
        // the first half of the next superblock's pieces into the free buffer
        __builtin_amdgcn_sched_barrier(0);
        store_x(sb + 1, h0);
        load_x(sb + 1, h1);
      }
    };
    sx_for<8>(step);
#pragma unroll
    for (int i = 0; i < XG; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int j = 0; j < RG; ++j) acc[j][i][q] = fmaf(c[j].d, part[j][i][q], acc[j][i][q]);
      }
    }
    if constexpr (L == 1) {
      // the window's min term: (X hi + X lo) . (b hi + b lo) without lo . lo
      const uint16_t* wb = xw + ((sb >> 1) & 1) * WBUF;
      const int r0 = sx_wslot(r, cu);  // rows 16 i + r: + 512 i; lo: ^ 16
#pragma unroll
      for (int i = 0; i < XG; ++i) {
        const bf16x4_t ah = *(const bf16x4_t*)(wb + r0 + 512 * i);
        const bf16x4_t al = *(const bf16x4_t*)(wb + (r0 ^ 16) + 512 * i);
#pragma unroll
        for (int j = 0; j < RG; ++j) {
          const bf16x4_t h = __builtin_bit_cast(bf16x4_t, bh[j]), l = __builtin_bit_cast(bf16x4_t, bl[j]);
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, h, acc[j][i], 0, 0, 0);
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, l, acc[j][i], 0, 0, 0);
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, h, acc[j][i], 0, 0, 0);
        }
      }
    }
    // double-buffered: the other buffers were last read before the previous
    // barrier; single-buffered: wait until every wave has read this chunk
    if constexpr (DB) {
      store_x(sb + 1, h1);
    } else {
      __syncthreads();
      store_x(sb + 1, h0);
    }
    __syncthreads();
  };
  for (int sb = 0; sb < nsb; sb += 2) {
    chunk(std::integral_constant<int, 0>{}, sb);
    chunk(std::integral_constant<int, 1>{}, sb + 1);
  }

  // lane l holds activation rows 16 i + 4 (l >> 4) + q of weight row
  // n0 + 16 RG wave + 16 j + (l & 15)
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    const int col = n0 + wave * 16 * RG + 16 * j + (lane & 15);
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

// Map entry t is a full tile whose successor is a tail of the same expert on
// the rows right after it, of at most SX_MERGE_MAX rows: the two are worked as
// one tile.  Both tiles' workgroups evaluate this on the same entries, so a
// tail is covered either by itself or by its merged head, never both.
__device__ __forceinline__ bool sx_merges(const uint32_t* __restrict__ map, int t, int live_tiles, int m_total,
                                          int n_experts) {
  if (t < 0 || t + 1 >= live_tiles) return false;
  const uint32_t* a = map + 3 * (size_t)t;
  const uint32_t e0 = a[0], r0 = a[1], n0 = a[2], e1 = a[3], r1 = a[4], n1 = a[5];
  return e0 < (uint32_t)n_experts && e1 == e0 && n0 == 64 && r0 < (uint32_t)m_total && r1 == r0 + 64 && n1 >= 1 &&
         n1 <= SX_MERGE_MAX && r1 <= (uint32_t)m_total && n1 <= (uint32_t)m_total - r1;
}

template <bool F16>
__global__ __launch_bounds__(SX_THREADS, 2) void seg_exact_kernel(const uint8_t* __restrict__ w, int n, int k,
                                                                  int64_t row_bytes, int64_t expert_stride,
                                                                  int n_experts, const half_t* __restrict__ x,
                                                                  int m_total, const uint32_t* __restrict__ map,
                                                                  const uint32_t* __restrict__ counts, int cap,
                                                                  void* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[SX_LDS];

  // Workgroup b runs on XCD b % 8; the map's live (tile, column block) pairs
  // are split into eight contiguous ranges, one per XCD, so the blocks of a
  // tile share its activations, and consecutive tiles of one expert its
  // weights, in that XCD's L2.  Workgroups past the live count leave at once.
  const int nb = (n + SX_BN - 1) / SX_BN;
  const int64_t live = (int64_t)min(counts[0], (uint32_t)cap) * nb;
  const int64_t per_xcd = (live + SX_NXCD - 1) / SX_NXCD;
  const int64_t idx = blockIdx.x / SX_NXCD;
  if (idx >= per_xcd) return;
  const int64_t t = (int64_t)(blockIdx.x % SX_NXCD) * per_xcd + idx;
  if (t >= live) return;
  const int by = (int)(t / nb), blk = (int)(t - (int64_t)by * nb);
  const int live_tiles = (int)min(counts[0], (uint32_t)cap);
  // a full tile and its merged tail share both tiles' workgroups: 2 nb blocks of 64 weight rows
  const bool tail = sx_merges(map, by - 1, live_tiles, m_total, n_experts);
  if (tail || sx_merges(map, by, live_tiles, m_total, n_experts)) {
    const uint32_t* mt = map + 3 * (size_t)(tail ? by - 1 : by);
    const int n0 = (tail ? nb + blk : blk) * 64;
    if (n0 >= n) return;
    const uint32_t e = mt[0], rs = mt[1], nr = 64 + mt[5];
    sx_tile<F16, 5, 1, false>(w + (int64_t)e * expert_stride, n, k, row_bytes, x + (int64_t)rs * k,
                              (int64_t)(m_total - rs) * k * 2, (int)nr, rs, n0, lds, y);
    return;
  }
  const int n0 = blk * SX_BN;
  const uint32_t* mt = map + 3 * (size_t)by;
  const uint32_t e = mt[0], rs = mt[1], nr = mt[2];
  if (e >= (uint32_t)n_experts || nr == 0 || nr > 64 || rs >= (uint32_t)m_total || nr > (uint32_t)m_total - rs)
    return;
  const uint8_t* wbase = w + (int64_t)e * expert_stride;
  const half_t* xtile = x + (int64_t)rs * k;
  const int64_t x_bytes = (int64_t)(m_total - rs) * k * 2;
  switch ((nr + 15) >> 4) {  // 16-row activation groups holding live rows
    case 1: sx_tile<F16, 1, SX_RG, true>(wbase, n, k, row_bytes, xtile, x_bytes, (int)nr, rs, n0, lds, y); break;
    case 2: sx_tile<F16, 2, SX_RG, true>(wbase, n, k, row_bytes, xtile, x_bytes, (int)nr, rs, n0, lds, y); break;
    case 3: sx_tile<F16, 3, SX_RG, true>(wbase, n, k, row_bytes, xtile, x_bytes, (int)nr, rs, n0, lds, y); break;
    default: sx_tile<F16, 4, SX_RG, true>(wbase, n, k, row_bytes, xtile, x_bytes, (int)nr, rs, n0, lds, y); break;
  }
}

}  // namespace

// q4_K with K a multiple of 512 (whole windows of two superblocks) and 64
// rows of K values addressable by 32-bit buffer offsets; the caller routes
// other shapes to the float16-weight kernel.
bool seg_exact_ok(int codec, int64_t k) { return codec == Q4_K && k % 512 == 0 && 64 * k * 2 < (1ll << 31); }

hipError_t launch_seg_exact(const uint8_t* w, int64_t n_experts, int64_t n, int64_t k, int64_t row_bytes,
                            const half_t* x, int64_t rows, const uint32_t* map, const uint32_t* counts, int64_t cap,
                            void* y, int f16out, hipStream_t s) {
  const int64_t pairs = cap * ((n + SX_BN - 1) / SX_BN);  // (tile, column block) pairs the map can hold
  const dim3 grid((unsigned)((pairs + SX_NXCD - 1) / SX_NXCD * SX_NXCD));
  if (f16out)
    hipLaunchKernelGGL((seg_exact_kernel<true>), grid, dim3(SX_THREADS), 0, s, w, (int)n, (int)k, row_bytes,
                       n * row_bytes, (int)n_experts, x, (int)rows, map, counts, (int)cap, y);
  else
    hipLaunchKernelGGL((seg_exact_kernel<false>), grid, dim3(SX_THREADS), 0, s, w, (int)n, (int)k, row_bytes,
                       n * row_bytes, (int)n_experts, x, (int)rows, map, counts, (int)cap, y);
  return hipGetLastError();
}

}  // namespace kq
