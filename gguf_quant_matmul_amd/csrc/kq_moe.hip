// kq_expert_tile_map: tiles of <= 64 rows per expert segment of expert-sorted
// routing ids, built on the GPU (mlx-kquant bindings.cpp page,
// expert_tile_map docstring: (expert, row_start, num_rows) tiles, only the
// last tile of a segment partial, a valid-tile count, no host sync).
//
// One workgroup: the ids are copied to LDS once (up to TM_LDS_IDS of them;
// longer inputs are searched in place), each thread finds its expert's segment
// with one binary search (the lower bound of e; the end of its segment is
// the next expert's lower bound, taken from the next thread), a wave-level prefix
// sum over ceil(count/64) plus one over the sixteen wave totals gives each
// expert its first slot, and tiles are written in expert-major order.  No
// atomics on the output: the map is the same bits run to run.  A linear pass
// over the ids reports unsorted ids and ids >= n_experts in the optional
// status word.
#include "kq_internal.h"

namespace kq {
namespace {

constexpr int TM_THREADS = 1024;
constexpr int TM_WAVES = TM_THREADS / 64;
constexpr uint32_t TM_LDS_IDS = 12288;  // 48 KB

template <typename P>
__device__ __forceinline__ uint32_t lower_bound(P ids, uint32_t rows, uint32_t key) {
  uint32_t lo = 0, hi = rows;
  while (lo < hi) {
    const uint32_t mid = lo + (hi - lo) / 2;
    if (ids[mid] < key)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// inclusive prefix sum over the 64 lanes of a wave (64-bit: with unsorted
// ids the segment counts are meaningless and their sum can pass 2^32)
__device__ __forceinline__ uint64_t wave_scan(uint64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// The map from ids at src (LDS or global): status flags, per-expert segments,
// the tile slots; returns through the shared carry / flags.
template <typename P>
__device__ __forceinline__ void tile_map_body(P src, uint32_t rows, uint32_t n_experts, uint32_t* __restrict__ map,
                                              uint32_t cap, uint64_t* wsum, uint32_t* wlo, uint32_t& flags,
                                              uint64_t& carry) {
  const uint32_t tid = threadIdx.x;
  const int lane = (int)(tid & 63), wave = (int)(tid >> 6);
  uint32_t f = 0;
  for (uint32_t i = tid; i < rows; i += TM_THREADS) {
    const uint32_t v = src[i];
    if (v >= n_experts) f |= 2u;
    if (i + 1 < rows && v > src[i + 1]) f |= 1u;
  }
  if (f) atomicOr(&flags, f);  // an OR: the result does not depend on the order

  for (uint32_t e0 = 0; e0 < n_experts; e0 += TM_THREADS) {
    // expert e's segment is [lower_bound(e), lower_bound(e + 1)): each thread
    // searches once and takes the end of its segment from the next lane (the
    // last lane of a wave from LDS, the last thread of the round searches it)
    const uint32_t e = e0 + tid;
    const uint32_t lo = e <= n_experts ? lower_bound(src, rows, e) : rows;  // e = n_experts: the first id >= E
    uint32_t hi = __shfl_down(lo, 1, 64);
    if (lane == 0) wlo[wave] = lo;  // the end of the previous wave's last segment
    const uint32_t last_hi = tid == TM_THREADS - 1 && e < n_experts ? lower_bound(src, rows, e + 1) : rows;
    __syncthreads();
    if (lane == 63) hi = wave + 1 < TM_WAVES ? wlo[wave + 1] : last_hi;
    uint32_t cnt = 0, nt = 0;
    if (e < n_experts) {
      cnt = hi > lo ? hi - lo : 0;
      nt = (cnt + 63) / 64;
    }
    // tiles before this expert: the wave's inclusive scan, plus the totals of
    // the waves before it, plus the experts of earlier rounds (carry)
    const uint64_t incl = wave_scan(nt, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint64_t before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const uint64_t first = before + incl - nt;
    for (uint32_t t = 0; t < nt; ++t) {
      const uint64_t slot = first + t;
      if (slot < cap) {
        const uint32_t left = cnt - 64 * t;
        uint32_t* m = map + 3 * (size_t)slot;
        m[0] = e;
        m[1] = lo + 64 * t;
        m[2] = left < 64 ? left : 64;
      }
    }
    __syncthreads();
    if (tid == TM_THREADS - 1) carry = first + nt;
    __syncthreads();
  }
}

__global__ __launch_bounds__(TM_THREADS) void tile_map_kernel(const uint32_t* __restrict__ ids, uint32_t rows,
                                                              uint32_t n_experts, uint32_t* __restrict__ map,
                                                              uint32_t* __restrict__ counts, uint32_t cap,
                                                              uint32_t* __restrict__ status) {
  __shared__ uint32_t sid[TM_LDS_IDS];
  __shared__ uint64_t wsum[TM_WAVES];
  __shared__ uint32_t wlo[TM_WAVES];
  __shared__ uint32_t flags;
  __shared__ uint64_t carry;
  const uint32_t tid = threadIdx.x;
  if (tid == 0) { flags = 0; carry = 0; }
  if (rows <= TM_LDS_IDS) {
    for (uint32_t i = tid; i < rows; i += TM_THREADS) sid[i] = ids[i];
    __syncthreads();
    tile_map_body((const uint32_t*)sid, rows, n_experts, map, cap, wsum, wlo, flags, carry);
  } else {
    __syncthreads();
    tile_map_body(ids, rows, n_experts, map, cap, wsum, wlo, flags, carry);
  }
  if (tid == 0) {
    uint64_t total = carry;
    uint32_t fl = flags;
    if (total > cap) { fl |= 4u; total = cap; }
    counts[0] = (uint32_t)total;
    if (status) *status = fl;
  }
}

// kq_gather_mix (mlx-kquant bindings.cpp page, gather_mix docstring): the
// unsort and score mix after a sorted-prefill MoE,
// out[t] = sum_s scores[t, s] * y[inv_order[t * top_k + s]], slots summed in
// order in float32 (fma), one rounding at the store.  Slots whose row is not
// below `rows` add nothing.  Each thread takes 4 consecutive columns of one
// token (one 8-byte float16 or 16-byte float32 load per slot); blockIdx.y is
// the token.
constexpr int GM_THREADS = 256;

template <typename T>
__global__ __launch_bounds__(GM_THREADS) void gather_mix_kernel(const T* __restrict__ y, uint32_t rows, int n,
                                                                const uint32_t* __restrict__ inv,
                                                                const float* __restrict__ scores, int top_k, int t0,
                                                                T* __restrict__ out) {
  typedef T T4 __attribute__((ext_vector_type(4)));
  const int64_t t = t0 + (int64_t)blockIdx.y;
  const int c = (int)(blockIdx.x * GM_THREADS + threadIdx.x) * 4;
  if (c >= n) return;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  // four slots at a time: their row indices, then their rows, go out together
  for (int s0 = 0; s0 < top_k; s0 += 4) {
    uint32_t r[4];
    float w[4];
    T4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool live = s0 + j < top_k;
      r[j] = live ? inv[t * top_k + s0 + j] : rows;
      w[j] = live ? scores[t * top_k + s0 + j] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = r[j] < rows ? *(const T4*)(y + (int64_t)r[j] * n + c) : T4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (r[j] < rows) {  // slots in order; a slot with no row adds nothing
        a0 = fmaf(w[j], (float)v[j].x, a0);
        a1 = fmaf(w[j], (float)v[j].y, a1);
        a2 = fmaf(w[j], (float)v[j].z, a2);
        a3 = fmaf(w[j], (float)v[j].w, a3);
      }
    }
  }
  *(T4*)(out + t * n + c) = T4{(T)a0, (T)a1, (T)a2, (T)a3};
}

template <typename T>
hipError_t launch_gather_mix_t(const void* y, int64_t rows, int64_t n, const uint32_t* inv, const float* scores,
                               int64_t tokens, int64_t top_k, void* out, hipStream_t s) {
  const unsigned gx = (unsigned)((n / 4 + GM_THREADS - 1) / GM_THREADS);
  for (int64_t t0 = 0; t0 < tokens; t0 += 65535) {  // grid y holds at most 65535 tokens per launch
    const dim3 grid(gx, (unsigned)(tokens - t0 < 65535 ? tokens - t0 : 65535));
    hipLaunchKernelGGL((gather_mix_kernel<T>), grid, dim3(GM_THREADS), 0, s, (const T*)y, (uint32_t)rows, (int)n, inv,
                       scores, (int)top_k, (int)t0, (T*)out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gather_mix(const void* y, int64_t rows, int64_t n, const uint32_t* inv_order, const float* scores,
                             int64_t tokens, int64_t top_k, void* out, int f16, hipStream_t s) {
  if (f16) return launch_gather_mix_t<half_t>(y, rows, n, inv_order, scores, tokens, top_k, out, s);
  return launch_gather_mix_t<float>(y, rows, n, inv_order, scores, tokens, top_k, out, s);
}

hipError_t launch_tile_map(const uint32_t* ids, int64_t rows, int64_t n_experts, uint32_t* map, uint32_t* counts,
                           int64_t cap, uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(TM_THREADS), 0, s, ids, (uint32_t)rows, (uint32_t)n_experts, map,
                     counts, (uint32_t)cap, status);
  return hipGetLastError();
}

}  // namespace kq
