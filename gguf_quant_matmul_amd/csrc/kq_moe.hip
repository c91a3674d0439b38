// kq_expert_tile_map: tiles of <= 64 rows per expert segment of expert-sorted
// routing ids, built on the GPU (mlx-kquant bindings.cpp page,
// expert_tile_map docstring: (expert, row_start, num_rows) tiles, only the
// last tile of a segment partial, a valid-tile count, no host sync).
//
// One workgroup: each thread finds its expert's segment with two binary
// searches over the sorted ids (lower bounds of e and e+1), a workgroup
// prefix sum over ceil(count/64) gives each expert its first slot, and tiles
// are written in expert-major order.  No atomics on the output: the map is
// the same bits run to run.  A linear pass over the ids reports unsorted ids
// and ids >= n_experts in the optional status word.
#include "kq_internal.h"

namespace kq {
namespace {

constexpr int TM_THREADS = 1024;

__device__ __forceinline__ uint32_t lower_bound(const uint32_t* __restrict__ ids, uint32_t rows, uint32_t key) {
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

__global__ __launch_bounds__(TM_THREADS) void tile_map_kernel(const uint32_t* __restrict__ ids, uint32_t rows,
                                                              uint32_t n_experts, uint32_t* __restrict__ map,
                                                              uint32_t* __restrict__ counts, uint32_t cap,
                                                              uint32_t* __restrict__ status) {
  __shared__ uint64_t scan[TM_THREADS];
  __shared__ uint32_t flags;
  __shared__ uint64_t carry;
  const uint32_t tid = threadIdx.x;
  if (tid == 0) { flags = 0; carry = 0; }
  __syncthreads();

  uint32_t f = 0;
  for (uint32_t i = tid; i < rows; i += TM_THREADS) {
    const uint32_t v = ids[i];
    if (v >= n_experts) f |= 2u;
    if (i + 1 < rows && v > ids[i + 1]) f |= 1u;
  }
  if (f) atomicOr(&flags, f);  // an OR: the result does not depend on the order

  for (uint32_t e0 = 0; e0 < n_experts; e0 += TM_THREADS) {
    const uint32_t e = e0 + tid;
    uint32_t lo = 0, cnt = 0, nt = 0;
    if (e < n_experts) {
      lo = lower_bound(ids, rows, e);
      const uint32_t hi = lower_bound(ids, rows, e + 1);
      cnt = hi > lo ? hi - lo : 0;
      nt = (cnt + 63) / 64;
    }
    // inclusive Hillis-Steele scan of nt over the workgroup
    scan[tid] = nt;
    __syncthreads();
    for (uint32_t o = 1; o < TM_THREADS; o <<= 1) {
      const uint64_t add = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const uint64_t first = carry + scan[tid] - nt;
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
    if (tid == TM_THREADS - 1) carry += scan[tid];
    __syncthreads();
  }
  if (tid == 0) {
    uint64_t total = carry;
    uint32_t fl = flags;
    if (total > cap) { fl |= 4u; total = cap; }
    counts[0] = (uint32_t)total;
    if (status) *status = fl;
  }
}

}  // namespace

hipError_t launch_tile_map(const uint32_t* ids, int64_t rows, int64_t n_experts, uint32_t* map, uint32_t* counts,
                           int64_t cap, uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(TM_THREADS), 0, s, ids, (uint32_t)rows, (uint32_t)n_experts, map,
                     counts, (uint32_t)cap, status);
  return hipGetLastError();
}

}  // namespace kq
