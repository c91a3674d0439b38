// kq_stream_read: the plain-read reference of the GEMV rows.  Each
// workgroup reads one contiguous 1/G of the buffer with nontemporal 16-byte
// loads, eight in flight per thread, and each of its waves writes the XOR of
// what it read to out[4 * blockIdx.x + wave] (so the loads cannot be dropped;
// no barrier or LDS at the end).  It moves the same bytes a GEMV's weight
// stream does, with no decode and no arithmetic, which puts a measured
// ceiling beside the GEMV rates under the same launch protocol.
#include "kq_internal.h"

namespace kq {
namespace {

constexpr int SR_THREADS = 256;

__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                 uint32_t* __restrict__ out) {
  constexpr int U = 8;
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per, b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  int64_t i = b0 + threadIdx.x;
  for (; i + (U - 1) * SR_THREADS < b1; i += U * SR_THREADS) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * SR_THREADS);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < b1; i += SR_THREADS) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) out[4 * blockIdx.x + (threadIdx.x >> 6)] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* out, int64_t groups, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)groups), dim3(SR_THREADS), 0, s, (const u32x4*)src, bytes / 16,
                     out);
  return hipGetLastError();
}

}  // namespace kq
