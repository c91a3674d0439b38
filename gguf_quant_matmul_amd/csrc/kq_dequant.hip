// kq_dequantize: wire bytes -> float32 / float16, bit-exact.
//
// mlx-kquant bindings.cpp page, dequantize docstring.  Each value is the
// codec formula evaluated exactly and rounded once to float32:
//   q4_K, q5_K  (d*sc)*q - dmin*m : d*sc (<= 17 bits) and (d*sc)*q (<= 22 bits)
//         and dmin*m are exact in float32, so the subtraction is the only
//         rounding (an FMA gives the same bits);
//   q6_K  (d*sc)*(q-32), q8_0 d*q, q4_0 d*(q-8), q5_0 d*(q-16): exact products;
//   q4_1, q5_1  d*q + m: one fma (the exact value rounded once).
// float16 output is the RNE conversion of that float32 value.
//
// One thread produces 8 consecutive values of a row, so each thread's store
// is one 16-byte (f16) or two 16-byte (f32) vector stores and a wave writes a
// contiguous span.  The kernel is HBM-bound: it reads block_bytes per
// block_values weights and writes 2 or 4 bytes per weight.
#include "kq_decode.h"

namespace kq {
namespace {

template <int C, bool F16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ w, int64_t rows, int64_t k,
                                                      int64_t row_bytes, void* __restrict__ out) {
  const int64_t gpr = k / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * gpr) return;
  const int64_t r = gid / gpr;
  const int64_t v0 = (gid - r * gpr) * 8;
  float v[8];
  decode8<C>(w + r * row_bytes, v0, v);
  const int64_t o = r * k + v0;
  if (F16) {
    half8_t hv;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // The float16 output is the RNE of the float32 value: keep the compiler
      // from fusing the float32 multiply-add into the conversion (v_fma_mix
      // rounds the exact result straight to float16).
      float f = v[i];
      asm volatile("" : "+v"(f));
      hv[i] = (half_t)f;
    }
    *(half8_t*)((half_t*)out + o) = hv;
  } else {
    float4_t a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    *(float4_t*)((float*)out + o) = a;
    *(float4_t*)((float*)out + o + 4) = b;
  }
}

template <int C>
hipError_t launch_c(const uint8_t* w, int64_t rows, int64_t k, int64_t rb, void* out, int f16, hipStream_t s) {
  const int64_t threads = rows * (k / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (f16)
    hipLaunchKernelGGL((dequant_kernel<C, true>), grid, dim3(256), 0, s, w, rows, k, rb, out);
  else
    hipLaunchKernelGGL((dequant_kernel<C, false>), grid, dim3(256), 0, s, w, rows, k, rb, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize(int codec, const uint8_t* w, int64_t rows, int64_t k, int64_t rb, void* out, int f16,
                             hipStream_t s) {
  switch (codec) {
    case Q4_0: return launch_c<Q4_0>(w, rows, k, rb, out, f16, s);
    case Q8_0: return launch_c<Q8_0>(w, rows, k, rb, out, f16, s);
    case Q2_K: return launch_c<Q2_K>(w, rows, k, rb, out, f16, s);
    case Q3_K: return launch_c<Q3_K>(w, rows, k, rb, out, f16, s);
    case Q4_K: return launch_c<Q4_K>(w, rows, k, rb, out, f16, s);
    case Q5_K: return launch_c<Q5_K>(w, rows, k, rb, out, f16, s);
    case Q4_1: return launch_c<Q4_1>(w, rows, k, rb, out, f16, s);
    case Q5_0: return launch_c<Q5_0>(w, rows, k, rb, out, f16, s);
    case Q5_1: return launch_c<Q5_1>(w, rows, k, rb, out, f16, s);
    case Q6_K: return launch_c<Q6_K>(w, rows, k, rb, out, f16, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kq
