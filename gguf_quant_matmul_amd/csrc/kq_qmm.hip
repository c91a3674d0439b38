// kq_qmm: the plain quantized GEMM and the kq_gather_qmm_seg dispatch (the
// segment kernel is in kq_seg.hip; K that is not a whole number of 64-value
// units takes the plain kernel for both)
// (the kernel and its launchers: kq_qmm_impl.h).
#include "kq_qmm_impl.h"

namespace kq {

hipError_t launch_qmm(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int64_t m,
                      void* y, int f16, hipStream_t s) {
  return launch_pass<EP_PLAIN, 0>(codec, w, n, k, rb, x, m, y, f16, Epi{nullptr, nullptr, nullptr, 1}, s);
}

hipError_t launch_gather_qmm_seg(int codec, const uint8_t* w, int64_t ne, int64_t n, int64_t k, int64_t rb,
                                 const half_t* x, int64_t rows, const uint32_t* map, const uint32_t* counts,
                                 int64_t cap, void* y, int f16, hipStream_t s) {
  if (k % 64 != 0 || k > (1 << 24)) {  // the segment kernel's buffer offsets are 32-bit
    switch (codec) {
      case Q4_0: return launch_generic<Q4_0, true>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
      case Q8_0: return launch_generic<Q8_0, true>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
      case Q4_1: return launch_generic<Q4_1, true>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
      case Q5_0: return launch_generic<Q5_0, true>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
      case Q5_1: return launch_generic<Q5_1, true>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
      case Q2_K: return launch_generic<Q2_K, true>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
      case Q3_K: return launch_generic<Q3_K, true>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
      case Q4_K: return launch_generic<Q4_K, true>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
      case Q5_K: return launch_generic<Q5_K, true>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
      case Q6_K: return launch_generic<Q6_K, true>(w, n, k, rb, n * rb, ne, x, rows, map, counts, cap, y, f16, s);
    }
    return hipErrorInvalidValue;
  }
  if (seg_exact_ok(codec, k))  // q4_K: exact integer weight operands
    return launch_seg_exact(w, ne, n, k, rb, x, rows, map, counts, cap, y, f16, s);
  return launch_seg_mma(codec, w, ne, n, k, rb, x, rows, map, counts, cap, y, f16, s);
}

}  // namespace kq
