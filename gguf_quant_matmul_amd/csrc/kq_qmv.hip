// kq_qmv: the quantized GEMV (decode, M <= 8)
// (the kernels and their launchers: kq_qmv_impl.h).
#include "kq_qmv_impl.h"

namespace kq {

hipError_t launch_qmv(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int m, void* y,
                      int f16, hipStream_t s) {
  switch (codec) {
    case Q4_0: return launch_c<Q4_0>(w, n, k, rb, x, m, y, f16, s);
    case Q8_0: return launch_c<Q8_0>(w, n, k, rb, x, m, y, f16, s);
    case Q4_1: return launch_c<Q4_1>(w, n, k, rb, x, m, y, f16, s);
    case Q5_0: return launch_c<Q5_0>(w, n, k, rb, x, m, y, f16, s);
    case Q5_1: return launch_c<Q5_1>(w, n, k, rb, x, m, y, f16, s);
    case Q2_K: return launch_c<Q2_K>(w, n, k, rb, x, m, y, f16, s);
    case Q3_K: return launch_c<Q3_K>(w, n, k, rb, x, m, y, f16, s);
    case Q4_K: return launch_c<Q4_K>(w, n, k, rb, x, m, y, f16, s);
    case Q5_K: return launch_c<Q5_K>(w, n, k, rb, x, m, y, f16, s);
    case Q6_K: return launch_c<Q6_K>(w, n, k, rb, x, m, y, f16, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kq
