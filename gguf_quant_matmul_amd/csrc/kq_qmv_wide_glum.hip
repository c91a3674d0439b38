// kq_qmv_wide_glum: the up pass of the GLU product on the wide matrix-core
// GEMV, y = round(y * (x . up)) with y the gate pass's activation (the
// kernel and its launchers: kq_qmv_wide_impl.h; the gate pass:
// kq_qmv_wide_glu.hip).
#include "kq_qmv_wide_impl.h"

namespace kq {

hipError_t launch_qmv_wide_glu_mul(int codec, const uint8_t* w_up, int64_t n, int64_t k, int64_t rb, const half_t* x,
                                   int m, void* y, int f16, hipStream_t s) {
  if (m < 1 || m > QMV_WIDE_MAX_M || k % 64 != 0) return hipErrorInvalidValue;
  return launch_wide<EP_GLU_MUL>(codec, w_up, n, k, rb, x, m, Epi{nullptr, nullptr, nullptr, 1}, 0, y, f16, s);
}

}  // namespace kq
