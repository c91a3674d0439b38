// kq_qmv_wide_epi: the residual / gate epilogue of
// kq_quantized_matmul_residual for 3..64 activation rows on the wide
// matrix-core GEMV (the kernel and its launchers: kq_qmv_wide_impl.h).
#include "kq_qmv_wide_impl.h"

namespace kq {

hipError_t launch_qmv_wide_epi(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int m,
                               const Epi& epi, void* y, int f16, hipStream_t s) {
  if (m < 1 || m > QMV_WIDE_MAX_M || k % 64 != 0) return hipErrorInvalidValue;
  return launch_wide<EP_EPI>(codec, w, n, k, rb, x, m, epi, 0, y, f16, s);
}

}  // namespace kq
