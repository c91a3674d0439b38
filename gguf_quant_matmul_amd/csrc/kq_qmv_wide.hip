// kq_qmv_wide: the plain product for 9..64 activation rows (kq_qmv's 9..16,
// kq_quantized_matmul's 17..64; the kernel and its launchers:
// kq_qmv_wide_impl.h).
#include "kq_qmv_wide_impl.h"

namespace kq {

hipError_t launch_qmv_wide(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t rb, const half_t* x, int m,
                           void* y, int f16, hipStream_t s) {
  if (m < 9 || m > QMV_WIDE_MAX_M || k % 64 != 0) return hipErrorInvalidValue;
  return launch_wide<EP_PLAIN>(codec, w, n, k, rb, x, m, Epi{nullptr, nullptr, nullptr, 1}, 0, y, f16, s);
}

}  // namespace kq
