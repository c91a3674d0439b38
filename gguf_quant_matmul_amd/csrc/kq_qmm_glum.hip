// kq_qmm_glum: the up pass of the GEMM GLU product (y = round(y * acc))
// (the kernel and its launchers: kq_qmm_impl.h).
#include "kq_qmm_impl.h"

namespace kq {

hipError_t launch_qmm_glu_mul(int codec, const uint8_t* w_up, int64_t n, int64_t k, int64_t row_bytes,
                              const half_t* x, int64_t m, void* y, int f16out, hipStream_t s) {
  return launch_pass<EP_GLU_MUL, 0>(codec, w_up, n, k, row_bytes, x, m, y, f16out, Epi{nullptr, nullptr, nullptr, 1}, s);
}

}  // namespace kq
