// kq_qmv_wide_glu: the GLU product of kq_quantized_matmul_glu for 4..64
// activation rows on the wide matrix-core GEMV, as two passes on the stream
// (the GEMM's split): the gate pass stores act(x . gate) rounded to y's type
// in y, the up pass multiplies it by x . up and rounds again (the kernel and
// its launchers: kq_qmv_wide_impl.h).  The up pass is in kq_qmv_wide_glum.hip.
#include "kq_qmv_wide_impl.h"

namespace kq {

hipError_t launch_qmv_wide_glu_act(int codec, const uint8_t* w_gate, int64_t n, int64_t k, int64_t rb, const half_t* x,
                                   int m, int act, void* y, int f16, hipStream_t s) {
  if (m < 1 || m > QMV_WIDE_MAX_M || k % 64 != 0 || (act != GLU_SILU && act != GLU_GELU_TANH))
    return hipErrorInvalidValue;
  return launch_wide<EP_GLU_ACT>(codec, w_gate, n, k, rb, x, m, Epi{nullptr, nullptr, nullptr, 1}, act, y, f16, s);
}

}  // namespace kq
