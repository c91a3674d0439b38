// kq_qmm_glu: the GEMM GLU product, its gate pass (activation stores)
// (the kernel and its launchers: kq_qmm_impl.h).
#include "kq_qmm_impl.h"

namespace kq {

// The GLU product as two passes on one stream: the gate pass stores the
// rounded activation in y, the up pass multiplies its product by it; each
// output element is read and written by the same lane of the same tile.
hipError_t launch_qmm_glu(int codec, const uint8_t* w_gate, const uint8_t* w_up, int64_t n, int64_t k,
                          int64_t row_bytes, const half_t* x, int64_t m, int act, void* y, int f16out, hipStream_t s) {
  const Epi none{nullptr, nullptr, nullptr, 1};
  hipError_t e;
  if (act == GLU_SILU)
    e = launch_pass<EP_GLU_ACT, GLU_SILU>(codec, w_gate, n, k, row_bytes, x, m, y, f16out, none, s);
  else if (act == GLU_GELU_TANH)
    e = launch_pass<EP_GLU_ACT, GLU_GELU_TANH>(codec, w_gate, n, k, row_bytes, x, m, y, f16out, none, s);
  else
    return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  return launch_qmm_glu_mul(codec, w_up, n, k, row_bytes, x, m, y, f16out, s);
}

}  // namespace kq
