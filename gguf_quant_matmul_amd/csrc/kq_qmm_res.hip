// kq_qmm_res: the GEMM with residual stores (y = acc + r, y = fma(g, acc, r))
// (the kernel and its launchers: kq_qmm_impl.h).
#include "kq_qmm_impl.h"

namespace kq {

// the GEMM takes a residual with or without a gate (no bias)
hipError_t launch_qmm_epi(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t row_bytes, const half_t* x,
                          int64_t m, const Epi& epi, void* y, int f16out, hipStream_t s) {
  if (!epi.resid || epi.bias) return hipErrorInvalidValue;
  if (epi.gate) return launch_pass<EP_RES_GATE, 0>(codec, w, n, k, row_bytes, x, m, y, f16out, epi, s);
  return launch_pass<EP_RES, 0>(codec, w, n, k, row_bytes, x, m, y, f16out, epi, s);
}

}  // namespace kq
