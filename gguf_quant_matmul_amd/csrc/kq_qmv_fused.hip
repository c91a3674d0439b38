// kq_qmv_fused: the GEMV with the matmul epilogue and the GLU product of two
// matrices
// (the kernels and their launchers: kq_qmv_impl.h).
#include "kq_qmv_impl.h"

namespace kq {

namespace {

hipError_t launch_fused(int codec, const uint8_t* w, const uint8_t* w2, int64_t n, int64_t k, int64_t rb,
                        const half_t* x, int m, const Epi& epi, int act, bool glu, void* y, int f16, hipStream_t s) {
  switch (codec) {
    case Q4_0: return launch_fused_c<Q4_0>(w, w2, n, k, rb, x, m, epi, act, glu, y, f16, s);
    case Q8_0: return launch_fused_c<Q8_0>(w, w2, n, k, rb, x, m, epi, act, glu, y, f16, s);
    case Q4_1: return launch_fused_c<Q4_1>(w, w2, n, k, rb, x, m, epi, act, glu, y, f16, s);
    case Q5_0: return launch_fused_c<Q5_0>(w, w2, n, k, rb, x, m, epi, act, glu, y, f16, s);
    case Q5_1: return launch_fused_c<Q5_1>(w, w2, n, k, rb, x, m, epi, act, glu, y, f16, s);
    case Q2_K: return launch_fused_c<Q2_K>(w, w2, n, k, rb, x, m, epi, act, glu, y, f16, s);
    case Q3_K: return launch_fused_c<Q3_K>(w, w2, n, k, rb, x, m, epi, act, glu, y, f16, s);
    case Q4_K: return launch_fused_c<Q4_K>(w, w2, n, k, rb, x, m, epi, act, glu, y, f16, s);
    case Q5_K: return launch_fused_c<Q5_K>(w, w2, n, k, rb, x, m, epi, act, glu, y, f16, s);
    case Q6_K: return launch_fused_c<Q6_K>(w, w2, n, k, rb, x, m, epi, act, glu, y, f16, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qmv_epi(int codec, const uint8_t* w, int64_t n, int64_t k, int64_t row_bytes, const half_t* x,
                          int m, const Epi& epi, void* y, int f16out, hipStream_t s) {
  return launch_fused(codec, w, nullptr, n, k, row_bytes, x, m, epi, 0, false, y, f16out, s);
}

hipError_t launch_qmv_glu(int codec, const uint8_t* w_gate, const uint8_t* w_up, int64_t n, int64_t k,
                          int64_t row_bytes, const half_t* x, int m, int act, void* y, int f16out, hipStream_t s) {
  if (act != GLU_SILU && act != GLU_GELU_TANH) return hipErrorInvalidValue;
  return launch_fused(codec, w_gate, w_up, n, k, row_bytes, x, m, Epi{nullptr, nullptr, nullptr, 1}, act, true, y,
                      f16out, s);
}

}  // namespace kq
