// kq_qmv_gather: the gathered GEMV and the MoE GLU gather (decode MoE)
// (the kernels and their launchers: kq_qmv_impl.h).
#include "kq_qmv_impl.h"

namespace kq {

hipError_t launch_gather_qmv(int codec, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k,
                             int64_t row_bytes, const half_t* x, const uint32_t* ids, int64_t rows, void* y,
                             int f16out, hipStream_t s) {
  switch (codec) {
    case Q4_0: return launch_gather_c<Q4_0>(w, n_experts, n, k, row_bytes, x, ids, rows, y, f16out, s);
    case Q8_0: return launch_gather_c<Q8_0>(w, n_experts, n, k, row_bytes, x, ids, rows, y, f16out, s);
    case Q4_1: return launch_gather_c<Q4_1>(w, n_experts, n, k, row_bytes, x, ids, rows, y, f16out, s);
    case Q5_0: return launch_gather_c<Q5_0>(w, n_experts, n, k, row_bytes, x, ids, rows, y, f16out, s);
    case Q5_1: return launch_gather_c<Q5_1>(w, n_experts, n, k, row_bytes, x, ids, rows, y, f16out, s);
    case Q2_K: return launch_gather_c<Q2_K>(w, n_experts, n, k, row_bytes, x, ids, rows, y, f16out, s);
    case Q3_K: return launch_gather_c<Q3_K>(w, n_experts, n, k, row_bytes, x, ids, rows, y, f16out, s);
    case Q4_K: return launch_gather_c<Q4_K>(w, n_experts, n, k, row_bytes, x, ids, rows, y, f16out, s);
    case Q5_K: return launch_gather_c<Q5_K>(w, n_experts, n, k, row_bytes, x, ids, rows, y, f16out, s);
    case Q6_K: return launch_gather_c<Q6_K>(w, n_experts, n, k, row_bytes, x, ids, rows, y, f16out, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_moe_glu_gather(int codec, const uint8_t* gate_w, const uint8_t* up_w, int64_t n_experts, int64_t n,
                                 int64_t k, int64_t row_bytes, const half_t* x, const uint32_t* ids, int64_t rows,
                                 int64_t top_k, int act, float limit, void* y, int f16out, hipStream_t s) {
  switch (codec) {
    case Q4_0:
      return launch_glu_c<Q4_0>(gate_w, up_w, n_experts, n, k, row_bytes, x, ids, rows, top_k, act, limit, y, f16out, s);
    case Q8_0:
      return launch_glu_c<Q8_0>(gate_w, up_w, n_experts, n, k, row_bytes, x, ids, rows, top_k, act, limit, y, f16out, s);
    case Q4_1:
      return launch_glu_c<Q4_1>(gate_w, up_w, n_experts, n, k, row_bytes, x, ids, rows, top_k, act, limit, y, f16out, s);
    case Q5_0:
      return launch_glu_c<Q5_0>(gate_w, up_w, n_experts, n, k, row_bytes, x, ids, rows, top_k, act, limit, y, f16out, s);
    case Q5_1:
      return launch_glu_c<Q5_1>(gate_w, up_w, n_experts, n, k, row_bytes, x, ids, rows, top_k, act, limit, y, f16out, s);
    case Q2_K:
      return launch_glu_c<Q2_K>(gate_w, up_w, n_experts, n, k, row_bytes, x, ids, rows, top_k, act, limit, y, f16out, s);
    case Q3_K:
      return launch_glu_c<Q3_K>(gate_w, up_w, n_experts, n, k, row_bytes, x, ids, rows, top_k, act, limit, y, f16out, s);
    case Q4_K:
      return launch_glu_c<Q4_K>(gate_w, up_w, n_experts, n, k, row_bytes, x, ids, rows, top_k, act, limit, y, f16out, s);
    case Q5_K:
      return launch_glu_c<Q5_K>(gate_w, up_w, n_experts, n, k, row_bytes, x, ids, rows, top_k, act, limit, y, f16out, s);
    case Q6_K:
      return launch_glu_c<Q6_K>(gate_w, up_w, n_experts, n, k, row_bytes, x, ids, rows, top_k, act, limit, y, f16out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kq
