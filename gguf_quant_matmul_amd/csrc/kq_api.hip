// C ABI of libkq: argument validation and kernel dispatch.
//
// Every entry point validates on the host and returns before any HIP call
// when an argument is wrong (outputs untouched); otherwise it enqueues the
// kernels on the caller's stream and returns without synchronizing.  The
// error style mirrors the "[module.op] message" invalid-argument text of the
// mlx-kquant bindings.cpp page and the "op: msg" errors of nuvec-core's
// quantized.rs page.
#include <ctype.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "kq_internal.h"
#include "../../include/kq.h"

namespace {

thread_local std::string g_err;

int fail(int status, const char* op, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = std::string("[") + op + "] " + buf;
  return status;
}

const char* codec_name(int c) {
  switch (c) {
    case KQ_Q4_0: return "q4_0";
    case KQ_Q8_0: return "q8_0";
    case KQ_Q4_K: return "q4_k";
    case KQ_Q5_K: return "q5_k";
    case KQ_Q2_K: return "q2_k";
    case KQ_Q3_K: return "q3_k";
    case KQ_Q4_1: return "q4_1";
    case KQ_Q5_0: return "q5_0";
    case KQ_Q5_1: return "q5_1";
    case KQ_Q6_K: return "q6_k";
    default: return "?";
  }
}

bool geometry(int c, int* bv, int* bb) {
  switch (c) {
    case KQ_Q4_0: *bv = 32; *bb = 18; return true;
    case KQ_Q8_0: *bv = 32; *bb = 34; return true;
    case KQ_Q4_K: *bv = 256; *bb = 144; return true;
    case KQ_Q5_K: *bv = 256; *bb = 176; return true;
    case KQ_Q2_K: *bv = 256; *bb = 84; return true;
    case KQ_Q3_K: *bv = 256; *bb = 110; return true;
    case KQ_Q4_1: *bv = 32; *bb = 20; return true;
    case KQ_Q5_0: *bv = 32; *bb = 22; return true;
    case KQ_Q5_1: *bv = 32; *bb = 24; return true;
    case KQ_Q6_K: *bv = 256; *bb = 210; return true;
    default: return false;
  }
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxElems = (int64_t)1 << 40;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Shared checks: codec, K, row bytes.  Returns KQ_OK and fills row_bytes.
int check_codec_k(const char* op, int codec, int64_t k, int64_t* row_bytes) {
  int bv, bb;
  if (!geometry(codec, &bv, &bb)) return fail(KQ_ERR_CODEC, op, "unknown codec id %d", codec);
  if (k <= 0 || k >= kMaxDim) return fail(KQ_ERR_SHAPE, op, "K=%lld out of range", (long long)k);
  if (k % bv)
    return fail(KQ_ERR_SHAPE, op, "K=%lld is not a multiple of %d for %s", (long long)k, bv, codec_name(codec));
  *row_bytes = k / bv * bb;
  return KQ_OK;
}

int check_dtype(const char* op, int dt, bool bf16 = false) {
  if (bf16 && dt == KQ_BF16) return KQ_OK;
  if (dt != KQ_F32 && dt != KQ_F16)
    return fail(KQ_ERR_ARG, op, "output dtype %d is not KQ_F32 or KQ_F16%s", dt, bf16 ? " or KQ_BF16" : "");
  return KQ_OK;
}

int hip_status(const char* op, hipError_t e) {
  if (e != hipSuccess) return fail(KQ_ERR_HIP, op, "HIP launch failed: %s", hipGetErrorString(e));
  g_err.clear();
  return KQ_OK;
}

int check_matmul(const char* op, int codec, const void* w, int64_t n, int64_t k, const void* x, int64_t m,
                 const void* y, int y_dtype, int64_t* rb, bool bf16 = false) {
  int st = check_codec_k(op, codec, k, rb);
  if (st) return st;
  if ((st = check_dtype(op, y_dtype, bf16))) return st;
  if (n < 0 || n >= kMaxDim) return fail(KQ_ERR_ARG, op, "N=%lld out of range", (long long)n);
  if (m < 0 || m >= kMaxDim) return fail(KQ_ERR_ARG, op, "M=%lld out of range", (long long)m);
  if (n * k >= kMaxElems || m * k >= kMaxElems || m * n >= kMaxElems)
    return fail(KQ_ERR_ARG, op, "tensor too large (M=%lld N=%lld K=%lld)", (long long)m, (long long)n, (long long)k);
  if (n == 0 || m == 0) return KQ_OK;
  if (!w || !x || !y) return fail(KQ_ERR_ARG, op, "null pointer (w=%p x=%p y=%p)", w, x, y);
  if (!aligned(w, 16)) return fail(KQ_ERR_ALIGN, op, "w=%p is not 16-byte aligned", w);
  if (!aligned(x, 16)) return fail(KQ_ERR_ALIGN, op, "x=%p is not 16-byte aligned", x);
  if (!aligned(y, y_dtype == KQ_F32 ? 4 : 2)) return fail(KQ_ERR_ALIGN, op, "y=%p is not element aligned", y);
  return KQ_OK;
}

}  // namespace

extern "C" {

const char* kq_last_error(void) { return g_err.c_str(); }

const char* kq_version(void) { return "kq 0.1 (gfx950)"; }

int kq_codec_from_name(const char* name, int* codec) {
  if (!name || !codec) return fail(KQ_ERR_ARG, "kq_codec_from_name", "null argument");
  char low[16];
  size_t i = 0;
  for (; name[i] && i + 1 < sizeof low; ++i) low[i] = (char)tolower((unsigned char)name[i]);
  low[i] = 0;
  static const struct { const char* n; int c; } table[] = {
      {"q4_0", KQ_Q4_0}, {"q8_0", KQ_Q8_0}, {"q4_k", KQ_Q4_K}, {"q5_k", KQ_Q5_K}, {"q6_k", KQ_Q6_K},
      {"q4_1", KQ_Q4_1}, {"q5_0", KQ_Q5_0}, {"q5_1", KQ_Q5_1}, {"q2_k", KQ_Q2_K}, {"q3_k", KQ_Q3_K}};
  for (const auto& t : table)
    if (!name[i] && strcmp(low, t.n) == 0) {
      *codec = t.c;
      return KQ_OK;
    }
  return fail(KQ_ERR_CODEC, "kq_codec_from_name", "unknown codec '%s' (known: q4_0, q4_1, q5_0, q5_1, q8_0, q2_k, q3_k, q4_k, q5_k, q6_k)", name);
}

int kq_codec_info(int codec, int* block_values, int* block_bytes) {
  int bv, bb;
  if (!geometry(codec, &bv, &bb)) return fail(KQ_ERR_CODEC, "kq_codec_info", "unknown codec id %d", codec);
  if (block_values) *block_values = bv;
  if (block_bytes) *block_bytes = bb;
  return KQ_OK;
}

int kq_row_bytes(int codec, int64_t k, int64_t* row_bytes) {
  int64_t rb;
  int st = check_codec_k("kq_row_bytes", codec, k, &rb);
  if (st) return st;
  if (!row_bytes) return fail(KQ_ERR_ARG, "kq_row_bytes", "null output");
  *row_bytes = rb;
  return KQ_OK;
}

int kq_dequantize(int codec, const void* w, int64_t rows, int64_t k, void* out, int out_dtype, void* stream) {
  const char* op = "kq_dequantize";
  int64_t rb;
  int st = check_codec_k(op, codec, k, &rb);
  if (st) return st;
  if ((st = check_dtype(op, out_dtype))) return st;
  if (rows < 0 || rows >= kMaxDim || rows * k >= kMaxElems)
    return fail(KQ_ERR_ARG, op, "rows=%lld out of range", (long long)rows);
  if (rows == 0) return KQ_OK;
  if (!w || !out) return fail(KQ_ERR_ARG, op, "null pointer (w=%p out=%p)", w, out);
  if (!aligned(w, 16)) return fail(KQ_ERR_ALIGN, op, "w=%p is not 16-byte aligned", w);
  if (!aligned(out, 16)) return fail(KQ_ERR_ALIGN, op, "out=%p is not 16-byte aligned", out);
  return hip_status(op, kq::launch_dequantize(codec, (const uint8_t*)w, rows, k, rb, out, out_dtype == KQ_F16,
                                              (hipStream_t)stream));
}

int kq_qmv(int codec, const void* w, int64_t n, int64_t k, const void* x, int64_t m, void* y, int y_dtype,
           void* stream) {
  const char* op = "kq_qmv";
  int64_t rb;
  int st = check_matmul(op, codec, w, n, k, x, m, y, y_dtype, &rb);
  if (st) return st;
  if (m > kq::QMV_MAX_M)
    return fail(KQ_ERR_SHAPE, op, "M=%lld rows; the GEMV takes 1..%d (use kq_qmm)", (long long)m, kq::QMV_MAX_M);
  if (n == 0 || m == 0) return KQ_OK;
  return hip_status(op, kq::launch_qmv(codec, (const uint8_t*)w, n, k, rb, (const kq::half_t*)x, (int)m, y,
                                       y_dtype == KQ_F16, (hipStream_t)stream));
}

int kq_qmm(int codec, const void* w, int64_t n, int64_t k, const void* x, int64_t m, void* y, int y_dtype,
           void* stream) {
  const char* op = "kq_qmm";
  int64_t rb;
  int st = check_matmul(op, codec, w, n, k, x, m, y, y_dtype, &rb);
  if (st) return st;
  if (n == 0 || m == 0) return KQ_OK;
  return hip_status(op, kq::launch_qmm(codec, (const uint8_t*)w, n, k, rb, (const kq::half_t*)x, m, y,
                                       y_dtype == KQ_F16, (hipStream_t)stream));
}

int kq_quantized_matmul(int codec, const void* w, int64_t n, int64_t k, const void* x, int64_t m, void* y,
                        int y_dtype, void* stream) {
  // 17..64 rows: the wide matrix-core GEMV (kq_qmv takes it from 9 rows)
  if (m >= 0 && m <= kq::QMV_MAX_M) return kq_qmv(codec, w, n, k, x, m, y, y_dtype, stream);
  if (m <= kq::QMV_WIDE_MAX_M && k % 64 == 0) {
    const char* op = "kq_quantized_matmul";
    int64_t rb;
    int st = check_matmul(op, codec, w, n, k, x, m, y, y_dtype, &rb);
    if (st) return st;
    if (n == 0) return KQ_OK;
    return hip_status(op, kq::launch_qmv_wide(codec, (const uint8_t*)w, n, k, rb, (const kq::half_t*)x, (int)m, y,
                                              y_dtype == KQ_F16, (hipStream_t)stream));
  }
  return kq_qmm(codec, w, n, k, x, m, y, y_dtype, stream);
}

// [a, a + na) and [b, b + nb) share a byte
static bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

int kq_quantized_matmul_residual(int codec, const void* w, int64_t n, int64_t k, const void* x, int64_t m,
                                 const void* residual, const void* gate, int64_t gate_rows, void* y, int y_dtype,
                                 void* stream) {
  const char* op = "kq_quantized_matmul_residual";
  int64_t rb;
  int st = check_matmul(op, codec, w, n, k, x, m, y, y_dtype, &rb);
  if (st) return st;
  if (gate && (gate_rows <= 0 || gate_rows > m || (m > 0 && m % gate_rows != 0)))
    return fail(KQ_ERR_SHAPE, op, "gate_rows=%lld must divide M=%lld", (long long)gate_rows, (long long)m);
  if (n == 0 || m == 0) return KQ_OK;
  if (!residual) return fail(KQ_ERR_ARG, op, "null residual");
  const int64_t es = y_dtype == KQ_F32 ? 4 : 2;
  if (!aligned(residual, es) || (gate && !aligned(gate, es)))
    return fail(KQ_ERR_ALIGN, op, "residual/gate must be element aligned");
  const int64_t ybytes = m * n * es;
  if (residual != y && overlaps(residual, ybytes, y, ybytes))
    return fail(KQ_ERR_ARG, op, "residual overlaps y without being y");
  if (gate && overlaps(gate, gate_rows * n * es, y, ybytes)) return fail(KQ_ERR_ARG, op, "gate overlaps y");
  const kq::Epi epi{residual, gate, nullptr, gate ? (int)(m / gate_rows) : 1};
  const bool f16 = y_dtype == KQ_F16;
  const kq::half_t* xh = (const kq::half_t*)x;
  hipError_t e;
  // the dot2 GEMV body (its cost grows with M); q8_0 keeps it to 4 rows, as
  // kq_qmv does, because its decode costs the matrix-core GEMV more per byte
  const int64_t dot2_max_m = codec == KQ_Q8_0 ? 4 : 2;
  if (m <= dot2_max_m || (m <= 8 && k % 64 != 0))
    e = kq::launch_qmv_epi(codec, (const uint8_t*)w, n, k, rb, xh, (int)m, epi, y, f16, (hipStream_t)stream);
  else if (m <= kq::QMV_WIDE_MAX_M && k % 64 == 0)  // small batches: the wide matrix-core GEMV
    e = kq::launch_qmv_wide_epi(codec, (const uint8_t*)w, n, k, rb, xh, (int)m, epi, y, f16, (hipStream_t)stream);
  else
    e = kq::launch_qmm_epi(codec, (const uint8_t*)w, n, k, rb, xh, m, epi, y, f16, (hipStream_t)stream);
  return hip_status(op, e);
}

int kq_quantized_matmul_qmv_bias(int codec, const void* w, int64_t n, int64_t k, const void* x, int64_t m,
                                 const void* bias, void* y, int y_dtype, void* stream) {
  const char* op = "kq_quantized_matmul_qmv_bias";
  int64_t rb;
  int st = check_matmul(op, codec, w, n, k, x, m, y, y_dtype, &rb);
  if (st) return st;
  if (m != 1) return fail(KQ_ERR_SHAPE, op, "M=%lld rows; the bias-fused GEMV takes exactly one", (long long)m);
  if (n == 0) return KQ_OK;
  if (!bias) return fail(KQ_ERR_ARG, op, "null bias");
  const int64_t es = y_dtype == KQ_F32 ? 4 : 2;
  if (!aligned(bias, es)) return fail(KQ_ERR_ALIGN, op, "bias must be element aligned");
  if (overlaps(bias, n * es, y, n * es)) return fail(KQ_ERR_ARG, op, "bias overlaps y");
  const kq::Epi epi{nullptr, nullptr, bias, 1};
  return hip_status(op, kq::launch_qmv_epi(codec, (const uint8_t*)w, n, k, rb, (const kq::half_t*)x, 1, epi, y,
                                           y_dtype == KQ_F16, (hipStream_t)stream));
}

int kq_quantized_matmul_glu(int codec, const void* w_gate, const void* w_up, int64_t n, int64_t k, const void* x,
                            int64_t m, int act, void* y, int y_dtype, void* stream) {
  const char* op = "kq_quantized_matmul_glu";
  int64_t rb;
  int st = check_matmul(op, codec, w_gate, n, k, x, m, y, y_dtype, &rb);
  if (st) return st;
  if (act != KQ_GLU_SILU && act != KQ_GLU_GELU_TANH)
    return fail(KQ_ERR_ARG, op, "act=%d is not KQ_GLU_SILU or KQ_GLU_GELU_TANH", act);
  if (n == 0 || m == 0) return KQ_OK;
  if (!w_up) return fail(KQ_ERR_ARG, op, "null w_up");
  if (!aligned(w_up, 16)) return fail(KQ_ERR_ALIGN, op, "w_up=%p is not 16-byte aligned", w_up);
  const bool f16 = y_dtype == KQ_F16;
  const kq::half_t* xh = (const kq::half_t*)x;
  hipError_t e;
  if (m <= kq::qmv_glu_max_m(codec)) {  // one GEMV pass over both weights
    e = kq::launch_qmv_glu(codec, (const uint8_t*)w_gate, (const uint8_t*)w_up, n, k, rb, xh, (int)m, act, y, f16,
                           (hipStream_t)stream);
  } else if (m <= kq::QMV_WIDE_MAX_M && k % 64 == 0) {  // two wide matrix-core GEMV passes
    e = kq::launch_qmv_wide_glu_act(codec, (const uint8_t*)w_gate, n, k, rb, xh, (int)m, act, y, f16,
                                    (hipStream_t)stream);
    if (e == hipSuccess)
      e = kq::launch_qmv_wide_glu_mul(codec, (const uint8_t*)w_up, n, k, rb, xh, (int)m, y, f16, (hipStream_t)stream);
  } else {  // two GEMM passes
    e = kq::launch_qmm_glu(codec, (const uint8_t*)w_gate, (const uint8_t*)w_up, n, k, rb, xh, m, act, y, f16,
                           (hipStream_t)stream);
  }
  return hip_status(op, e);
}

int64_t kq_expert_tile_map_capacity(int64_t rows, int64_t n_experts) {
  if (rows < 0 || n_experts < 0) return -1;
  return (rows + 63) / 64 + (n_experts < rows ? n_experts : rows);
}

int kq_expert_tile_map(const uint32_t* ids, int64_t rows, int64_t n_experts, uint32_t* map, uint32_t* counts,
                       int64_t cap, uint32_t* status, void* stream) {
  const char* op = "kq_expert_tile_map";
  if (rows < 0 || rows >= kMaxDim) return fail(KQ_ERR_ARG, op, "rows=%lld out of range", (long long)rows);
  if (n_experts <= 0 || n_experts >= kMaxDim)
    return fail(KQ_ERR_ARG, op, "n_experts=%lld out of range", (long long)n_experts);
  const int64_t need = kq_expert_tile_map_capacity(rows, n_experts);
  if (cap < need || cap >= kMaxDim)
    return fail(KQ_ERR_CAPACITY, op, "cap=%lld is below the bound %lld for rows=%lld, n_experts=%lld",
                (long long)cap, (long long)need, (long long)rows, (long long)n_experts);
  if (!counts || (rows > 0 && (!ids || !map))) return fail(KQ_ERR_ARG, op, "null pointer");
  if (!aligned(counts, 4) || (ids && !aligned(ids, 4)) || (map && !aligned(map, 4)) || (status && !aligned(status, 4)))
    return fail(KQ_ERR_ALIGN, op, "ids/map/counts/status must be 4-byte aligned");
  return hip_status(op, kq::launch_tile_map(ids, rows, n_experts, map, counts, cap, status, (hipStream_t)stream));
}

int kq_gather_qmm_seg(int codec, const void* w, int64_t n_experts, int64_t n, int64_t k, const void* x,
                      int64_t rows, const uint32_t* map, const uint32_t* counts, int64_t cap, void* y, int y_dtype,
                      void* stream) {
  const char* op = "kq_gather_qmm_seg";
  int64_t rb;
  int st = check_matmul(op, codec, w, n, k, x, rows, y, y_dtype, &rb);
  if (st) return st;
  if (n_experts <= 0 || n_experts >= kMaxDim || n_experts * n >= kMaxDim * 64)
    return fail(KQ_ERR_ARG, op, "n_experts=%lld out of range", (long long)n_experts);
  if (cap < 0 || cap >= kMaxDim) return fail(KQ_ERR_ARG, op, "cap=%lld out of range", (long long)cap);
  if (n == 0 || rows == 0 || cap == 0) return KQ_OK;
  if (!map || !counts) return fail(KQ_ERR_ARG, op, "null map or counts");
  if (!aligned(map, 4) || !aligned(counts, 4)) return fail(KQ_ERR_ALIGN, op, "map/counts must be 4-byte aligned");
  return hip_status(op, kq::launch_gather_qmm_seg(codec, (const uint8_t*)w, n_experts, n, k, rb,
                                                  (const kq::half_t*)x, rows, map, counts, cap, y,
                                                  y_dtype == KQ_F16, (hipStream_t)stream));
}

int kq_gather_mix(const void* y, int64_t rows, int64_t n, const uint32_t* inv_order, const float* scores,
                  int64_t tokens, int64_t top_k, void* out, int dtype, void* stream) {
  const char* op = "kq_gather_mix";
  int st = check_dtype(op, dtype);
  if (st) return st;
  if (rows < 0 || rows >= kMaxDim) return fail(KQ_ERR_ARG, op, "rows=%lld out of range", (long long)rows);
  if (n < 0 || n >= kMaxDim) return fail(KQ_ERR_ARG, op, "N=%lld out of range", (long long)n);
  if (tokens < 0 || tokens >= kMaxDim) return fail(KQ_ERR_ARG, op, "tokens=%lld out of range", (long long)tokens);
  if (top_k < 0 || top_k >= kMaxDim || (top_k && tokens >= kMaxDim / top_k))
    return fail(KQ_ERR_ARG, op, "top_k=%lld out of range", (long long)top_k);
  if (n % 4) return fail(KQ_ERR_SHAPE, op, "N=%lld is not a multiple of 4", (long long)n);
  if (rows * n >= kMaxElems || tokens * n >= kMaxElems)
    return fail(KQ_ERR_ARG, op, "tensor too large (rows=%lld tokens=%lld N=%lld)", (long long)rows, (long long)tokens,
                (long long)n);
  if (n == 0 || tokens == 0) return KQ_OK;
  const int vec = 4 * (dtype == KQ_F16 ? 2 : 4);
  if (!out) return fail(KQ_ERR_ARG, op, "null out");
  if (!aligned(out, vec)) return fail(KQ_ERR_ALIGN, op, "out=%p is not aligned to 4 elements", out);
  if (top_k > 0) {
    if (!inv_order || !scores || (rows > 0 && !y)) return fail(KQ_ERR_ARG, op, "null y, inv_order or scores");
    if (y && !aligned(y, vec)) return fail(KQ_ERR_ALIGN, op, "y=%p is not aligned to 4 elements", y);
    if (!aligned(inv_order, 4) || !aligned(scores, 4))
      return fail(KQ_ERR_ALIGN, op, "inv_order/scores must be 4-byte aligned");
  }
  return hip_status(op, kq::launch_gather_mix(y, rows, n, inv_order, scores, tokens, top_k, out, dtype == KQ_F16,
                                              (hipStream_t)stream));
}

int kq_gather_qmv(int codec, const void* w, int64_t n_experts, int64_t n, int64_t k, const void* x,
                  const uint32_t* ids, int64_t rows, void* y, int y_dtype, void* stream) {
  const char* op = "kq_gather_qmv";
  int64_t rb;
  int st = check_matmul(op, codec, w, n, k, x, rows, y, y_dtype, &rb);
  if (st) return st;
  if (k % 256)
    return fail(KQ_ERR_SHAPE, op, "K=%lld is not a multiple of 256 (one activation row per slot)", (long long)k);
  if (n_experts <= 0 || n_experts >= kMaxDim || n_experts * n >= kMaxDim * 64)
    return fail(KQ_ERR_ARG, op, "n_experts=%lld out of range", (long long)n_experts);
  if (n == 0 || rows == 0) return KQ_OK;
  if (!ids) return fail(KQ_ERR_ARG, op, "null ids");
  if (!aligned(ids, 4)) return fail(KQ_ERR_ALIGN, op, "ids=%p is not 4-byte aligned", (const void*)ids);
  return hip_status(op, kq::launch_gather_qmv(codec, (const uint8_t*)w, n_experts, n, k, rb, (const kq::half_t*)x,
                                              ids, rows, y, y_dtype == KQ_F16, (hipStream_t)stream));
}

int kq_moe_glu_gather(int codec, const void* gate_w, const void* up_w, int64_t n_experts, int64_t n, int64_t k,
                      const void* x, int64_t tokens, const uint32_t* ids, int64_t top_k, int act, float limit,
                      void* y, int y_dtype, void* stream) {
  const char* op = "kq_moe_glu_gather";
  if (tokens < 0 || tokens >= kMaxDim) return fail(KQ_ERR_ARG, op, "tokens=%lld out of range", (long long)tokens);
  if (top_k < 0 || top_k >= kMaxDim || (top_k && tokens >= kMaxDim / top_k))
    return fail(KQ_ERR_ARG, op, "top_k=%lld out of range", (long long)top_k);
  const int64_t rows = tokens * top_k;
  int64_t rb;
  int st = check_matmul(op, codec, gate_w, n, k, x, rows, y, y_dtype, &rb);
  if (st) return st;
  if (k % 256)
    return fail(KQ_ERR_SHAPE, op, "K=%lld is not a multiple of 256 (one activation row per token)", (long long)k);
  if (n_experts <= 0 || n_experts >= kMaxDim || n_experts * n >= kMaxDim * 64)
    return fail(KQ_ERR_ARG, op, "n_experts=%lld out of range", (long long)n_experts);
  if (act != KQ_GLU_SILU && act != KQ_GLU_GELU_TANH && act != KQ_GLU_SILU_LIMIT)
    return fail(KQ_ERR_ARG, op, "act=%d is not a kq_glu_act", act);
  if (act == KQ_GLU_SILU_LIMIT && !(limit > 0.f && limit <= 3.0e38f))
    return fail(KQ_ERR_ARG, op, "limit=%g must be finite and > 0 for KQ_GLU_SILU_LIMIT", (double)limit);
  if (n == 0 || rows == 0) return KQ_OK;
  if (!up_w) return fail(KQ_ERR_ARG, op, "null up_w");
  if (!aligned(up_w, 16)) return fail(KQ_ERR_ALIGN, op, "up_w=%p is not 16-byte aligned", up_w);
  if (!ids) return fail(KQ_ERR_ARG, op, "null ids");
  if (!aligned(ids, 4)) return fail(KQ_ERR_ALIGN, op, "ids=%p is not 4-byte aligned", (const void*)ids);
  return hip_status(op, kq::launch_moe_glu_gather(codec, (const uint8_t*)gate_w, (const uint8_t*)up_w, n_experts, n,
                                                  k, rb, (const kq::half_t*)x, ids, rows, top_k, act, limit, y,
                                                  y_dtype == KQ_F16, (hipStream_t)stream));
}

int kq_quantize(int codec, const float* w, int64_t rows, int64_t k, void* out, void* stream) {
  const char* op = "kq_quantize";
  int64_t rb;
  int st = check_codec_k(op, codec, k, &rb);
  if (st) return st;
  if (rows < 0 || rows >= kMaxDim || rows * k >= kMaxElems)
    return fail(KQ_ERR_ARG, op, "rows=%lld out of range", (long long)rows);
  if (rows == 0) return KQ_OK;
  if (!w || !out) return fail(KQ_ERR_ARG, op, "null pointer (w=%p out=%p)", (const void*)w, out);
  if (!aligned(w, 16) || !aligned(out, 16)) return fail(KQ_ERR_ALIGN, op, "w and out must be 16-byte aligned");
  return hip_status(op, kq::launch_quantize(codec, w, rows, k, rb, (uint8_t*)out, (hipStream_t)stream));
}

int kq_stream_read(const void* src, int64_t bytes, uint32_t* out, int64_t groups, void* stream) {
  const char* op = "kq_stream_read";
  if (bytes < 0 || bytes % 16 != 0 || bytes >= kMaxElems)
    return fail(KQ_ERR_ARG, op, "bytes=%lld must be a non-negative multiple of 16", (long long)bytes);
  if (groups < 1 || groups > (1 << 20)) return fail(KQ_ERR_ARG, op, "groups=%lld out of 1..2^20", (long long)groups);
  // out holds 4 * groups words (one per wave)
  if (!src || !out) return fail(KQ_ERR_ARG, op, "null pointer (src=%p out=%p)", src, (void*)out);
  if (!aligned(src, 16) || !aligned(out, 4)) return fail(KQ_ERR_ALIGN, op, "src must be 16-byte, out 4-byte aligned");
  return hip_status(op, kq::launch_stream_read(src, bytes, out, groups, (hipStream_t)stream));
}

// ---- bfloat16 activations ----
// y dtype: KQ_F32, KQ_F16 or KQ_BF16 (2)
static int bf16_out(int y_dtype) { return y_dtype == KQ_BF16 ? 2 : y_dtype == KQ_F16 ? 1 : 0; }

int kq_qmv_bf16(int codec, const void* w, int64_t n, int64_t k, const void* x, int64_t m, void* y, int y_dtype,
                void* stream) {
  const char* op = "kq_qmv_bf16";
  int64_t rb;
  int st = check_matmul(op, codec, w, n, k, x, m, y, y_dtype, &rb, true);
  if (st) return st;
  if (m > kq::QMV_MAX_M)
    return fail(KQ_ERR_SHAPE, op, "M=%lld rows; the GEMV takes 1..%d (use kq_qmm_bf16)", (long long)m, kq::QMV_MAX_M);
  if (n == 0 || m == 0) return KQ_OK;
  return hip_status(op, kq::launch_mm_bf16(codec, (const uint8_t*)w, n, k, rb, x, m, y, bf16_out(y_dtype),
                                           (hipStream_t)stream));
}

int kq_qmm_bf16(int codec, const void* w, int64_t n, int64_t k, const void* x, int64_t m, void* y, int y_dtype,
                void* stream) {
  const char* op = "kq_qmm_bf16";
  int64_t rb;
  int st = check_matmul(op, codec, w, n, k, x, m, y, y_dtype, &rb, true);
  if (st) return st;
  if (n == 0 || m == 0) return KQ_OK;
  return hip_status(op, kq::launch_mm_bf16(codec, (const uint8_t*)w, n, k, rb, x, m, y, bf16_out(y_dtype),
                                           (hipStream_t)stream));
}

int kq_gather_qmm_seg_bf16(int codec, const void* w, int64_t n_experts, int64_t n, int64_t k, const void* x,
                           int64_t rows, const uint32_t* map, const uint32_t* counts, int64_t cap, void* y,
                           int y_dtype, void* stream) {
  const char* op = "kq_gather_qmm_seg_bf16";
  int64_t rb;
  int st = check_matmul(op, codec, w, n, k, x, rows, y, y_dtype, &rb, true);
  if (st) return st;
  if (n_experts <= 0 || n_experts >= kMaxDim || n_experts * n >= kMaxDim * 64)
    return fail(KQ_ERR_ARG, op, "n_experts=%lld out of range", (long long)n_experts);
  if (cap < 0 || cap >= kMaxDim) return fail(KQ_ERR_ARG, op, "cap=%lld out of range", (long long)cap);
  if (n == 0 || rows == 0 || cap == 0) return KQ_OK;
  if (!map || !counts) return fail(KQ_ERR_ARG, op, "null map or counts");
  if (!aligned(map, 4) || !aligned(counts, 4)) return fail(KQ_ERR_ALIGN, op, "map/counts must be 4-byte aligned");
  return hip_status(op, kq::launch_seg_bf16(codec, (const uint8_t*)w, n_experts, n, k, rb, x, rows, map, counts, cap,
                                            y, bf16_out(y_dtype), (hipStream_t)stream));
}

}  // extern "C"
