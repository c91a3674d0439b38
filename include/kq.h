/*
 * kq.h -- C ABI of libkq: GGUF K-quant dequantize and quantized matmul on
 * AMD Instinct MI355X (gfx950).
 *
 * Operations follow the mlx-kquant ops as documented on the mlx-kquant
 * bindings.cpp page (docstrings of dequantize, quantized_matmul,
 * expert_tile_map, gather_qmm_seg, gather_qmv_kq, quantize) and the codec
 * geometry of the mlx-kquant README ("Codec reference" table).  Byte layouts
 * inside a block are GGUF's.
 *
 * Conventions shared by every entry point
 *  - Pointers named w, x, y, out, map, counts, ids, status are DEVICE
 *    pointers; the caller owns every buffer.  The library allocates no device
 *    memory and keeps no state except a thread-local error message.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work on that stream; none synchronizes the
 *    device or the host.
 *  - Weights are the codec's wire bytes, row-major [rows][row_bytes] with
 *    row_bytes = K / block_values * block_bytes (the quantized_matmul
 *    docstring's transpose=True layout: one weight row per output column).
 *    The "scales" argument of the pages' ops is vestigial (their docstrings
 *    say the kernel ignores it) and is absent here.
 *  - Activations x are float16, row-major [M][K].
 *  - w and x must be 16-byte aligned, y/out 16-byte aligned, map/counts/ids
 *    4-byte aligned: otherwise KQ_ERR_ALIGN.
 *  - K must be a positive multiple of the codec's block (256 for the
 *    K-quants q2_K .. q6_K, 32 for the others): otherwise KQ_ERR_SHAPE.  Sizes must be
 *    below 2^31 (element counts below 2^40).
 *  - On any error nothing is launched and outputs are untouched; the return
 *    value is a kq_status and kq_last_error() describes it.
 *  - Calls on one stream are ordered; calls on different streams that write
 *    the same output race.
 */
#ifndef KQ_H
#define KQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Codec ids: GGML's type numbers for these codecs (the names are the
 * authority: "q4_0", "q4_1", "q5_0", "q5_1", "q8_0", "q4_k", "q5_k",
 * "q2_k", "q3_k", "q6_k").  Geometry per the mlx-kquant README "Codec reference" table:
 *   q4_0  32 values,  4 bits,  18 bytes per block (scale)
 *   q4_1  32 values,  4 bits,  20 bytes per block (scale + min)
 *   q5_0  32 values,  5 bits,  22 bytes per block (scale)
 *   q5_1  32 values,  5 bits,  24 bytes per block (scale + min)
 *   q8_0  32 values,  8 bits,  34 bytes per block
 *   q2_K 256 values,  2 bits,  84 bytes per superblock
 *   q3_K 256 values,  3 bits, 110 bytes per superblock
 *   q4_K 256 values,  4 bits, 144 bytes per superblock
 *   q5_K 256 values,  5 bits, 176 bytes per superblock
 *   q6_K 256 values,  6 bits, 210 bytes per superblock */
typedef enum {
  KQ_Q4_0 = 2, KQ_Q4_1 = 3, KQ_Q5_0 = 6, KQ_Q5_1 = 7, KQ_Q8_0 = 8,
  KQ_Q2_K = 10, KQ_Q3_K = 11, KQ_Q4_K = 12, KQ_Q5_K = 13, KQ_Q6_K = 14
} kq_codec;

/* Output element types (KQ_BF16: the bfloat16-activation entry points only). */
typedef enum { KQ_F32 = 0, KQ_F16 = 1, KQ_BF16 = 2 } kq_dtype;

/* GLU epilogues of kq_moe_glu_gather and kq_quantized_matmul_glu (the pages'
 * act names in comments; kq_quantized_matmul_glu takes the first two). */
typedef enum {
  KQ_GLU_SILU = 0,       /* 'silu':       silu(g) * u                          */
  KQ_GLU_GELU_TANH = 1,  /* 'gelu':       gelu(g) * u, tanh form               */
  KQ_GLU_SILU_LIMIT = 2  /* 'silu_limit': silu(min(g, L)) * clip(u, -L, L)     */
} kq_glu_act;

typedef enum {
  KQ_OK = 0,
  KQ_ERR_ARG = -1,      /* null pointer, bad dtype, size out of range       */
  KQ_ERR_CODEC = -2,    /* unknown codec id or name                          */
  KQ_ERR_SHAPE = -3,    /* K not a multiple of the block, M out of range     */
  KQ_ERR_ALIGN = -4,    /* pointer not aligned as required                   */
  KQ_ERR_CAPACITY = -5, /* tile-map capacity below kq_expert_tile_map_capacity */
  KQ_ERR_HIP = -6       /* a HIP launch failed; message has the HIP error    */
} kq_status;

/* ---- codec registry (mlx-kquant bindings.cpp page: codecs(); README codec table) ---- */

/* Name -> codec id: "q4_0", "q4_1", "q5_0", "q5_1", "q8_0", "q2_k", "q3_k",
 * "q4_k", "q5_k", "q6_k" (case-insensitive); KQ_ERR_CODEC otherwise. */
int kq_codec_from_name(const char* name, int* codec);
/* Values and bytes per block of a codec. */
int kq_codec_info(int codec, int* block_values, int* block_bytes);
/* Bytes of one weight row of K values. */
int kq_row_bytes(int codec, int64_t k, int64_t* row_bytes);
/* Message of the last failed call on this thread ("" if none). */
const char* kq_last_error(void);
/* Library version string. */
const char* kq_version(void);

/* ---- dequantize (mlx-kquant bindings.cpp page, dequantize docstring) ----
 * w [rows][row_bytes] -> out [rows][K] as float32 or float16.
 * Bit-exact: each value is the codec formula evaluated exactly and rounded
 * once to float32 (q4_K: (d*sc)*q - dmin*m; q6_K: (d*sc)*(q-32);
 * q8_0: d*q; q4_0: d*(q-8)); float16 output is RNE of that float32 value. */
int kq_dequantize(int codec, const void* w, int64_t rows, int64_t k,
                  void* out, int out_dtype, void* stream);

/* ---- quantized matmul (mlx-kquant bindings.cpp page, quantized_matmul docstring) ----
 * y[m][n] = sum_k x[m][k] * dequant(w)[n][k], float32 accumulation.
 * w [N][row_bytes], x float16 [M][K], y [M][N] float32 or float16.
 *
 * kq_qmv: decode-shaped GEMV, 1 <= M <= 16 (one weight read serves all M rows;
 *         3 or more rows run on the matrix cores).
 * kq_qmm: prefill GEMM on f16 matrix cores, any M >= 1.
 * kq_quantized_matmul: kq_qmv for M <= 16; for 17 <= M <= 64 with K a
 *         multiple of 64, the matrix-core GEMV that kq_qmv uses from 9 rows,
 *         with each decoded weight operand meeting two or four 16-row
 *         activation operands; else kq_qmm.
 * The K-reduction order is fixed per (codec, N, K, M): results are
 * deterministic run to run, and a row's result does not depend on the other
 * rows of x. */
int kq_qmv(int codec, const void* w, int64_t n, int64_t k,
           const void* x, int64_t m, void* y, int y_dtype, void* stream);
int kq_qmm(int codec, const void* w, int64_t n, int64_t k,
           const void* x, int64_t m, void* y, int y_dtype, void* stream);
int kq_quantized_matmul(int codec, const void* w, int64_t n, int64_t k,
                        const void* x, int64_t m, void* y, int y_dtype, void* stream);

/* ---- fused epilogues (mlx-kquant bindings.cpp page: quantized_matmul_residual,
 *      quantized_matmul_qmv_bias and quantized_matmul_glu docstrings) ----
 * The product p[m][n] of kq_quantized_matmul (same w, x, M, N, K rules)
 * finished in the store, in float32, rounded once to y_dtype.  The residual
 * and bias run on the dot2 GEMV body for M <= 2 (M <= 8 when K is not a
 * multiple of 64), on the matrix-core GEMVs up to M = 64 with K a multiple
 * of 64, else on the GEMM:
 *
 * kq_quantized_matmul_residual:  y = residual + gate * p.
 *   residual [M][N] and gate [gate_rows][N] are in y_dtype; output row m takes
 *   gate row m / (M / gate_rows), so gate_rows = 1 is one gate for every row
 *   and gate_rows = B is one row per batch of M / B rows.  gate = NULL drops
 *   the gate (y = residual + p; gate_rows is then ignored).  gate_rows must
 *   divide M (KQ_ERR_SHAPE).  residual may be y itself (updated in place);
 *   otherwise residual and gate must not overlap y (KQ_ERR_ARG).
 * kq_quantized_matmul_qmv_bias:  y = p + bias, decode only: M must be 1
 *   (KQ_ERR_SHAPE otherwise).  bias [N] in y_dtype, not overlapping y.
 * kq_quantized_matmul_glu:  y = act(x @ dequant(w_gate)^T) * (x @ dequant(w_up)^T)
 *   with act KQ_GLU_SILU or KQ_GLU_GELU_TANH (KQ_ERR_ARG otherwise).  w_gate
 *   and w_up have the same codec and shape (they may be row slices of one
 *   wider weight).  The activation of the gate product is rounded to y_dtype,
 *   then multiplied by the up product in float32 and rounded again; a
 *   float16 store turns a finite value beyond the float16 range into the
 *   largest finite half of its sign (infinities and NaN pass).  M <= 3
 *   (q3_K: M = 1) runs both weights through one GEMV pass; larger M runs two
 *   passes on the stream (gate, then up), with y as the only buffer between
 *   them: on the wide matrix-core GEMV for M <= 64 with K a multiple of 64,
 *   else on the GEMM.
 *
 * Element alignment for residual, gate and bias; the rest as in
 * kq_quantized_matmul. */
int kq_quantized_matmul_residual(int codec, const void* w, int64_t n, int64_t k,
                                 const void* x, int64_t m, const void* residual,
                                 const void* gate, int64_t gate_rows, void* y,
                                 int y_dtype, void* stream);
int kq_quantized_matmul_qmv_bias(int codec, const void* w, int64_t n, int64_t k,
                                 const void* x, int64_t m, const void* bias, void* y,
                                 int y_dtype, void* stream);
int kq_quantized_matmul_glu(int codec, const void* w_gate, const void* w_up, int64_t n,
                            int64_t k, const void* x, int64_t m, int act, void* y,
                            int y_dtype, void* stream);

/* ---- expert tile map (mlx-kquant bindings.cpp page, expert_tile_map docstring) ----
 * From expert ids sorted ascending (uint32 [rows]), write tiles
 * map[t] = (expert, row_start, num_rows) that cut each expert's segment into
 * 64-row tiles, only the last tile of a segment partial, and counts[0] = the
 * number of valid tiles.  Built on the GPU: no host sync.  Tiles are written
 * in expert-major order; slots past counts[0] are left as they were.
 * Ids >= n_experts get no tile (their rows stay uncovered).
 * cap (rows of map) must be >= kq_expert_tile_map_capacity(rows, n_experts).
 * status (nullable device word) is overwritten with: bit0 = ids not sorted,
 * bit1 = an id >= n_experts, bit2 = tiles exceeded cap (only possible with
 * unsorted ids; counts[0] is then clamped to cap). */
int64_t kq_expert_tile_map_capacity(int64_t rows, int64_t n_experts);
int kq_expert_tile_map(const uint32_t* sorted_ids, int64_t rows, int64_t n_experts,
                       uint32_t* map, uint32_t* counts, int64_t cap,
                       uint32_t* status, void* stream);

/* ---- expert-sorted gather GEMM (mlx-kquant bindings.cpp page, gather_qmm_seg docstring) ----
 * w [n_experts][N][row_bytes]; x float16 [rows][K], rows sorted by expert;
 * map/counts as written by kq_expert_tile_map (device memory, read on the
 * device: no host sync).  For each valid tile (e, s, c):
 *   y[r][n] = sum_k x[r][k] * dequant(w[e])[n][k]   for s <= r < s+c.
 * Rows no valid tile covers are left unwritten.  Tiles with e >= n_experts,
 * num_rows outside 1..64 or rows past `rows` are skipped.  Valid tiles must
 * not overlap (the pages' contract); overlapping tiles race. */
int kq_gather_qmm_seg(int codec, const void* w, int64_t n_experts, int64_t n, int64_t k,
                      const void* x, int64_t rows,
                      const uint32_t* map, const uint32_t* counts, int64_t cap,
                      void* y, int y_dtype, void* stream);

/* ---- bfloat16 activations (mlx-kquant bindings.cpp page: quantized_matmul
 *      and gather_qmm_seg return x's dtype, float32 promoted to bfloat16) ----
 * kq_qmv_bf16, kq_qmm_bf16 and kq_gather_qmm_seg_bf16 are kq_qmv, kq_qmm and
 * kq_gather_qmm_seg with x bfloat16 [M][K] (16-byte aligned); y_dtype is
 * KQ_F32, KQ_F16 or KQ_BF16 (the store rounds once, to nearest even).  Same
 * shapes, map semantics and errors as the float16 calls (kq_qmv_bf16:
 * 1 <= M <= 16).  On the matrix cores the activations are exact and each
 * weight enters as the sum of two bfloat16 terms holding 16 significant
 * bits of its exact value (relative error below 2^-16); accumulation is
 * float32. */
int kq_qmv_bf16(int codec, const void* w, int64_t n, int64_t k,
                const void* x, int64_t m, void* y, int y_dtype, void* stream);
int kq_qmm_bf16(int codec, const void* w, int64_t n, int64_t k,
                const void* x, int64_t m, void* y, int y_dtype, void* stream);
int kq_gather_qmm_seg_bf16(int codec, const void* w, int64_t n_experts, int64_t n, int64_t k,
                           const void* x, int64_t rows,
                           const uint32_t* map, const uint32_t* counts, int64_t cap,
                           void* y, int y_dtype, void* stream);

/* ---- unsort and score mix (mlx-kquant bindings.cpp page, gather_mix
 * docstring) ----
 * After a sorted-prefill MoE: y [rows][N] holds the expert outputs in
 * routing-sorted row order, inv_order uint32 [tokens * top_k] the sorted row
 * of each (token, slot), scores float32 [tokens][top_k] the routing weights.
 *   out[t][n] = sum_{s < top_k} scores[t][s] * y[inv_order[t * top_k + s]][n]
 * summed over s in order in float32, rounded once to `dtype` (y and out share
 * it: KQ_F16 or KQ_F32).  A slot whose inv_order entry is not below `rows`
 * adds nothing (entries are read on the device).  N must be a multiple of 4,
 * else KQ_ERR_SHAPE; y and out aligned to 4 elements, inv_order and scores
 * to 4 bytes. */
int kq_gather_mix(const void* y, int64_t rows, int64_t n, const uint32_t* inv_order,
                  const float* scores, int64_t tokens, int64_t top_k, void* out,
                  int dtype, void* stream);

/* ---- gathered GEMV (mlx-kquant bindings.cpp page, gather_qmv_kq docstring) ----
 * The decode-shaped MoE product: one activation row per (token, slot).
 * w [n_experts][N][row_bytes]; x float16 [rows][K] (the pages' [T, R, K]
 * flattened); ids uint32 [rows] (device memory, any order).  For each row r
 * with ids[r] < n_experts:
 *   y[r][n] = sum_k x[r][k] * dequant(w[ids[r]])[n][k]
 * float32 accumulation.  Rows with ids[r] >= n_experts are left unwritten
 * (ids are read on the device, not checked on the host).  K must be a
 * multiple of 256 (the pages' constraint), else KQ_ERR_SHAPE; ids 4-byte
 * aligned.  The pages' bias (for other codecs) and LoRA arguments are not
 * supported. */
int kq_gather_qmv(int codec, const void* w, int64_t n_experts, int64_t n, int64_t k,
                  const void* x, const uint32_t* ids, int64_t rows,
                  void* y, int y_dtype, void* stream);

/* ---- MoE GLU gather (mlx-kquant bindings.cpp page, moe_glu_gather_kq
 * docstring) ----
 * The decode-shaped MoE gate/up pair with its GLU epilogue in one launch.
 * gate_w, up_w [n_experts][N][row_bytes] (same codec and shape); x float16
 * [tokens][K], one activation row per token shared by its top_k slots; ids
 * uint32 [tokens][top_k] (device memory).  For slot r = t * top_k + j with
 * e = ids[r] < n_experts:
 *   g = sum_k x[t][k] * dequant(gate_w[e])[n][k]
 *   u = sum_k x[t][k] * dequant(up_w[e])[n][k]
 *   y[r][n] = act(g, u)
 * float32 accumulation and epilogue; y [tokens * top_k][N] (the pages'
 * [T, R, N]).  act is a kq_glu_act; limit is the clamp bound L of
 * KQ_GLU_SILU_LIMIT (finite and > 0, else KQ_ERR_ARG; ignored by the other
 * two).  silu(v) = v / (1 + exp(-v)); gelu in its tanh form
 * 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))).  Slots with
 * ids[r] >= n_experts are left unwritten.  K must be a multiple of 256, else
 * KQ_ERR_SHAPE; ids 4-byte aligned.  The pages' 'swiglu_clamp' act and its
 * biases belong to the mxfp4/nvfp4 layouts and are not offered. */
int kq_moe_glu_gather(int codec, const void* gate_w, const void* up_w, int64_t n_experts,
                      int64_t n, int64_t k, const void* x, int64_t tokens,
                      const uint32_t* ids, int64_t top_k, int act, float limit,
                      void* y, int y_dtype, void* stream);

/* ---- encoder (mlx-kquant bindings.cpp page, quantize docstring; no imatrix) ----
 * float32 w [rows][K] -> wire bytes out [rows][row_bytes], round to nearest
 * against the stored fp16 block parameters, every step in IEEE float32 in a
 * fixed order, each code then moved to the nearest point of its block's
 * decoded grid (distance in float64, ties to the lower code). */
int kq_quantize(int codec, const float* w, int64_t rows, int64_t k,
                void* out, void* stream);

/* ---- measurement helper: plain read of device memory ----
 * Reads `bytes` (a multiple of 16) at src with nontemporal 16-byte loads,
 * split over `groups` workgroups (1..2^20) of four waves that each read one
 * contiguous share; wave v of group g writes the XOR of the words it read to
 * out[4 g + v], so out (device, 4-byte aligned, caller-owned) holds
 * 4 * groups words.  It moves a GEMV's weight bytes with no decode,
 * which gives the measured read ceiling the GEMV rates are set against (the
 * mlx-kquant README calls decode weight-read bound). */
int kq_stream_read(const void* src, int64_t bytes, uint32_t* out, int64_t groups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
