/*
 * qrp_oracle.h -- CPU oracle for the ragged RoPE / split / paged-store pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-threaded C
 * implementation of what the pass computes, written from the Modular MAX
 * kernel documentation pages it cites.  Only the test-suite, the smoke check
 * and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, helper or constant with the HIP library under qk_rope_paged_amd/,
 * and the HIP library never calls it.
 *
 * Arithmetic: every input element is widened exactly to double; RoPE and
 * RMSNorm are evaluated in double and rounded ONCE to the output dtype with
 * round-to-nearest-even (the multiply_before_cast=false branch adds the
 * intermediate roundings that flag asks for).  radd is one IEEE fp32 add.
 * Copies (V, un-roped dimensions of the rope-only op) move raw bits.
 *
 * Readings of points the pages leave open:
 *   - freqs_cis rows hold (cos, sin) pairs for frequency i at columns
 *     (2i, 2i+1) whatever the Q/K layout (the table is described as holding
 *     interleaved frequencies: rope_split_store_paged_ragged page, Args:
 *     freqs_cis);
 *   - the rotation multiplies by cos + i*sin;
 *   - half-split pairs element i with element i + rope_dim/2;
 *   - a partial rope rotates the FIRST rope_dim dimensions of a head, or
 *     with rope_tail the LAST rope_dim (parity unpinned: the pages fix no
 *     location; both conventions are offered);
 *   - position = cache_lengths[b + batch_offset] + local token index;
 *   - RMSNorm: mean of squares over the head, epsilon inside the square
 *     root, gamma + weight_offset as the scale, norm before rope;
 *   - multiply_before_cast=false: parity unpinned (named only on the
 *     fused_dual_qk_rms_norm_rope_ragged_paged page, signature);
 *   - FP8 caches (the pages name a cache collection's scale dtype and
 *     quantization granularity, nothing more): OCP E4M3 codes, one dynamic
 *     absmax scale per written head row, every decision in binary32 (see
 *     quantize_row); parity of the encoding is pinned, the granularity and
 *     scale rule are a reading (unpinned);
 *   - q_out_dtype (rope_split_store_paged_ragged page, Parameters): Q is
 *     rounded once to it; un-roped elements move as bits when it equals the
 *     input dtype and are converted (nearest-even) otherwise;
 *   - the fused GEMV + partial RMSNorm (MatmulFusedPartialRMSNorm page):
 *     n_normed is the length of gamma and of a normed row; the norm's mean
 *     runs over those n_normed columns only; epsilon sits inside the root,
 *     as in the other RMSNorm ops; several input rows are independent.
 */
#ifndef QRP_ORACLE_H
#define QRP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F16 = 2, ORC_FP8 = 3 /* e4m3 codes: caches only */ };

enum {
  ORC_OK = 0,
  ORC_EINVAL = -1,   /* bad argument */
  ORC_EDATA = -6     /* metadata out of range (position, page, offsets) */
};

/* A paged K/V cache as the oracle sees it (host memory).  dtype is the op's
 * dtype, or ORC_FP8: then every (page, plane, layer, slot, head) row of D
 * codes has one scale, at the s_* strides in `scales` (ORC_F32 or ORC_BF16
 * values); a row's value j is code_j * scale in binary32. */
typedef struct orc_cache {
  void* pool;                 /* elements of `dtype` */
  int32_t dtype;
  uint32_t num_kv_heads;
  uint32_t head_dim;
  uint32_t page_size;
  uint32_t kv_planes;         /* 2: K and V planes; 1: K only */
  uint32_t num_layers;
  uint64_t num_pages;
  /* element strides */
  int64_t page_stride, plane_stride, layer_stride, slot_stride, head_stride;
  const uint32_t* cache_lengths;   /* [cache_batch] */
  const uint32_t* lookup_table;    /* [cache_batch][max_pages_per_seq] */
  uint32_t cache_batch;
  uint32_t max_pages_per_seq;
  void* scales;               /* ORC_FP8 only, else NULL */
  int32_t scale_dtype;
  int64_t s_page_stride, s_plane_stride, s_layer_stride, s_slot_stride, s_head_stride;
} orc_cache;

/* Optional record of the unrounded results, for tolerance checks.
 * Any pointer may be NULL.  Shapes: q_* [T][n_q_heads][head_dim],
 * k_* [T][num_kv_heads][head_dim], *_row_off [T][num_kv_heads]. */
typedef struct orc_trace {
  double* q_exact;     /* value before the final rounding */
  double* q_mag;       /* hypot of its RoPE pair (roped dims) or |value| */
  double* k_exact;
  double* k_mag;
  int64_t* k_row_off;  /* pool element offset of each K row written */
  int64_t* v_row_off;  /* pool element offset of each V row written */
  int64_t* k_scale_off; /* FP8 caches: scale offset of each K row written */
  int64_t* v_scale_off;
  /* Normalised roles only: x_j * r, the normalised value before any
   * rounding (with multiply_before_cast=false it is the value the first
   * rounding to dtype takes).  Shapes as q_exact / k_exact. */
  double* q_pre;
  double* k_pre;
} orc_trace;

/* One band of the norm+rope op. */
typedef struct orc_band {
  uint64_t q_col;          /* first column of the band's Q heads in the buffer */
  uint32_t n_q_heads;
  int64_t k_col;           /* first K column in the buffer; < 0: K is read from the cache */
  int64_t v_col;           /* first V column; < 0: no V */
  const void* q_gamma;     /* [head_dim] of dtype, NULL: no norm on Q */
  const void* k_gamma;     /* [head_dim] of dtype, NULL: no norm on K */
  float epsilon;
  orc_cache* cache;
  void* q_output;          /* dtype, row stride q_out_row_stride */
  uint64_t q_out_row_stride;
} orc_band;

/* Exact double -> bf16 bits, round to nearest even. */
uint16_t orc_round_bf16(double x);
double orc_bf16_to_double(uint16_t b);

/* Exact double -> IEEE binary16 bits, round to nearest even. */
uint16_t orc_round_f16(double x);
double orc_f16_to_double(uint16_t h);

/* OCP FP8 E4M3 (finite-only variant): nearest-even, magnitudes past 448
 * saturate to 448, NaN -> 0x7F with the sign kept. */
uint8_t orc_round_e4m3(double x);
double orc_e4m3_to_double(uint8_t q);

/* rope_split_store_paged_ragged page (signature, Summary, Args). */
int32_t orc_rope_split_store_paged(
    const void* qkv, int32_t dtype, uint32_t total_seq_len, uint64_t qkv_row_stride,
    uint32_t n_q_heads, const uint32_t* input_row_offsets, uint32_t batch_size,
    const float* freqs_cis, uint32_t max_seq_len, uint32_t rope_dim, int32_t interleaved,
    int32_t rope_tail, orc_cache* cache, uint32_t layer_idx, void* q_output, int32_t q_out_dtype,
    uint64_t q_out_row_stride, orc_trace* trace);

/* Single-band fused per-head RMSNorm + RoPE (fused_dual_qk_rms_norm_rope_ragged_paged
 * page, Summary and Description). */
int32_t orc_qk_rmsnorm_rope_paged(
    const void* buf, int32_t dtype, uint32_t total_seq_len, uint64_t buf_row_stride,
    const orc_band* band, float weight_offset, int32_t multiply_before_cast,
    const uint32_t* input_row_offsets, uint32_t batch_size,
    const float* freqs_cis, uint32_t max_seq_len, uint32_t rope_dim, int32_t interleaved,
    int32_t rope_tail, uint32_t layer_idx, orc_trace* trace);

/* Dual band: the main band then the index band, same offsets and freqs. */
int32_t orc_dual_band(
    const void* buf, int32_t dtype, uint32_t total_seq_len, uint64_t buf_row_stride,
    const orc_band* main_band, const orc_band* index_band, float weight_offset,
    int32_t multiply_before_cast, const uint32_t* input_row_offsets, uint32_t batch_size,
    const float* freqs_cis, uint32_t max_seq_len, uint32_t rope_dim, int32_t interleaved,
    int32_t rope_tail, uint32_t layer_idx, orc_trace* main_trace, orc_trace* index_trace);

/* generic_kv_cache_radd_dispatch page (Summary, Description, Args). */
int32_t orc_kv_cache_radd(
    const void* a, int32_t dtype, uint32_t total_rows, uint64_t a_row_stride,
    const uint32_t* input_row_offsets, uint32_t batch_size, uint32_t batch_offset,
    orc_cache* cache, uint32_t layer_idx, orc_trace* trace);

/* generic_fused_qk_rope_bshd_continuous_batch page (signature, Args):
 * q_proj and output [B][S][n_q_heads][head_dim], valid_lengths [B]; the
 * cache's sequence b is batch row b (a continuous-batching cache is the
 * one-page-per-sequence case).  Rows s >= valid_lengths[b] pass through
 * (output = input bits, cache untouched: parity unpinned, the page only
 * says RoPE is confined to the valid rows). */
int32_t orc_fused_qk_rope_bshd(const void* q_proj, int32_t dtype, uint32_t batch_size,
                               uint32_t seq_len, uint32_t n_q_heads,
                               const uint32_t* valid_lengths, const float* freqs_cis,
                               uint32_t max_seq_len, uint32_t rope_dim, int32_t interleaved,
                               int32_t rope_tail, orc_cache* cache, uint32_t layer_idx,
                               void* output,
                               orc_trace* trace);

/* MatmulFusedPartialRMSNorm page (Summary, execute, Args): per input row i,
 * y = x_i W^T with W stored [n][k] (transpose_b != 0, the page's default),
 * or y = x_i W with W stored [k][n] (transpose_b == 0; weight_row_stride is
 * then the stride of W's k rows), then the
 * first n_normed columns of y are RMS-normalised as one vector,
 *   normed[i][j] = y_j / sqrt(mean_{j < n_normed} y_j^2 + epsilon) * gamma_j,
 * and the other n - n_normed columns pass through:
 *   unnormed[i][j - n_normed] = y_j.
 * y is exact up to double rounding; each output is rounded once to dtype.
 * weight_offset is taken and not used (Args: weight_offset).  The page names
 * a GEMV (one input row); several rows are handled one after another.
 * Optional traces: y_exact and abs_dot [m][n] (y, and sum_k |x_k w_jk|),
 * r_out [m] (the row's reciprocal root; 0 when n_normed is 0). */
int32_t orc_matmul_fused_partial_rmsnorm(
    void* normed_output, uint64_t normed_row_stride, void* unnormed_output,
    uint64_t unnormed_row_stride, const void* input, uint64_t input_row_stride, uint32_t m,
    const void* weight, uint64_t weight_row_stride, uint32_t n, uint32_t k, const void* gamma,
    uint32_t n_normed, float epsilon, float weight_offset, int32_t dtype, int32_t transpose_b,
    double* y_exact, double* abs_dot, double* r_out);

#ifdef __cplusplus
}
#endif

#endif /* QRP_ORACLE_H */
