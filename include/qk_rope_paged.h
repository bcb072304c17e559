/*
 * qk_rope_paged.h -- C ABI of the MI355X (gfx950) ragged RoPE / split /
 * paged-KV-store library.
 *
 * The operations are the ones the Modular MAX kernel documentation describes
 * for a ragged batch right after an attention block's QKV projection:
 *
 *   rope_split_store_paged   "rope_split_store_paged_ragged" page
 *   qk_rmsnorm_rope_paged    the single-band op named in the Summary of the
 *                            "fused_dual_qk_rms_norm_rope_ragged_paged" page
 *   dual_band                "fused_dual_qk_rms_norm_rope_ragged_paged" page
 *   kv_cache_radd            "generic_kv_cache_radd_dispatch" page
 *   fused_qk_rope_bshd_continuous_batch
 *                            "generic_fused_qk_rope_bshd_continuous_batch" page
 *   matmul_fused_partial_rmsnorm
 *                            "MatmulFusedPartialRMSNorm" page (the GEMV that
 *                            feeds such a pass, with a partial RMSNorm)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership    The caller allocates and owns every buffer.  The library
 *              allocates no device memory, keeps no pointer after a call
 *              returns and holds no global state apart from a thread-local
 *              error string and the launch-shape overrides (set by
 *              qrp_set_launch_override).  The one op that needs scratch memory
 *              (matmul_fused_partial_rmsnorm) takes a caller-owned
 *              workspace; its _noalloc form uses a fixed device array of
 *              the library's own instead.
 * Asynchrony   Each call checks its host-visible arguments, enqueues ONE
 *              kernel on `stream` (a hipStream_t passed as void*; NULL is the
 *              null stream) and returns without synchronising.
 * Metadata     input_row_offsets, cache_lengths and lookup_table are device
 *              arrays the library does not read on the host.  The caller
 *              guarantees them; qrp_validate() checks them on demand.  A
 *              token whose metadata is out of range (position >= max_seq_len,
 *              page index >= max_pages_per_seq, page id >= num_pages,
 *              offsets not covering it) is skipped by the kernel: nothing is
 *              read out of bounds and nothing is written for that token.
 * Layout       Row-major.  A head row is head_dim contiguous elements.  All
 *              strides are in ELEMENTS.  Buffers and row/cache strides must
 *              be 16-byte aligned (QRP_EALIGN otherwise).
 * Rounding     Arithmetic is binary32; results are rounded to the storage
 *              dtype with round-to-nearest-even.  Values that are only moved
 *              (V rows, un-roped dimensions of the rope-only op) keep every
 *              bit.  Denormals are kept.
 * Errors       Every call returns a qrp_status; qrp_last_error() gives text
 *              for the last failure on the calling thread.
 * Degenerate   total_seq_len == 0 returns QRP_OK without a launch.
 * Size         One launch holds fewer than 2^31 work items (tokens times
 *              pass groups, or token blocks times pass groups); a larger
 *              batch returns QRP_EINVAL and is split by the caller.
 * Aliasing     Outputs must not overlap inputs or each other, except the
 *              in-place cache updates the operation defines.  Two written
 *              rows must not share a cache slot.
 */
#ifndef QK_ROPE_PAGED_H
#define QK_ROPE_PAGED_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QRP_ABI_VERSION 8

typedef enum qrp_status {
  QRP_OK = 0,
  QRP_EINVAL = -1,       /* null pointer, bad size or index */
  QRP_EALIGN = -2,       /* pointer or stride not 16-byte aligned */
  QRP_EUNSUPPORTED = -3, /* dtype / head_dim / rope_dim combination not built */
  QRP_EGEOMETRY = -4,    /* dual band: the two bands' RoPE geometry differs */
  QRP_EHIP = -5,         /* the HIP runtime reported an error */
  QRP_EDATA = -6         /* qrp_validate: metadata inconsistent */
} qrp_status;

typedef enum qrp_dtype {
  QRP_F32 = 0,   /* IEEE binary32 */
  QRP_BF16 = 1,  /* bfloat16: the top 16 bits of a binary32 */
  QRP_F16 = 2,   /* IEEE binary16 */
  QRP_FP8 = 3    /* OCP FP8 E4M3 codes with a scale per row: caches only */
} qrp_dtype;

/*
 * A paged K/V cache collection (rope_split_store_paged_ragged page, Args:
 * kv_collection; fused_dual_qk_rms_norm_rope_ragged_paged page, signature:
 * per-collection static params, page size and cache dtype).
 *
 * Element (page, plane, layer, slot, head, d) lives at
 *   blocks + page*page_stride + plane*plane_stride + layer*layer_stride
 *          + slot*slot_stride + head*head_stride + d
 * Plane 0 holds K, plane 1 holds V (kv_planes == 1: a K-only cache).
 * Sequence s (s < cache_batch) stores its position p in row p % page_size of
 * page lookup_table[s * max_pages_per_seq + p / page_size].
 * blocks is device memory; cache_lengths [cache_batch] and lookup_table
 * [cache_batch * max_pages_per_seq] are device arrays of uint32.
 *
 * dtype QRP_FP8 (the collection's scale dtype and quantization granularity:
 * rope_split_store_paged_ragged page, Args: kv_collection; named there, not
 * defined -- this library's reading): every (page, plane, layer, slot,
 * head) row holds head_dim OCP E4M3 codes and has one scale at
 *   scales + page*scale_page_stride + plane*scale_plane_stride
 *          + layer*scale_layer_stride + slot*scale_slot_stride
 *          + head*scale_head_stride
 * of scale_dtype (QRP_F32 or QRP_BF16); the row's values are code * scale.
 * A row written by an op is quantized from its binary32 values v: amax =
 * max |v|, scale = amax / 448 (rounded to scale_dtype), codes = nearest-even
 * of clamp(v * (1 / scale), -448, 448) (all zero for an all-zero row); V
 * rows are quantized too.  Values must be finite.  Other cache dtypes must
 * equal the op's dtype and leave `scales` NULL.
 */
typedef struct qrp_paged_cache {
  void* blocks;
  int32_t dtype;               /* the op's dtype, or QRP_FP8 */
  uint32_t num_kv_heads;
  uint32_t head_dim;           /* 64, 128 or 256 */
  uint32_t page_size;          /* > 0 */
  uint32_t num_layers;
  uint32_t kv_planes;          /* 2: K and V; 1: K only */
  uint64_t num_pages;
  int64_t page_stride, plane_stride, layer_stride, slot_stride, head_stride;
  const uint32_t* cache_lengths;
  const uint32_t* lookup_table;
  uint32_t cache_batch;
  uint32_t max_pages_per_seq;
  void* scales;                /* QRP_FP8: device array of scale_dtype, else NULL */
  int32_t scale_dtype;         /* QRP_F32 or QRP_BF16 */
  int64_t scale_page_stride, scale_plane_stride, scale_layer_stride, scale_slot_stride,
      scale_head_stride;       /* in scale elements */
} qrp_paged_cache;

/*
 * The RoPE table (rope_split_store_paged_ragged page, Args: freqs_cis;
 * Parameters: freq_dtype, interleaved).  freqs_cis is a device array
 * [max_seq_len][rope_dim] whose entries (2i, 2i+1) hold cos and sin of
 * frequency i at that position.  rope_dim <= head_dim; the first rope_dim
 * dimensions of a head are rotated and the rest pass through (the width of
 * the table fixes rope_dim: fused_dual_qk_rms_norm_rope_ragged_paged page,
 * Description); with rope_tail = 1 the LAST rope_dim dimensions rotate
 * instead (the pages do not say which; both conventions are offered), and
 * the pairs are formed within those dims in the same two layouts.  interleaved != 0 pairs dims (2i, 2i+1); interleaved == 0
 * (half-split) pairs dims (i, i + rope_dim/2).  A pair (x, y) becomes
 * (x cos - y sin, x sin + y cos).  rope_dim must be a multiple of
 * 16 bytes / sizeof(dtype) * 2 (16 for bf16 and f16, 8 for f32).
 * freq_dtype QRP_BF16 / QRP_F16 store each entry as a bfloat16 / binary16
 * (the table's dtype is a parameter of its own on the page, independent of
 * the op's dtype); its values are widened exactly to binary32 before use.
 */
typedef struct qrp_rope {
  const void* freqs_cis;
  int32_t freq_dtype;          /* QRP_F32, QRP_BF16 or QRP_F16 (any op dtype) */
  uint32_t max_seq_len;
  uint32_t rope_dim;
  int32_t interleaved;
  int32_t rope_tail;           /* 0: the first rope_dim dims rotate; 1: the last rope_dim */
} qrp_rope;

/*
 * One band of the fused per-head RMSNorm + RoPE op
 * (fused_dual_qk_rms_norm_rope_ragged_paged page, signature and
 * Description: per band a cache, a gamma per role, an epsilon, a DPS output
 * and a Q reader).  The Q reader is affine: head h of token t starts at
 * column q_col + h*head_dim of row t of the input buffer.
 *   k_col >= 0 : K heads are read from columns k_col.. of the buffer and
 *                stored into the cache (V heads from v_col.. copied when
 *                v_col >= 0);
 *   k_col <  0 : K is already in the cache and is normalised and rotated in
 *                place (each band's key cache is modified in place).
 * A NULL gamma skips the norm for that role.  The norm of a head x is
 *   x_j / sqrt(mean(x^2) + epsilon) * (gamma_j + weight_offset)
 * and it is applied before the rotation.
 */
typedef struct qrp_band {
  uint64_t q_col;
  uint32_t n_q_heads;
  int64_t k_col;
  int64_t v_col;
  const void* q_gamma;         /* [head_dim] of dtype, device, or NULL */
  const void* k_gamma;         /* [head_dim] of dtype, device, or NULL */
  float epsilon;
  const qrp_paged_cache* cache;
  void* q_output;              /* [total_seq_len][q_out_row_stride] of dtype, device */
  uint64_t q_out_row_stride;
} qrp_band;

/*
 * rope_split_store_paged_ragged page (signature, Summary, Parameters, Args).
 *
 * qkv               device [total_seq_len][qkv_row_stride] of dtype, columns
 *                   Q heads | K heads | V heads (n_q_heads, then
 *                   cache->num_kv_heads twice, head_dim each).
 * input_row_offsets device uint32 [batch_size + 1]: sequence b's new tokens
 *                   are rows [offsets[b], offsets[b+1]); offsets[0] == 0 and
 *                   offsets[batch_size] == total_seq_len.
 * Token t of sequence b sits at position p = cache_lengths[b] + t - offsets[b].
 * Q head h of token t, rotated at p, goes to q_output[t][h*head_dim ..];
 * K heads, rotated, and V heads, copied bit for bit, go to row p of sequence
 * b's pages at layer layer_idx (an FP8 cache quantizes both rows).
 * cache_lengths are not updated.  q_out_dtype (QRP_F32, QRP_BF16 or
 * QRP_F16) may differ from dtype: Q is rounded once to it, and its
 * un-rotated elements are converted (nearest-even) rather than copied;
 * q_out_row_stride is in q_out_dtype elements.
 */
int32_t rope_split_store_paged(const void* qkv, int32_t dtype, uint32_t total_seq_len,
                               uint64_t qkv_row_stride, uint32_t n_q_heads,
                               const uint32_t* input_row_offsets, uint32_t batch_size,
                               const qrp_rope* rope, const qrp_paged_cache* cache,
                               uint32_t layer_idx, void* q_output, int32_t q_out_dtype,
                               uint64_t q_out_row_stride, void* stream);

/*
 * Single-band fused per-head RMSNorm + RoPE (named in the Summary of the
 * fused_dual_qk_rms_norm_rope_ragged_paged page; semantics from its
 * Description).  Same ragged addressing as rope_split_store_paged, through
 * band->cache.  weight_offset is a Scalar[dtype]: it is rounded to dtype
 * first.  multiply_before_cast != 0: y = x * r * (gamma + w) in binary32,
 * rounded once after the rotation; == 0: n = dtype(x * r),
 * g = dtype(gamma + w), y = dtype(n * g), then the rotation and a final
 * rounding.
 */
int32_t qk_rmsnorm_rope_paged(const void* qkv, int32_t dtype, uint32_t total_seq_len,
                              uint64_t qkv_row_stride, const qrp_band* band, float weight_offset,
                              int32_t multiply_before_cast, const uint32_t* input_row_offsets,
                              uint32_t batch_size, const qrp_rope* rope, uint32_t layer_idx,
                              void* stream);

/*
 * fused_dual_qk_rms_norm_rope_ragged_paged page: the main band and the index
 * band in ONE launch over the four row groups
 * [q_main | k_main | q_index | k_index] of each token.  Both bands read the
 * same buffer, offsets and freqs table; each row takes its own band's cache,
 * gamma, epsilon, output and Q columns.  The two caches must have the same
 * head_dim (QRP_EGEOMETRY otherwise: the page requires identical RoPE
 * geometry across the bands).  Their element types are independent
 * parameters on the page (Signature: main_cache_dtype, index_cache_dtype):
 * each cache may hold the op's dtype or FP8 codes, in any pairing.  The
 * result equals main_band's qk_rmsnorm_rope_paged call followed by
 * index_band's.
 */
int32_t dual_band(const void* buf, int32_t dtype, uint32_t total_seq_len, uint64_t buf_row_stride,
                  const qrp_band* main_band, const qrp_band* index_band, float weight_offset,
                  int32_t multiply_before_cast, const uint32_t* input_row_offsets,
                  uint32_t batch_size, const qrp_rope* rope, uint32_t layer_idx, void* stream);

/*
 * generic_kv_cache_radd_dispatch page (signature, Summary, Description,
 * Args).  a is device [total_rows][a_row_stride] of dtype; its first
 * num_kv_heads*head_dim columns are added into the K rows and the next
 * num_kv_heads*head_dim into the V rows of cache sequence b + batch_offset,
 * at positions cache_lengths[b + batch_offset] + t - offsets[b], layer
 * layer_idx.  Each element becomes dtype(float(cache) + float(a)), one
 * binary32 add.  Requires batch_offset + batch_size <= cache_batch and
 * kv_planes == 2.
 */
int32_t kv_cache_radd(const void* a, int32_t dtype, uint32_t total_rows, uint64_t a_row_stride,
                      const uint32_t* input_row_offsets, uint32_t batch_size, uint32_t batch_offset,
                      const qrp_paged_cache* cache, uint32_t layer_idx, void* stream);

/*
 * generic_fused_qk_rope_bshd_continuous_batch page (signature, Summary,
 * Args).  Padded continuous batching: q_proj and output are device
 * [batch_size][seq_len][n_q_heads][head_dim] of dtype, contiguous (output
 * may not alias q_proj).  valid_lengths is device uint32 [batch_size].  For
 * sequence b and row s < valid_lengths[b], at position
 * p = cache_lengths[b] + s:
 *   output[b][s][h] = RoPE(q_proj[b][s][h], p) for every Q head h;
 *   the K row of every KV head at position p of sequence b (plane 0, layer
 *   layer_idx) is read from the cache, rotated and written back in place
 *   (the projection has already stored it there).
 * Rows s >= valid_lengths[b] get no RoPE: their output row is q_proj's row,
 * bit for bit, and their cache rows are not touched.  V is never touched.
 * A continuous-batching cache (one contiguous block of rows per sequence)
 * is the case page_size = rows per block, max_pages_per_seq = 1,
 * lookup_table[b] = the block of sequence b; any paged cache also works.
 * The table's entry type (freq_dtype) may be QRP_F32, QRP_BF16 or QRP_F16
 * (the page gives the table the op's dtype).  Requires batch_size <=
 * cache_batch and batch_size * seq_len < 2^31.  A valid row whose position
 * or page is out of range writes nothing (run qrp_validate to find such
 * metadata); batch_size == 0 or seq_len == 0 returns QRP_OK without a launch.
 */
int32_t fused_qk_rope_bshd_continuous_batch(const void* q_proj, int32_t dtype, uint32_t batch_size,
                                            uint32_t seq_len, uint32_t n_q_heads,
                                            const uint32_t* valid_lengths, const qrp_rope* rope,
                                            const qrp_paged_cache* cache, uint32_t layer_idx,
                                            void* output, void* stream);

/*
 * MatmulFusedPartialRMSNorm page (Summary, execute, Args): a GEMV fused with
 * a partial RMSNorm.  For each of the m input rows x_i (m = 1 is the page's
 * GEMV; up to 8 rows per call, each independent):
 *   y = x_i W^T,  W stored [n][k] row-major (transpose_b = 1, the page's
 *                 default), or
 *   y = x_i W,    W stored [k][n] row-major (transpose_b = 0; the page's
 *                 Parameters: transpose_b),
 *   normed_output[i][j]   = y_j / sqrt(mean_{j' < n_normed} y_j'^2 + epsilon)
 *                           * gamma_j                   for j <  n_normed,
 *   unnormed_output[i][j - n_normed] = y_j              for j >= n_normed.
 * The mean runs over the n_normed leading columns only (n_normed is gamma's
 * length); weight_offset is accepted and not used (the page's Args say the
 * kernel does not consume it).  Products and sums are binary32.  With W
 * stored [n][k] one wave computes a column, each lane adding its terms in k
 * order -- one fused multiply-add per term for QRP_F32, one packed dot
 * product per pair of terms for QRP_BF16 and QRP_F16 (both products exact,
 * so at most one rounding per term) -- then a fixed 64-way tree adds the
 * lanes.  With W stored [k][n] the columns are cut into tiles of 128 bytes
 * of a row and k into slices (their count depends on n, k, the dtype and
 * the device's compute-unit count, never on m); for each tile and slice,
 * 512 threads each add the terms of 8 consecutive rows of every 512 in k
 * order (one fused multiply-add per term), then a fixed 8-way tree, the 8
 * wave sums in order, and the slices' sums in slice order.  With W stored
 * [k][n], n times the element size need not be a multiple of 16 bytes, but
 * the row stride must.  The norm
 * is binary32 (a row's sum of squares over 256 threads in a fixed order),
 * and each output is rounded once to dtype (QRP_F32, QRP_BF16 or QRP_F16;
 * x, W, gamma and both outputs share it).
 * Layout: input [m][input_row_stride], weight [n][weight_row_stride]
 * (transpose_b = 1) or [k][weight_row_stride] (transpose_b = 0),
 * normed_output [m][normed_row_stride], unnormed_output
 * [m][unnormed_row_stride], gamma [n_normed]; all device memory, strides in
 * elements.  input, weight and workspace are 16-byte aligned, k and the
 * input/weight strides are multiples of 16 bytes (QRP_EALIGN otherwise);
 * outputs and gamma are element-aligned.
 * Workspace: device memory the caller owns, at least
 * qrp_gemv_norm_workspace_bytes(m, n_normed, transpose_b) bytes: 1280 bytes
 * of arrival counters, then 4 * m * n_normed bytes of binary32 y values, and
 * with W stored [k][n] (transpose_b = 0), from the next 256-byte boundary,
 * 65536 * m bytes of binary32 partial sums of the k slices.  With W stored
 * [n][k] and n_normed = 0 the size is 0 and NULL is allowed.  It must be
 * zero-filled before its first use; every call leaves its counters at zero
 * again, so it is reused without clearing.
 * Calls that overlap in time must not share a workspace.
 * The summation order is fixed, so results are the same bits on every call
 * and for every row count (a row gives the same outputs alone or among 8).
 * Errors: QRP_EINVAL for a NULL buffer that the call needs, n_normed > n,
 * n >= 2^31, a stride below its row or a short workspace; QRP_EUNSUPPORTED
 * for m > 8 or another dtype; QRP_EINVAL for transpose_b other than 0 or
 * 1, or a weight row stride below k (transpose_b = 1) or n (transpose_b =
 * 0).  m == 0 or n == 0 returns
 * QRP_OK without a launch; k == 0 gives y = 0.
 */
uint64_t qrp_gemv_norm_workspace_bytes(uint32_t m, uint32_t n_normed, int32_t transpose_b);

int32_t matmul_fused_partial_rmsnorm(void* normed_output, uint64_t normed_row_stride,
                                     void* unnormed_output, uint64_t unnormed_row_stride,
                                     const void* input, uint64_t input_row_stride, uint32_t m,
                                     const void* weight, uint64_t weight_row_stride, uint32_t n,
                                     uint32_t k, const void* gamma, uint32_t n_normed,
                                     float epsilon, float weight_offset, int32_t dtype,
                                     int32_t transpose_b, void* workspace,
                                     uint64_t workspace_bytes, void* stream);

/*
 * matmul_fused_partial_rmsnorm for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors
 * (the same kernel, bit for bit) without the workspace: the scratch is the
 * library's own, a device array of 1280 + 4 * 131072 + 8 * 65536 bytes
 * (1 MiB and 1280 bytes) that each GPU the library runs on holds until the
 * process ends.  It serves m * n_normed <= 131072 (m rows of up to
 * 131072 / m normed columns);
 * larger calls return QRP_EINVAL and go through the workspace form.  The
 * first call on a device (the device current on the calling thread, which
 * must be the stream's) looks the array up and clears its counter with a
 * kernel on `stream`; no call allocates or frees memory.  Every call on a
 * GPU shares that GPU's array, and each call leaves its counters at zero:
 * calls that overlap in time on one GPU (other streams, other threads)
 * race and give wrong results; order them on one stream or use the
 * workspace form.
 */
int32_t matmul_fused_partial_rmsnorm_noalloc(void* normed_output, uint64_t normed_row_stride,
                                             void* unnormed_output, uint64_t unnormed_row_stride,
                                             const void* input, uint64_t input_row_stride,
                                             uint32_t m, const void* weight,
                                             uint64_t weight_row_stride, uint32_t n, uint32_t k,
                                             const void* gamma, uint32_t n_normed, float epsilon,
                                             float weight_offset, int32_t dtype,
                                             int32_t transpose_b, void* stream);

/*
 * Debug check of the device metadata one of the calls above would use:
 * copies offsets, cache_lengths and lookup_table to the host (synchronising
 * `stream`) and runs qrp_validate_host.  Returns QRP_EDATA with a message
 * on the first inconsistency.
 */
int32_t qrp_validate(const uint32_t* input_row_offsets, uint32_t batch_size,
                     uint32_t total_seq_len, uint32_t batch_offset, const qrp_paged_cache* cache,
                     uint32_t max_seq_len, void* stream);

/*
 * The same checks on host arrays: offsets start at 0, never decrease and end
 * at total_seq_len; batch_offset + batch_size <= cache_batch; every token's
 * position is below max_seq_len (when max_seq_len > 0), its page index below
 * max_pages_per_seq and its page id below num_pages; no two tokens land on
 * the same (page, row).
 */
int32_t qrp_validate_host(const uint32_t* input_row_offsets, uint32_t batch_size,
                          uint32_t total_seq_len, uint32_t batch_offset,
                          const uint32_t* cache_lengths, const uint32_t* lookup_table,
                          uint32_t cache_batch, uint32_t max_pages_per_seq, uint32_t page_size,
                          uint64_t num_pages, uint32_t max_seq_len);

/* Text of the last failure on the calling thread ("" if none). */
const char* qrp_last_error(void);

/* QRP_ABI_VERSION of the loaded library. */
int32_t qrp_abi_version(void);

/*
 * Launch-shape overrides, for measurement and tests.  They change how a
 * call's work is cut into waves and blocks, never what it computes (tests
 * check every setting gives the same bits).  Each knob is one process-wide
 * value; -1, the default, lets the library choose:
 *   QRP_KNOB_PACK             0: per-token passes, 1: token-packed passes
 *                             (ops that have both; the others ignore it)
 *   QRP_KNOB_PASSES_PER_WAVE  1 .. 8, capped by the op's register budget
 *   QRP_KNOB_WAVES_PER_BLOCK  1 .. 4
 *   QRP_KNOB_XCD_REMAP        0: blocks dealt to the XCDs round-robin,
 *                             1: consecutive blocks kept on one XCD,
 *                             2: each token's (or token block's) waves
 *                             kept on one XCD, tokens dealt round-robin
 *   QRP_KNOB_TAIL_UNITS       >= 0: the last this-many tokens (token blocks
 *                             when packed) of a launch of several passes
 *                             per wave run one pass per wave (the
 *                             library's choice: about 1536 such waves, 768
 *                             for the store op over FP8 caches, at most a
 *                             quarter of the launch's tokens)
 *   QRP_KNOB_LDS_BYTES        0 .. 65536: LDS bytes reserved per block,
 *                             unused by the kernel (it caps the blocks
 *                             resident on a compute unit; the library's
 *                             choice: 32768 for radd over a plain cache,
 *                             else 0).  The norm kernels' own 4 KB per
 *                             block comes on top; a launch whose total
 *                             passes the device's per-block LDS limit fails
 *                             (QRP_EHIP).
 * The environment variables QRP_PACK, QRP_PASSES_PER_WAVE (0: the
 * library's choice), QRP_WAVES_PER_BLOCK (0: the library's choice),
 * QRP_XCD_REMAP, QRP_TAIL_UNITS and QRP_LDS_BYTES give the first values,
 * read once when the library is loaded.  A launch reads the values current when it is enqueued; changing
 * them while other threads launch is allowed but gives those launches
 * either value.  `previous` (may be NULL) receives the old value.
 * QRP_EINVAL for an unknown knob or a value out of range.
 */
enum {
  QRP_KNOB_PACK = 0,
  QRP_KNOB_PASSES_PER_WAVE = 1,
  QRP_KNOB_WAVES_PER_BLOCK = 2,
  QRP_KNOB_XCD_REMAP = 3,
  QRP_KNOB_TAIL_UNITS = 4,
  QRP_KNOB_LDS_BYTES = 5
};
int32_t qrp_set_launch_override(int32_t knob, int32_t value, int32_t* previous);

#ifdef __cplusplus
}
#endif

#endif /* QK_ROPE_PAGED_H */
