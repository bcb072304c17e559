/*
 * qrp_oracle.c -- CPU oracle (TEST INFRASTRUCTURE ONLY; see qrp_oracle.h).
 *
 * Each function writes out the plain definition of the operation, in the
 * order the documentation pages describe it, with no blocking or fusion:
 *
 *   seq(t)   the sequence b whose ragged row range [off[b], off[b+1])
 *            holds token t (rope_split_store_paged_ragged page, Args:
 *            input_row_offsets; generic_kv_cache_radd_dispatch page, Args:
 *            input_row_offsets: one start row per sequence);
 *   pos(t)   cache_lengths[seq(t) + batch_offset] + t - off[seq(t)]
 *            (generic_kv_cache_radd_dispatch page, Description: batch
 *            offset and per-batch cache lengths locate the target rows);
 *   slot     page = lookup_table[seq][pos / page_size], row pos % page_size
 *            of that page, at layer layer_idx (rope_split_store_paged_ragged
 *            page, Args: kv_collection, layer_idx);
 *   rope     pairs rotated by the (cos, sin) freqs_cis entry of their
 *            frequency at pos (rope_split_store_paged_ragged page,
 *            Parameters: interleaved; Args: freqs_cis);
 *   norm     per-head RMSNorm with gamma + weight_offset, epsilon added to
 *            the mean square before the reciprocal square root
 *            (fused_dual_qk_rms_norm_rope_ragged_paged page, signature and
 *            Description; MatmulFusedPartialRMSNorm page, Args: epsilon);
 *   radd     cache += a, K half then V half of a's last dimension
 *            (generic_kv_cache_radd_dispatch page, Summary, Description).
 *
 * Built with -ffp-contract=off and no fast-math, so double and float
 * expressions round exactly as written.
 */
#include "qrp_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* element access                                                      */
/* ------------------------------------------------------------------ */

static size_t elem_bytes(int32_t dt) { return dt == ORC_F32 ? 4u : dt == ORC_FP8 ? 1u : 2u; }

/* element types of the operations' inputs and outputs */
static int dtype_ok(int32_t dt) { return dt == ORC_F32 || dt == ORC_BF16 || dt == ORC_F16; }

/* a cache holds the op's dtype, or FP8 codes with a scale per row */
static int cache_dtype_ok(const orc_cache* c, int32_t dtype) {
  if (c->dtype == dtype) return 1;
  return c->dtype == ORC_FP8 && c->scales &&
         (c->scale_dtype == ORC_F32 || c->scale_dtype == ORC_BF16);
}

double orc_bf16_to_double(uint16_t b) {
  /* a bf16 value is the upper half of an IEEE binary32 word */
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

uint16_t orc_round_bf16(double x) {
  float f;
  uint32_t u;
  if (isnan(x)) {
    f = (float)x;
    memcpy(&u, &f, 4);
    return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN, sign and top payload kept */
  }
  if (x == 0.0 || isinf(x)) {
    f = (float)x; /* exact */
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
  }
  /* bf16 keeps 8 significant bits; its exponent range is binary32's, so
   * below 2^-126 the spacing stays 2^-133 (subnormals). */
  int e = ilogb(x);
  if (e < -126) e = -126;
  double quantum = ldexp(1.0, e - 7);
  double r = nearbyint(x / quantum) * quantum; /* ties to even (default rounding mode) */
  if (fabs(r) >= ldexp(1.0, 128)) return (uint16_t)(x < 0 ? 0xFF80u : 0x7F80u);
  f = (float)r; /* exact: r has at most 8 significant bits */
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_to_double(uint16_t h) {
  const int sign = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  return sign ? -v : v;
}

uint16_t orc_round_f16(double x) {
  const uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return (uint16_t)(sign | 0x7E00u); /* a quiet NaN */
  if (isinf(x)) return (uint16_t)(sign | 0x7C00u);
  if (x == 0.0) return sign;
  /* 11 significant bits; below 2^-14 the spacing stays 2^-24 (subnormals) */
  int e = ilogb(x);
  if (e < -14) e = -14;
  double quantum = ldexp(1.0, e - 10);
  double r = fabs(nearbyint(x / quantum) * quantum); /* ties to even */
  if (r >= 65536.0) return (uint16_t)(sign | 0x7C00u); /* past 65504 by half a spacing or more */
  if (r < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
  int re = ilogb(r); /* the rounded value may have moved up one binade */
  uint16_t mant = (uint16_t)((r / ldexp(1.0, re) - 1.0) * 1024.0);
  return (uint16_t)(sign | (uint16_t)((re + 15) << 10) | mant);
}

/* OCP FP8 E4M3, the finite-only variant: 1 sign, 4 exponent (bias 7) and 3
 * fraction bits; exponent field 0 holds subnormals m * 2^-9; the all-ones
 * pattern S.1111.111 is NaN; the largest finite value is 1.75 * 2^8 = 448. */
double orc_e4m3_to_double(uint8_t q) {
  const int sign = q >> 7, e = (q >> 3) & 0xF, m = q & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

uint8_t orc_round_e4m3(double x) {
  const uint8_t sign = signbit(x) ? 0x80u : 0u;
  if (isnan(x)) return (uint8_t)(sign | 0x7Fu);
  double a = fabs(x);
  if (a == 0.0) return sign;
  /* 4 significant bits; below 2^-6 the spacing stays 2^-9 (subnormals) */
  int e = isinf(a) ? 8 : ilogb(a);
  if (e < -6) e = -6;
  double quantum = ldexp(1.0, e - 3);
  double r = isinf(a) ? 448.0 : nearbyint(a / quantum) * quantum; /* ties to even */
  if (r > 448.0) r = 448.0; /* no infinity in this format: saturate */
  if (r < ldexp(1.0, -6)) return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9)));
  int re = ilogb(r); /* the rounded value may have moved up one binade */
  uint8_t mant = (uint8_t)((r / ldexp(1.0, re) - 1.0) * 8.0);
  return (uint8_t)(sign | (uint8_t)((re + 7) << 3) | mant);
}

static double get(const void* base, int32_t dt, int64_t i) {
  if (dt == ORC_F32) return (double)((const float*)base)[i];
  if (dt == ORC_F16) return orc_f16_to_double(((const uint16_t*)base)[i]);
  return orc_bf16_to_double(((const uint16_t*)base)[i]);
}

/* value rounded to dtype, returned as double */
static double round_to(int32_t dt, double v) {
  if (dt == ORC_F32) return (double)(float)v;
  if (dt == ORC_F16) return orc_f16_to_double(orc_round_f16(v));
  return orc_bf16_to_double(orc_round_bf16(v));
}

static void put(void* base, int32_t dt, int64_t i, double v) {
  if (dt == ORC_F32)
    ((float*)base)[i] = (float)v;
  else if (dt == ORC_F16)
    ((uint16_t*)base)[i] = orc_round_f16(v);
  else
    ((uint16_t*)base)[i] = orc_round_bf16(v);
}

static void copy_bits(void* dst, int64_t di, const void* src, int64_t si, int32_t dt) {
  size_t n = elem_bytes(dt);
  memcpy((char*)dst + (size_t)di * n, (const char*)src + (size_t)si * n, n);
}

/* ------------------------------------------------------------------ */
/* ragged batch and paged placement                                    */
/* ------------------------------------------------------------------ */

static int32_t check_offsets(const uint32_t* off, uint32_t B, uint32_t T) {
  if (off[0] != 0 || off[B] != T) return ORC_EDATA;
  for (uint32_t b = 0; b < B; ++b)
    if (off[b + 1] < off[b]) return ORC_EDATA;
  return ORC_OK;
}

/* the unique b with off[b] <= t < off[b+1], by linear scan */
static int64_t seq_of(const uint32_t* off, uint32_t B, uint32_t t) {
  for (uint32_t b = 0; b < B; ++b)
    if (off[b] <= t && t < off[b + 1]) return (int64_t)b;
  return -1;
}

/* page and in-page row of position `pos` of cache sequence `cseq` */
static int32_t locate(const orc_cache* c, uint32_t cseq, uint32_t pos, uint64_t* page,
                      uint32_t* slot) {
  if (cseq >= c->cache_batch) return ORC_EDATA;
  uint32_t idx = pos / c->page_size;
  if (idx >= c->max_pages_per_seq) return ORC_EDATA;
  uint64_t pg = c->lookup_table[(uint64_t)cseq * c->max_pages_per_seq + idx];
  if (pg >= c->num_pages) return ORC_EDATA;
  *page = pg;
  *slot = pos % c->page_size;
  return ORC_OK;
}

/* element offset of head `h` of row `slot` in plane `plane`, layer `layer` */
static int64_t row_offset(const orc_cache* c, uint64_t page, uint32_t plane, uint32_t layer,
                          uint32_t slot, uint32_t h) {
  return (int64_t)page * c->page_stride + (int64_t)plane * c->plane_stride +
         (int64_t)layer * c->layer_stride + (int64_t)slot * c->slot_stride +
         (int64_t)h * c->head_stride;
}

/* Token t -> (cache sequence, position, page, slot), with every bound checked. */
typedef struct {
  uint32_t cseq, pos, slot;
  uint64_t page;
} where_t;

static int32_t where_is(const orc_cache* c, const uint32_t* off, uint32_t B, uint32_t batch_offset,
                        uint32_t t, uint32_t max_seq_len, where_t* w) {
  int64_t b = seq_of(off, B, t);
  if (b < 0) return ORC_EDATA;
  uint32_t cseq = (uint32_t)b + batch_offset;
  if (cseq >= c->cache_batch) return ORC_EDATA;
  uint64_t pos = (uint64_t)c->cache_lengths[cseq] + (t - off[b]);
  if (max_seq_len && pos >= max_seq_len) return ORC_EDATA;
  if (pos > 0xFFFFFFFFull) return ORC_EDATA;
  w->cseq = cseq;
  w->pos = (uint32_t)pos;
  return locate(c, cseq, w->pos, &w->page, &w->slot);
}

/* ------------------------------------------------------------------ */
/* per-head arithmetic                                                 */
/* ------------------------------------------------------------------ */

/* RoPE of one head x[D] at position pos over dims start .. start + R - 1;
 * y gets the rotated values and mag[j] the length of the pair j belongs to
 * (|x_j| for dims that do not rotate). */
static void rope_head(const double* x, double* y, double* mag, uint32_t D, const float* freqs,
                      uint32_t pos, uint32_t R, int32_t interleaved, uint32_t start) {
  for (uint32_t j = 0; j < D; ++j) {
    y[j] = x[j];
    mag[j] = fabs(x[j]);
  }
  const float* row = freqs + (uint64_t)pos * R;
  for (uint32_t i = 0; i < R / 2; ++i) {
    double c = (double)row[2 * i];     /* cos(pos * theta_i) */
    double s = (double)row[2 * i + 1]; /* sin(pos * theta_i) */
    uint32_t j0 = start + (interleaved ? 2 * i : i);
    uint32_t j1 = start + (interleaved ? 2 * i + 1 : i + R / 2);
    double re = x[j0], im = x[j1];
    /* (re + i im) * (c + i s) */
    y[j0] = re * c - im * s;
    y[j1] = re * s + im * c;
    double m = hypot(y[j0], y[j1]);
    mag[j0] = m;
    mag[j1] = m;
  }
}

/* per-head RMSNorm: y_j = x_j / sqrt(mean(x^2) + eps) * (gamma_j + w);
 * pre_j gets x_j * r, the normalised value before any rounding */
static void rmsnorm_head(const double* x, double* y, double* pre, uint32_t D, const void* gamma,
                         int32_t dt, double w, double eps, int32_t multiply_before_cast) {
  double ss = 0.0;
  for (uint32_t j = 0; j < D; ++j) ss += x[j] * x[j];
  double r = 1.0 / sqrt(ss / (double)D + eps);
  for (uint32_t j = 0; j < D; ++j) {
    double g = get(gamma, dt, j);
    pre[j] = x[j] * r;
    if (multiply_before_cast) {
      y[j] = x[j] * r * (g + w);
    } else {
      double n = round_to(dt, x[j] * r);
      double gw = round_to(dt, g + w);
      y[j] = round_to(dt, n * gw);
    }
  }
}

/* Scratch for one head. */
typedef struct {
  double *x, *xn, *y, *mag, *pre;
} head_buf;

static int head_buf_alloc(head_buf* hb, uint32_t D) {
  hb->x = (double*)malloc(sizeof(double) * D * 5);
  if (!hb->x) return 0;
  hb->xn = hb->x + D;
  hb->y = hb->x + 2 * D;
  hb->mag = hb->x + 3 * D;
  hb->pre = hb->x + 4 * D;
  return 1;
}

/* hb->x (already read) -> optional norm -> rope -> hb->y, pair lengths in hb->mag */
static void head_math(head_buf* hb, uint32_t D, const void* gamma, int32_t dt, double w,
                      double eps, int32_t mbc, const float* freqs, uint32_t pos, uint32_t R,
                      int32_t interleaved, uint32_t start) {
  const double* in = hb->x;
  if (gamma) {
    rmsnorm_head(hb->x, hb->xn, hb->pre, D, gamma, dt, w, eps, mbc);
    in = hb->xn;
  }
  rope_head(in, hb->y, hb->mag, D, freqs, pos, R, interleaved, start);
}

static void record(const head_buf* hb, uint32_t D, double* exact, double* mag) {
  for (uint32_t j = 0; j < D; ++j) {
    if (exact) exact[j] = hb->y[j];
    if (mag) mag[j] = hb->mag[j];
  }
}

/* the normalised values before rounding, for a role that was normalised */
static void record_pre(const head_buf* hb, uint32_t D, double* pre) {
  if (pre)
    for (uint32_t j = 0; j < D; ++j) pre[j] = hb->pre[j];
}

/* Store a head's result in a plain buffer of dtype dst_dt.  Elements lo ..
 * hi - 1 (the roped ones; all of them after a norm) are rounded to dst_dt;
 * the others move as raw bits when the source has dst_dt, and are rounded
 * (converted) when it does not. */
static void store_plain(void* dst, int64_t dst_off, int32_t dst_dt, const double* y,
                        const void* src, int64_t src_off, int32_t src_dt, uint32_t D,
                        uint32_t lo, uint32_t hi) {
  for (uint32_t j = 0; j < D; ++j) {
    if ((j >= lo && j < hi) || src_dt != dst_dt)
      put(dst, dst_dt, dst_off + j, y[j]);
    else
      copy_bits(dst, dst_off + j, src, src_off + j, dst_dt);
  }
}

/* ---- FP8 cache rows: one scale per (page, plane, layer, slot, head) row ---- */

static int64_t scale_offset(const orc_cache* c, uint64_t page, uint32_t plane, uint32_t layer,
                            uint32_t slot, uint32_t h) {
  return (int64_t)page * c->s_page_stride + (int64_t)plane * c->s_plane_stride +
         (int64_t)layer * c->s_layer_stride + (int64_t)slot * c->s_slot_stride +
         (int64_t)h * c->s_head_stride;
}

static float get_scale(const orc_cache* c, int64_t so) {
  if (c->scale_dtype == ORC_F32) return ((const float*)c->scales)[so];
  return (float)orc_bf16_to_double(((const uint16_t*)c->scales)[so]);
}

static void put_scale(orc_cache* c, int64_t so, float s) {
  if (c->scale_dtype == ORC_F32)
    ((float*)c->scales)[so] = s;
  else
    ((uint16_t*)c->scales)[so] = orc_round_bf16((double)s); /* exact: s is a bf16 value */
}

/* Quantize one head row (reading of the cache collection's scale dtype and
 * granularity parameters, which the pages name without defining): every
 * decision is taken in binary32.  v_j = binary32(y_j); amax = max |v_j|;
 * s = amax / 448 (binary32 division), rounded to the scale dtype;
 * r = 1 / s (binary32; 0 when s = 0); code_j = e4m3(clamp(v_j * r, +-448))
 * with the product rounded to binary32 and the code by nearest-even. */
static void quantize_row(orc_cache* c, int64_t off, int64_t so, const double* y, uint32_t D) {
  float amax = 0.0f;
  for (uint32_t j = 0; j < D; ++j) {
    float v = (float)y[j];
    if (fabsf(v) > amax) amax = fabsf(v);
  }
  float s = amax / 448.0f;
  if (c->scale_dtype == ORC_BF16) s = (float)orc_bf16_to_double(orc_round_bf16((double)s));
  float r = s > 0.0f ? 1.0f / s : 0.0f;
  uint8_t* codes = (uint8_t*)c->pool + off;
  for (uint32_t j = 0; j < D; ++j) {
    float q = (float)y[j] * r;
    if (q > 448.0f) q = 448.0f;
    if (q < -448.0f) q = -448.0f;
    codes[j] = orc_round_e4m3((double)q);
  }
  put_scale(c, so, s);
}

/* A cache row's values: plain dtypes widen exactly; FP8 codes are scaled by
 * the row's scale with one binary32 multiply. */
static void read_cache_row(const orc_cache* c, int64_t off, int64_t so, uint32_t D, double* x) {
  if (c->dtype != ORC_FP8) {
    for (uint32_t j = 0; j < D; ++j) x[j] = get(c->pool, c->dtype, off + j);
    return;
  }
  const float s = get_scale(c, so);
  const uint8_t* codes = (const uint8_t*)c->pool + off;
  for (uint32_t j = 0; j < D; ++j) x[j] = (double)((float)orc_e4m3_to_double(codes[j]) * s);
}

/* Store a head's result in a cache row: a plain cache as store_plain does
 * (its dtype is the op's), an FP8 cache by quantizing the whole row. */
static void store_cache_row(orc_cache* c, int64_t off, int64_t so, const double* y,
                            const void* src, int64_t src_off, int32_t src_dt, uint32_t D,
                            uint32_t lo, uint32_t hi) {
  if (c->dtype == ORC_FP8)
    quantize_row(c, off, so, y, D);
  else
    store_plain(c->pool, off, c->dtype, y, src, src_off, src_dt, D, lo, hi);
}

static void read_plain(const void* src, int32_t dt, int64_t off, uint32_t D, double* x) {
  for (uint32_t j = 0; j < D; ++j) x[j] = get(src, dt, off + j);
}

static int32_t check_common(int32_t dtype, const orc_cache* c, uint32_t rope_dim,
                            uint32_t layer_idx, uint32_t max_seq_len) {
  if (!c || !c->pool || !c->cache_lengths || !c->lookup_table) return ORC_EINVAL;
  if (!dtype_ok(dtype)) return ORC_EINVAL;
  if (!cache_dtype_ok(c, dtype)) return ORC_EINVAL;
  if (c->head_dim == 0 || c->page_size == 0) return ORC_EINVAL;
  if (rope_dim == 0 || rope_dim % 2 || rope_dim > c->head_dim) return ORC_EINVAL;
  if (layer_idx >= c->num_layers) return ORC_EINVAL;
  if (max_seq_len == 0) return ORC_EINVAL;
  return ORC_OK;
}

static void set_off(int64_t* rec, uint64_t i, int64_t v) {
  if (rec) rec[i] = v;
}

/* ------------------------------------------------------------------ */
/* operations                                                          */
/* ------------------------------------------------------------------ */

int32_t orc_rope_split_store_paged(const void* qkv, int32_t dtype, uint32_t T,
                                   uint64_t qkv_row_stride, uint32_t n_q_heads,
                                   const uint32_t* off, uint32_t B, const float* freqs,
                                   uint32_t max_seq_len, uint32_t R, int32_t interleaved,
                                   int32_t rope_tail, orc_cache* c, uint32_t layer_idx, void* q_out,
                                   int32_t q_out_dtype, uint64_t q_out_row_stride,
                                   orc_trace* tr) {
  int32_t st = check_common(dtype, c, R, layer_idx, max_seq_len);
  if (st) return st;
  if (!dtype_ok(q_out_dtype)) return ORC_EINVAL;
  if (c->kv_planes != 2) return ORC_EINVAL;
  if (T == 0) return ORC_OK;
  if (!qkv || !off || !freqs || !q_out) return ORC_EINVAL;
  if (B > c->cache_batch) return ORC_EINVAL;
  const uint32_t D = c->head_dim, Hq = n_q_heads, Hk = c->num_kv_heads;
  /* the rotated dims: the first rope_dim, or with rope_tail the last */
  const uint32_t r0 = rope_tail ? D - R : 0;
  if (qkv_row_stride < (uint64_t)(Hq + 2 * Hk) * D || q_out_row_stride < (uint64_t)Hq * D)
    return ORC_EINVAL;
  if ((st = check_offsets(off, B, T))) return st;
  where_t w;
  for (uint32_t t = 0; t < T; ++t)
    if ((st = where_is(c, off, B, 0, t, max_seq_len, &w))) return st;

  head_buf hb;
  if (!head_buf_alloc(&hb, D)) return ORC_EINVAL;
  for (uint32_t t = 0; t < T; ++t) {
    where_is(c, off, B, 0, t, max_seq_len, &w);
    const int64_t in_row = (int64_t)t * (int64_t)qkv_row_stride;
    /* Q heads -> dense q_output (of q_out_dtype) */
    for (uint32_t h = 0; h < Hq; ++h) {
      const int64_t src = in_row + (int64_t)h * D;
      read_plain(qkv, dtype, src, D, hb.x);
      head_math(&hb, D, NULL, dtype, 0.0, 0.0, 1, freqs, w.pos, R, interleaved, r0);
      store_plain(q_out, (int64_t)t * (int64_t)q_out_row_stride + (int64_t)h * D, q_out_dtype,
                  hb.y, qkv, src, dtype, D, r0, r0 + R);
      if (tr)
        record(&hb, D, tr->q_exact ? tr->q_exact + ((uint64_t)t * Hq + h) * D : NULL,
               tr->q_mag ? tr->q_mag + ((uint64_t)t * Hq + h) * D : NULL);
    }
    /* K heads -> plane 0 of the cache, roped */
    for (uint32_t h = 0; h < Hk; ++h) {
      const int64_t src = in_row + (int64_t)(Hq + h) * D;
      const int64_t dst = row_offset(c, w.page, 0, layer_idx, w.slot, h);
      const int64_t so = c->scales ? scale_offset(c, w.page, 0, layer_idx, w.slot, h) : -1;
      read_plain(qkv, dtype, src, D, hb.x);
      head_math(&hb, D, NULL, dtype, 0.0, 0.0, 1, freqs, w.pos, R, interleaved, r0);
      store_cache_row(c, dst, so, hb.y, qkv, src, dtype, D, r0, r0 + R);
      if (tr) {
        record(&hb, D, tr->k_exact ? tr->k_exact + ((uint64_t)t * Hk + h) * D : NULL,
               tr->k_mag ? tr->k_mag + ((uint64_t)t * Hk + h) * D : NULL);
        set_off(tr->k_row_off, (uint64_t)t * Hk + h, dst);
        set_off(tr->k_scale_off, (uint64_t)t * Hk + h, so);
      }
    }
    /* V heads -> plane 1 of the cache: bits moved as they are (an FP8 cache
     * quantizes the row instead) */
    for (uint32_t h = 0; h < Hk; ++h) {
      const int64_t src = in_row + (int64_t)(Hq + Hk + h) * D;
      const int64_t dst = row_offset(c, w.page, 1, layer_idx, w.slot, h);
      const int64_t so = c->scales ? scale_offset(c, w.page, 1, layer_idx, w.slot, h) : -1;
      read_plain(qkv, dtype, src, D, hb.x);
      store_cache_row(c, dst, so, hb.x, qkv, src, dtype, D, 0, 0);
      if (tr) {
        set_off(tr->v_row_off, (uint64_t)t * Hk + h, dst);
        set_off(tr->v_scale_off, (uint64_t)t * Hk + h, so);
      }
    }
  }
  free(hb.x);
  return ORC_OK;
}

int32_t orc_qk_rmsnorm_rope_paged(const void* buf, int32_t dtype, uint32_t T,
                                  uint64_t buf_row_stride, const orc_band* band,
                                  float weight_offset, int32_t multiply_before_cast,
                                  const uint32_t* off, uint32_t B, const float* freqs,
                                  uint32_t max_seq_len, uint32_t R, int32_t interleaved,
                                  int32_t rope_tail, uint32_t layer_idx, orc_trace* tr) {
  if (!band) return ORC_EINVAL;
  orc_cache* c = band->cache;
  int32_t st = check_common(dtype, c, R, layer_idx, max_seq_len);
  if (st) return st;
  if (band->v_col >= 0 && (band->k_col < 0 || c->kv_planes != 2)) return ORC_EINVAL;
  if (T == 0) return ORC_OK;
  if (!buf || !off || !freqs || (band->n_q_heads && !band->q_output)) return ORC_EINVAL;
  if (B > c->cache_batch) return ORC_EINVAL;
  const uint32_t D = c->head_dim, Hq = band->n_q_heads, Hk = c->num_kv_heads;
  /* the rotated dims: the first rope_dim, or with rope_tail the last */
  const uint32_t r0 = rope_tail ? D - R : 0;
  if ((st = check_offsets(off, B, T))) return st;
  where_t w;
  for (uint32_t t = 0; t < T; ++t)
    if ((st = where_is(c, off, B, 0, t, max_seq_len, &w))) return st;

  /* weight_offset is a Scalar[dtype] (fused_dual_qk_rms_norm_rope_ragged_paged
   * page, signature): take its dtype value. */
  const double wv = round_to(dtype, (double)weight_offset);
  const double eps = (double)band->epsilon;
  head_buf hb;
  if (!head_buf_alloc(&hb, D)) return ORC_EINVAL;
  for (uint32_t t = 0; t < T; ++t) {
    where_is(c, off, B, 0, t, max_seq_len, &w);
    const int64_t in_row = (int64_t)t * (int64_t)buf_row_stride;
    for (uint32_t h = 0; h < Hq; ++h) {
      const int64_t src = in_row + (int64_t)band->q_col + (int64_t)h * D;
      read_plain(buf, dtype, src, D, hb.x);
      head_math(&hb, D, band->q_gamma, dtype, wv, eps, multiply_before_cast, freqs, w.pos, R,
                interleaved, r0);
      store_plain(band->q_output, (int64_t)t * (int64_t)band->q_out_row_stride + (int64_t)h * D,
                  dtype, hb.y, buf, src, dtype, D, band->q_gamma ? 0 : r0,
                  band->q_gamma ? D : r0 + R);
      if (tr) {
        record(&hb, D, tr->q_exact ? tr->q_exact + ((uint64_t)t * Hq + h) * D : NULL,
               tr->q_mag ? tr->q_mag + ((uint64_t)t * Hq + h) * D : NULL);
        if (band->q_gamma)
          record_pre(&hb, D, tr->q_pre ? tr->q_pre + ((uint64_t)t * Hq + h) * D : NULL);
      }
    }
    for (uint32_t h = 0; h < Hk; ++h) {
      const int64_t dst = row_offset(c, w.page, 0, layer_idx, w.slot, h);
      const int64_t so = c->scales ? scale_offset(c, w.page, 0, layer_idx, w.slot, h) : -1;
      const uint32_t lo = band->k_gamma ? 0 : r0, hi = band->k_gamma ? D : r0 + R;
      if (band->k_col >= 0) { /* K from the buffer */
        const int64_t src = in_row + band->k_col + (int64_t)h * D;
        read_plain(buf, dtype, src, D, hb.x);
        head_math(&hb, D, band->k_gamma, dtype, wv, eps, multiply_before_cast, freqs, w.pos, R,
                  interleaved, r0);
        store_cache_row(c, dst, so, hb.y, buf, src, dtype, D, lo, hi);
      } else { /* K already in the cache: updated in place (the row is read whole first) */
        read_cache_row(c, dst, so, D, hb.x);
        head_math(&hb, D, band->k_gamma, dtype, wv, eps, multiply_before_cast, freqs, w.pos, R,
                  interleaved, r0);
        store_cache_row(c, dst, so, hb.y, c->pool, dst, c->dtype, D, lo, hi);
      }
      if (tr) {
        record(&hb, D, tr->k_exact ? tr->k_exact + ((uint64_t)t * Hk + h) * D : NULL,
               tr->k_mag ? tr->k_mag + ((uint64_t)t * Hk + h) * D : NULL);
        if (band->k_gamma)
          record_pre(&hb, D, tr->k_pre ? tr->k_pre + ((uint64_t)t * Hk + h) * D : NULL);
        set_off(tr->k_row_off, (uint64_t)t * Hk + h, dst);
        set_off(tr->k_scale_off, (uint64_t)t * Hk + h, so);
      }
    }
    if (band->v_col >= 0) {
      for (uint32_t h = 0; h < Hk; ++h) {
        const int64_t src = in_row + band->v_col + (int64_t)h * D;
        const int64_t dst = row_offset(c, w.page, 1, layer_idx, w.slot, h);
        const int64_t so = c->scales ? scale_offset(c, w.page, 1, layer_idx, w.slot, h) : -1;
        read_plain(buf, dtype, src, D, hb.x);
        store_cache_row(c, dst, so, hb.x, buf, src, dtype, D, 0, 0);
        if (tr) {
          set_off(tr->v_row_off, (uint64_t)t * Hk + h, dst);
          set_off(tr->v_scale_off, (uint64_t)t * Hk + h, so);
        }
      }
    }
  }
  free(hb.x);
  return ORC_OK;
}

int32_t orc_dual_band(const void* buf, int32_t dtype, uint32_t T, uint64_t buf_row_stride,
                      const orc_band* main_band, const orc_band* index_band, float weight_offset,
                      int32_t multiply_before_cast, const uint32_t* off, uint32_t B,
                      const float* freqs, uint32_t max_seq_len, uint32_t R, int32_t interleaved,
                      int32_t rope_tail, uint32_t layer_idx, orc_trace* main_trace,
                      orc_trace* index_trace) {
  if (!main_band || !index_band || !main_band->cache || !index_band->cache) return ORC_EINVAL;
  /* the two bands share the op's dtype and must agree on head size
   * (fused_dual_qk_rms_norm_rope_ragged_paged page, Description: identical
   * RoPE geometry across both bands); their caches' element types are
   * independent parameters (signature: main_cache_dtype, index_cache_dtype) */
  if (main_band->cache->head_dim != index_band->cache->head_dim) return ORC_EINVAL;
  /* one launch fusing two single-band launches: the same result as the two in turn */
  int32_t st = orc_qk_rmsnorm_rope_paged(buf, dtype, T, buf_row_stride, main_band, weight_offset,
                                         multiply_before_cast, off, B, freqs, max_seq_len, R,
                                         interleaved, rope_tail, layer_idx, main_trace);
  if (st) return st;
  return orc_qk_rmsnorm_rope_paged(buf, dtype, T, buf_row_stride, index_band, weight_offset,
                                   multiply_before_cast, off, B, freqs, max_seq_len, R,
                                   interleaved, rope_tail, layer_idx, index_trace);
}

int32_t orc_kv_cache_radd(const void* a, int32_t dtype, uint32_t T, uint64_t a_row_stride,
                          const uint32_t* off, uint32_t B, uint32_t batch_offset, orc_cache* c,
                          uint32_t layer_idx, orc_trace* tr) {
  if (!c || !c->pool || !c->cache_lengths || !c->lookup_table) return ORC_EINVAL;
  if (!dtype_ok(dtype) || !cache_dtype_ok(c, dtype)) return ORC_EINVAL;
  if (c->kv_planes != 2 || layer_idx >= c->num_layers) return ORC_EINVAL;
  if ((uint64_t)batch_offset + B > c->cache_batch) return ORC_EINVAL;
  if (T == 0) return ORC_OK;
  if (!a || !off) return ORC_EINVAL;
  const uint32_t D = c->head_dim, Hk = c->num_kv_heads;
  const uint64_t hidden = (uint64_t)Hk * D; /* a is (rows, 2 * hidden) */
  if (a_row_stride < 2 * hidden) return ORC_EINVAL;
  int32_t st = check_offsets(off, B, T);
  if (st) return st;
  where_t w;
  for (uint32_t t = 0; t < T; ++t)
    if ((st = where_is(c, off, B, batch_offset, t, 0, &w))) return st;

  double* row = (double*)malloc(sizeof(double) * D);
  if (!row) return ORC_EINVAL;
  for (uint32_t t = 0; t < T; ++t) {
    where_is(c, off, B, batch_offset, t, 0, &w);
    for (uint32_t plane = 0; plane < 2; ++plane) { /* first half of a -> K, second -> V */
      for (uint32_t h = 0; h < Hk; ++h) {
        const int64_t dst = row_offset(c, w.page, plane, layer_idx, w.slot, h);
        const int64_t so = c->scales ? scale_offset(c, w.page, plane, layer_idx, w.slot, h) : -1;
        const int64_t src = (int64_t)t * (int64_t)a_row_stride + (int64_t)(plane * hidden) + (int64_t)h * D;
        read_cache_row(c, dst, so, D, row);
        for (uint32_t j = 0; j < D; ++j) {
          float cur = (float)row[j];
          float add = (float)get(a, dtype, src + j);
          float sum = cur + add; /* one IEEE binary32 add */
          row[j] = (double)sum;
        }
        if (c->dtype == ORC_FP8)
          quantize_row(c, dst, so, row, D);
        else
          for (uint32_t j = 0; j < D; ++j) put(c->pool, c->dtype, dst + j, row[j]);
        if (tr) {
          set_off(plane == 0 ? tr->k_row_off : tr->v_row_off, (uint64_t)t * Hk + h, dst);
          set_off(plane == 0 ? tr->k_scale_off : tr->v_scale_off, (uint64_t)t * Hk + h, so);
        }
      }
    }
  }
  free(row);
  return ORC_OK;
}

/* Padded continuous batching (generic_fused_qk_rope_bshd_continuous_batch
 * page, signature and Args): q_proj and output are [B][S][n_q_heads][D].
 * Row s of sequence b is a real token when s < valid_lengths[b]; it sits at
 * position cache_lengths[b] + s, its Q heads are rotated into output and its
 * K rows, already in the cache, are rotated in place.  Other rows get no
 * rotation: their output row is the input row's bits and the cache is left
 * alone.  Trace rows of Q are filled for every row (a copied row records its
 * own values); k_row_off stays untouched (-1 from the caller) for rows
 * without K work. */
int32_t orc_fused_qk_rope_bshd(const void* q_proj, int32_t dtype, uint32_t B, uint32_t S,
                               uint32_t n_q_heads, const uint32_t* valid_lengths,
                               const float* freqs, uint32_t max_seq_len, uint32_t R,
                               int32_t interleaved, int32_t rope_tail, orc_cache* c,
                               uint32_t layer_idx,
                               void* output, orc_trace* tr) {
  int32_t st = check_common(dtype, c, R, layer_idx, max_seq_len);
  if (st) return st;
  if (B == 0 || S == 0) return ORC_OK;
  if (!q_proj || !valid_lengths || !freqs || !output || n_q_heads == 0) return ORC_EINVAL;
  if (B > c->cache_batch) return ORC_EINVAL;
  const uint32_t D = c->head_dim, Hq = n_q_heads, Hk = c->num_kv_heads;
  /* the rotated dims: the first rope_dim, or with rope_tail the last */
  const uint32_t r0 = rope_tail ? D - R : 0;
  const int64_t row_len = (int64_t)Hq * D;

  /* every real token's position and page must exist before anything is written */
  for (uint32_t b = 0; b < B; ++b) {
    for (uint32_t s = 0; s < S && s < valid_lengths[b]; ++s) {
      uint64_t pos = (uint64_t)c->cache_lengths[b] + s;
      if (pos >= max_seq_len) return ORC_EDATA;
      uint64_t page;
      uint32_t slot;
      if ((st = locate(c, b, (uint32_t)pos, &page, &slot))) return st;
    }
  }

  head_buf hb;
  if (!head_buf_alloc(&hb, D)) return ORC_EINVAL;
  for (uint32_t b = 0; b < B; ++b) {
    for (uint32_t s = 0; s < S; ++s) {
      const uint64_t t = (uint64_t)b * S + s;
      const int64_t row = (int64_t)t * row_len;
      if (s >= valid_lengths[b]) {
        for (int64_t e = 0; e < row_len; ++e) copy_bits(output, row + e, q_proj, row + e, dtype);
        if (tr && tr->q_exact)
          for (int64_t e = 0; e < row_len; ++e) tr->q_exact[t * row_len + e] = get(q_proj, dtype, row + e);
        if (tr && tr->q_mag)
          for (int64_t e = 0; e < row_len; ++e) tr->q_mag[t * row_len + e] = fabs(get(q_proj, dtype, row + e));
        continue;
      }
      const uint32_t pos = c->cache_lengths[b] + s;
      uint64_t page = 0;
      uint32_t slot = 0;
      locate(c, b, pos, &page, &slot); /* checked above */
      for (uint32_t h = 0; h < Hq; ++h) {
        const int64_t src = row + (int64_t)h * D;
        read_plain(q_proj, dtype, src, D, hb.x);
        head_math(&hb, D, NULL, dtype, 0.0, 0.0, 1, freqs, pos, R, interleaved, r0);
        store_plain(output, src, dtype, hb.y, q_proj, src, dtype, D, r0, r0 + R);
        if (tr)
          record(&hb, D, tr->q_exact ? tr->q_exact + (t * Hq + h) * D : NULL,
                 tr->q_mag ? tr->q_mag + (t * Hq + h) * D : NULL);
      }
      for (uint32_t h = 0; h < Hk; ++h) {
        const int64_t dst = row_offset(c, page, 0, layer_idx, slot, h);
        const int64_t so = c->scales ? scale_offset(c, page, 0, layer_idx, slot, h) : -1;
        read_cache_row(c, dst, so, D, hb.x);
        head_math(&hb, D, NULL, dtype, 0.0, 0.0, 1, freqs, pos, R, interleaved, r0);
        store_cache_row(c, dst, so, hb.y, c->pool, dst, c->dtype, D, r0, r0 + R);
        if (tr) {
          record(&hb, D, tr->k_exact ? tr->k_exact + (t * Hk + h) * D : NULL,
                 tr->k_mag ? tr->k_mag + (t * Hk + h) * D : NULL);
          set_off(tr->k_row_off, t * Hk + h, dst);
          set_off(tr->k_scale_off, t * Hk + h, so);
        }
      }
    }
  }
  free(hb.x);
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* fused GEMV + partial RMSNorm                                        */
/* ------------------------------------------------------------------ */

int32_t orc_matmul_fused_partial_rmsnorm(
    void* normed_output, uint64_t normed_row_stride, void* unnormed_output,
    uint64_t unnormed_row_stride, const void* input, uint64_t input_row_stride, uint32_t m,
    const void* weight, uint64_t weight_row_stride, uint32_t n, uint32_t k, const void* gamma,
    uint32_t n_normed, float epsilon, float weight_offset, int32_t dtype, int32_t transpose_b,
    double* y_exact, double* abs_dot, double* r_out) {
  (void)weight_offset; /* not consumed (MatmulFusedPartialRMSNorm page, Args) */
  if (!dtype_ok(dtype) || n_normed > n) return ORC_EINVAL;
  if (m == 0 || n == 0) return ORC_OK;
  if (!input || !weight || (n_normed && (!gamma || !normed_output)) ||
      (n_normed < n && !unnormed_output))
    return ORC_EINVAL;
  double* y = (double*)malloc(sizeof(double) * n);
  if (!y) return ORC_EINVAL;
  for (uint32_t i = 0; i < m; ++i) {
    /* the GEMV: y_j = sum_k x_k B[k][j] with B = W^T (W stored [n][k],
     * transpose_b) or B = W (W stored [k][n]); bf16, f16 and f32 products
     * are exact in double */
    for (uint32_t j = 0; j < n; ++j) {
      double s = 0.0, a = 0.0;
      for (uint32_t kk = 0; kk < k; ++kk) {
        const int64_t widx = transpose_b
                                 ? (int64_t)j * (int64_t)weight_row_stride + kk
                                 : (int64_t)kk * (int64_t)weight_row_stride + j;
        const double p = get(input, dtype, (int64_t)i * (int64_t)input_row_stride + kk) *
                         get(weight, dtype, widx);
        s += p;
        a += fabs(p);
      }
      y[j] = s;
      if (y_exact) y_exact[(uint64_t)i * n + j] = s;
      if (abs_dot) abs_dot[(uint64_t)i * n + j] = a;
    }
    /* RMSNorm over the leading n_normed columns as one vector */
    double r = 0.0;
    if (n_normed) {
      double ss = 0.0;
      for (uint32_t j = 0; j < n_normed; ++j) ss += y[j] * y[j];
      r = 1.0 / sqrt(ss / (double)n_normed + (double)epsilon);
      for (uint32_t j = 0; j < n_normed; ++j)
        put(normed_output, dtype, (int64_t)i * (int64_t)normed_row_stride + j,
            y[j] * r * get(gamma, dtype, j));
    }
    if (r_out) r_out[i] = r;
    /* the trailing columns pass through */
    for (uint32_t j = n_normed; j < n; ++j)
      put(unnormed_output, dtype, (int64_t)i * (int64_t)unnormed_row_stride + (j - n_normed),
          y[j]);
  }
  free(y);
  return ORC_OK;
}
