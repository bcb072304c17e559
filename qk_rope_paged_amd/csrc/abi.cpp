// abi.cpp -- the library's extern "C" entry points: argument checks, the
// launch descriptor of the band engine, and the metadata validator.
//
// Each entry point checks what it can see on the host (pointers, sizes,
// alignment, dtype and geometry), turns the call into at most four row
// segments per token and enqueues one kernel on the caller's stream.  Device
// metadata (offsets, cache lengths, page tables) is never read here; the
// kernel skips tokens whose metadata is out of range and qrp_validate()
// reports it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "engine.hpp"
#include "errors.hpp"
#include "qk_rope_paged.h"

namespace {

thread_local std::string g_err;

int32_t fail(int32_t code, const std::string& msg) {
  g_err = msg;
  return code;
}

}  // namespace

namespace qrp {
int32_t set_error(int32_t code, const std::string& msg) { return fail(code, msg); }
void clear_error() { g_err.clear(); }
}  // namespace qrp

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
uint32_t elem_bytes(int32_t dt) { return dt == QRP_F32 ? 4u : dt == QRP_FP8 ? 1u : 2u; }
uint32_t chunk_elems(int32_t dt) { return 16u / elem_bytes(dt); }
bool dtype_ok(int32_t dt) { return dt == QRP_F32 || dt == QRP_BF16 || dt == QRP_F16; }

// binary32 -> nearest-even bf16 or binary16 -> binary32 (weight_offset is a Scalar[dtype])
float to_dtype(int32_t dt, float v) {
  if (dt == QRP_F32) return v;
  if (dt == QRP_F16) return (float)(_Float16)v;
  uint32_t u;
  std::memcpy(&u, &v, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) {
    u = (u | 0x00400000u) & 0xFFFF0000u;
  } else {
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
  }
  std::memcpy(&v, &u, 4);
  return v;
}

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  return std::atoi(s);
}

// Launch-shape overrides (qrp_set_launch_override), process-wide; -1 lets
// the library choose.  The environment gives the first values, read once
// when the library is loaded.
constexpr int kKnobs = 6;
std::atomic<int32_t> g_knob[kKnobs];

bool knob_value_ok(int32_t knob, int32_t v) {
  if (v == -1) return true;
  switch (knob) {
    case QRP_KNOB_PACK: return v == 0 || v == 1;
    case QRP_KNOB_PASSES_PER_WAVE: return v >= 1 && v <= 8;
    case QRP_KNOB_WAVES_PER_BLOCK: return v >= 1 && v <= qrp::kMaxWavesPerBlock;
    case QRP_KNOB_XCD_REMAP: return v >= 0 && v <= 2;
    case QRP_KNOB_TAIL_UNITS: return v >= 0;
    case QRP_KNOB_LDS_BYTES: return v >= 0 && v <= 65536;
    default: return false;
  }
}

struct KnobInit {
  KnobInit() {
    const char* names[kKnobs] = {"QRP_PACK", "QRP_PASSES_PER_WAVE", "QRP_WAVES_PER_BLOCK",
                                 "QRP_XCD_REMAP", "QRP_TAIL_UNITS", "QRP_LDS_BYTES"};
    for (int k = 0; k < kKnobs; ++k) {
      int v = env_int(names[k], -1);
      // 0 meant "the library's choice" for the two counts
      if ((k == QRP_KNOB_PASSES_PER_WAVE || k == QRP_KNOB_WAVES_PER_BLOCK) && v == 0) v = -1;
      g_knob[k].store(knob_value_ok(k, v) ? v : -1);
    }
  }
} g_knob_init;

int32_t knob(int32_t k) { return g_knob[k].load(std::memory_order_relaxed); }

int32_t check_cache(const qrp_paged_cache* c, int32_t dtype, uint32_t layer_idx, const char* what) {
  const std::string w(what);
  if (!c) return fail(QRP_EINVAL, w + ": cache is NULL");
  if (!c->blocks || !c->cache_lengths || !c->lookup_table)
    return fail(QRP_EINVAL, w + ": blocks, cache_lengths and lookup_table must be non-NULL");
  if (c->dtype != dtype && c->dtype != QRP_FP8)
    return fail(QRP_EUNSUPPORTED, w + ": cache dtype must be the op dtype or QRP_FP8");
  if (c->dtype == QRP_FP8) {
    if (!c->scales) return fail(QRP_EINVAL, w + ": an FP8 cache needs scales");
    if (c->scale_dtype != QRP_F32 && c->scale_dtype != QRP_BF16)
      return fail(QRP_EUNSUPPORTED, w + ": scale_dtype must be QRP_F32 or QRP_BF16");
    if (reinterpret_cast<uintptr_t>(c->scales) & (elem_bytes(c->scale_dtype) - 1))
      return fail(QRP_EALIGN, w + ": scales not aligned to their element size");
    if (c->scale_page_stride < 0 || c->scale_plane_stride < 0 || c->scale_layer_stride < 0 ||
        c->scale_slot_stride < 0 || c->scale_head_stride < 0)
      return fail(QRP_EINVAL, w + ": negative scale stride");
  }
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return fail(QRP_EUNSUPPORTED, w + ": head_dim must be 64, 128 or 256");
  if (c->num_kv_heads == 0 || c->page_size == 0 || c->num_pages == 0 || c->cache_batch == 0 ||
      c->max_pages_per_seq == 0)
    return fail(QRP_EINVAL, w + ": num_kv_heads, page_size, num_pages, cache_batch and "
                                "max_pages_per_seq must be positive");
  if (c->kv_planes != 1 && c->kv_planes != 2) return fail(QRP_EINVAL, w + ": kv_planes must be 1 or 2");
  if (layer_idx >= c->num_layers) return fail(QRP_EINVAL, w + ": layer_idx >= num_layers");
  if (!aligned16(c->blocks)) return fail(QRP_EALIGN, w + ": blocks not 16-byte aligned");
  const int64_t ce = chunk_elems(c->dtype);
  const int64_t st[5] = {c->page_stride, c->plane_stride, c->layer_stride, c->slot_stride,
                         c->head_stride};
  for (int64_t s : st) {
    if (s < 0) return fail(QRP_EINVAL, w + ": negative cache stride");
    if (s % ce) return fail(QRP_EALIGN, w + ": cache strides must be multiples of 16 bytes");
  }
  if ((reinterpret_cast<uintptr_t>(c->cache_lengths) | reinterpret_cast<uintptr_t>(c->lookup_table)) & 3u)
    return fail(QRP_EALIGN, w + ": cache_lengths / lookup_table not 4-byte aligned");
  return QRP_OK;
}

int32_t check_rope(const qrp_rope* r, int32_t dtype, uint32_t head_dim) {
  if (!r || !r->freqs_cis) return fail(QRP_EINVAL, "rope / freqs_cis is NULL");
  if (!dtype_ok(r->freq_dtype))
    return fail(QRP_EUNSUPPORTED, "freq_dtype must be QRP_F32, QRP_BF16 or QRP_F16");
  if (!aligned16(r->freqs_cis)) return fail(QRP_EALIGN, "freqs_cis not 16-byte aligned");
  if (r->max_seq_len == 0) return fail(QRP_EINVAL, "max_seq_len must be positive");
  if (r->rope_tail != 0 && r->rope_tail != 1) return fail(QRP_EINVAL, "rope_tail must be 0 or 1");
  if (r->rope_dim == 0 || r->rope_dim > head_dim || r->rope_dim % 2)
    return fail(QRP_EINVAL, "rope_dim must be even, positive and <= head_dim");
  if (r->rope_dim % (2 * chunk_elems(dtype)))
    return fail(QRP_EUNSUPPORTED, "rope_dim must be a multiple of 32 bytes of dtype");
  return QRP_OK;
}

qrp::CacheDesc make_cache(const qrp_paged_cache* c, uint32_t layer_idx) {
  qrp::CacheDesc d{};
  d.blocks = c->blocks;
  d.page_stride = c->page_stride;
  d.plane_stride = c->plane_stride;
  d.slot_stride = c->slot_stride;
  d.head_stride = c->head_stride;
  d.layer_off = (int64_t)layer_idx * c->layer_stride;
  d.cache_lengths = c->cache_lengths;
  d.table = c->lookup_table;
  d.num_pages = c->num_pages;
  d.max_pages = c->max_pages_per_seq;
  d.page_size = c->page_size;
  d.page_shift = 0xFFFFFFFFu;
  if ((c->page_size & (c->page_size - 1)) == 0) {
    uint32_t s = 0;
    while ((1u << s) < c->page_size) ++s;
    d.page_shift = s;
  }
  d.cache_batch = c->cache_batch;
  return d;
}

// Bit i of the launch's fp8_caches: cache i holds FP8 codes.
uint32_t fp8_bit(const qrp_paged_cache* c, uint32_t i) { return c->dtype == QRP_FP8 ? 1u << i : 0u; }

qrp::ScaleDesc make_scales(const qrp_paged_cache* c, uint32_t layer_idx) {
  qrp::ScaleDesc d{};
  if (c->dtype == QRP_FP8) {
    d.scales = c->scales;
    d.s_page_stride = c->scale_page_stride;
    d.s_plane_stride = c->scale_plane_stride;
    d.s_slot_stride = c->scale_slot_stride;
    d.s_head_stride = c->scale_head_stride;
    d.s_layer_off = (int64_t)layer_idx * c->scale_layer_stride;
    d.scale_bf16 = c->scale_dtype == QRP_BF16;
  }
  return d;
}

// One-pass waves at the end of a multi-pass launch (see Builder::finish).
constexpr uint32_t kTailWaves = 1536;
// LDS reserved per block of a radd launch over a plain cache (an occupancy
// cap; see Builder::finish).
constexpr uint32_t kRaddLdsBytes = 32768;

struct Builder {
  qrp::BandArgs a{};
  int32_t dtype = QRP_BF16;
  uint32_t head_dim = 0;
  uint32_t rpp = 0;
  bool pack = false;  // token-packed passes

  void add_seg(qrp::SegKind kind, const void* src, int64_t src_stride, void* dst, int64_t dst_stride,
               const void* gamma, float eps, uint32_t n_heads, uint32_t cache, uint32_t plane) {
    if (n_heads == 0) return;
    qrp::SegDesc& s = a.seg[a.nseg];
    s.src = src;
    s.dst = dst;
    s.gamma = gamma;
    s.src_row_stride = src_stride;
    s.dst_row_stride = dst_stride;
    s.eps = eps;
    s.n_heads = n_heads;
    s.kind = kind;
    s.cache = cache;
    s.plane = plane;
    s.pass_begin = a.passes_per_token;
    s.n_passes = (n_heads + rpp - 1) / rpp;
    if (kind == qrp::SEG_K_INPLACE) a.inplace_segs |= 1u << a.nseg;
    a.passes_per_token += s.n_passes;
    ++a.nseg;
  }

  // split tokens x passes into waves and blocks (one pass per wave: radd, and
  // the padded grid, whose waves resolve their row with one division).
  // allow_pack: the op has a token-packed build.
  int32_t finish(uint32_t total_tokens, bool radd, bool one_pass = false,
                 bool allow_pack = false, bool norm_build = false) {
    // norm_build: the launch runs the norm kernels whatever its gammas
    bool norm = norm_build;
    for (uint32_t s = 0; s < a.nseg; ++s) norm = norm || a.seg[s].gamma != nullptr;
    // Per-token passes leave lanes idle when a segment's head count is not a
    // multiple of the rows a pass holds (a GPU's share of the heads under
    // head parallelism: 4 Q, 1 K, 1 V heads fill 6 of 24 rows).  Below 85 %
    // of rows filled, the token-packed layout is used: one pass per head,
    // over a block of rpp consecutive tokens (one row each).  The
    // QRP_KNOB_PACK override forces it off / on.
    uint32_t units = total_tokens;  // waves' work units: tokens, or token blocks
    if (allow_pack) {
      uint64_t rows = 0, slots = 0;
      for (uint32_t s = 0; s < a.nseg; ++s) {
        rows += a.seg[s].n_heads;
        slots += (uint64_t)a.seg[s].n_passes * rpp;
      }
      pack = rows * 100 < slots * 85;
      const int32_t forced_pack = knob(QRP_KNOB_PACK);
      if (forced_pack >= 0) pack = forced_pack != 0;
    }
    if (pack) {
      uint32_t pb = 0;
      for (uint32_t s = 0; s < a.nseg; ++s) {
        a.seg[s].pass_begin = pb;
        a.seg[s].n_passes = a.seg[s].n_heads;
        pb += a.seg[s].n_heads;
      }
      a.passes_per_token = pb;
      units = (total_tokens + rpp - 1) / rpp;
    }
    const uint32_t ppt = a.passes_per_token;
    if (ppt == 0) return fail(QRP_EINVAL, "no head rows to process");  // keeps n_items >= 1
    const bool fp8 = a.fp8_caches != 0;
    const uint32_t npmax = qrp::max_passes(radd, norm, pack, fp8);
    uint32_t ppg = std::min<uint32_t>(qrp::default_passes(radd, norm, pack, fp8), ppt);
    const int32_t forced = knob(QRP_KNOB_PASSES_PER_WAVE);
    if (forced > 0) {
      ppg = std::min<uint32_t>((uint32_t)forced, std::min(npmax, ppt));
    } else if (radd || one_pass) {
      // a radd pass already carries two loads per chunk (a and the cache
      // row), and a padded-grid wave's metadata is one division: one pass
      // per wave measured fastest for both
      ppg = 1;
    } else {
      // enough waves to cover every SIMD a few times over: shrink the group.
      // A packed wave resolves the metadata of a block of tokens, so fewer,
      // fuller waves pay off sooner (measured: 2 passes per wave for the
      // store op and 3 for the norm op at 8-way head parallelism's shapes).
      const uint64_t want = pack ? 2048 : 4096;
      while (ppg > 1 && (uint64_t)units * ((ppt + ppg - 1) / ppg) < want) --ppg;
    }
    for (uint32_t i = 1; i < (uint32_t)qrp::kMaxSegs; ++i)
      a.seg_begin[i - 1] = i < a.nseg ? a.seg[i].pass_begin : 0xFFFFFFFFu;
    a.passes_per_group = ppg;
    a.groups_per_token = (ppt + ppg - 1) / ppg;
    int32_t remap = knob(QRP_KNOB_XCD_REMAP);
    if (remap < 0) remap = (pack && ppg == 1) ? 2 : 0;
    // Multi-pass launches end on one-pass waves: the last `tail` units'
    // passes each get a wave of their own, so the grid drains on short
    // waves.  About 1536 such waves, at most a quarter of the units
    // (measured: prefill 33.55 -> 33.31 us, dual 54.30 -> 53.6, dual over
    // FP8 caches 55.6 -> 54.8; tails of 4000 waves and more were slower).
    // Not with every unit's waves on one XCD: that mapping counts groups of
    // passes_per_group.
    uint32_t tail = 0;
    if (ppg > 1 && remap != 2) {
      const int32_t forced_tail = knob(QRP_KNOB_TAIL_UNITS);
      // the store op over FP8 caches drains best on about half as many
      // (prefill over FP8: 34.04 -> 33.73 us with 768 instead of 1536)
      const uint32_t waves = (fp8 && !norm) ? kTailWaves / 2 : kTailWaves;
      tail = forced_tail >= 0 ? std::min<uint32_t>((uint32_t)forced_tail, units)
                              : std::min<uint32_t>((waves + ppt - 1) / ppt, units / 4);
    }
    const uint64_t head_units = units - tail;
    const uint64_t items = head_units * a.groups_per_token + (uint64_t)tail * ppt;
    if (items >= (1ull << 31)) return fail(QRP_EINVAL, "batch too large for one launch");
    a.n_items = (uint32_t)items;
    a.tail_item = (uint32_t)(head_units * a.groups_per_token);
    a.tail_unit = (uint32_t)head_units;
    // Rope/store launches of one pass per wave (decode-sized batches, the
    // padded grid) run two waves per block, large multi-pass ones one wave
    // per block, norm, radd and the other small launches four (measured:
    // decode 3.09 -> 3.01 us per launch with two instead of four, the padded
    // grid 49.11 -> 48.98 with two instead of one).
    uint32_t wpb = (uint32_t)qrp::kMaxWavesPerBlock;
    if (!radd && !norm) wpb = ppg == 1 ? 2u : (items >= 8192 ? 1u : wpb);
    const int32_t forced_wpb = knob(QRP_KNOB_WAVES_PER_BLOCK);
    if (forced_wpb > 0) wpb = std::min<uint32_t>((uint32_t)forced_wpb, qrp::kMaxWavesPerBlock);
    a.waves_per_block = wpb;
    // radd over a plain cache streams best with at most 5 blocks (20 waves)
    // resident per compute unit: reserving 32 KB of the 160 KB LDS per block
    // caps it (measured: 19.59 -> 18.99 us on the radd workload; 4 blocks
    // gave the same, 3 were 21 % slower, and the cap slowed radd over FP8
    // caches, the prefill and the padded grid).
    const int32_t forced_lds = knob(QRP_KNOB_LDS_BYTES);
    a.lds_bytes = forced_lds >= 0 ? (uint32_t)forced_lds
                  : (radd && a.fp8_caches == 0 && !pack && wpb == 4) ? kRaddLdsBytes : 0u;
    a.n_blocks = (uint32_t)((items + wpb - 1) / wpb);
    // Token-packed launches of one pass per wave (a decode batch's share
    // of the heads) keep each token block's waves on one XCD, so they share
    // its L2 for their metadata and freqs rows (decode at 8-way head
    // parallelism: 3.08 -> 2.86 us per launch).  Everything else is dealt
    // round-robin: keeping units on one XCD measured 1-6 % slower there.
    a.per_xcd = remap == 1 ? (a.n_blocks + qrp::kXcds - 1) / qrp::kXcds : 0;
    if (remap == 2) {
      // every unit's waves on one XCD: bpu blocks per unit, units dealt to
      // the XCDs in turn
      const uint64_t bpu = (a.groups_per_token + wpb - 1) / wpb;
      const uint64_t per = (units + qrp::kXcds - 1) / qrp::kXcds;
      const uint64_t blocks = (uint64_t)qrp::kXcds * bpu * per;
      if (blocks >= (1ull << 31)) return fail(QRP_EINVAL, "batch too large for one launch");
      a.per_xcd = qrp::kUnitsOnXcd | (uint32_t)bpu;
      a.n_blocks = (uint32_t)blocks;
    }
    a.total_tokens = total_tokens;
    a.guess_mul = (((uint64_t)a.batch) << 32) / total_tokens;
    return QRP_OK;
  }
};

int32_t launch(const Builder& b, bool interleaved, bool radd, void* stream, bool bshd = false,
               int32_t q_dtype = -1) {
  qrp::LaunchSpec s{};
  s.dtype = b.dtype;
  s.q_dtype = q_dtype < 0 ? b.dtype : q_dtype;
  // one plain and one FP8 cache: the mixed build; otherwise every cache alike
  s.cache_mixed = b.a.ncache == 2 && (b.a.fp8_caches == 1u || b.a.fp8_caches == 2u);
  s.cache_fp8 = b.a.fp8_caches != 0 && !s.cache_mixed;
  s.head_dim = b.head_dim;
  s.interleaved = interleaved;
  s.radd = radd;
  s.bshd = bshd;
  s.pack = b.pack;
  const int e = qrp::launch_band(b.a, s, stream);
  if (e != 0)
    return fail(QRP_EHIP, std::string("kernel launch failed: ") +
                               hipGetErrorString(static_cast<hipError_t>(e)));
  return QRP_OK;
}

const char* elem_ptr(const void* base, uint64_t elems, int32_t dt) {
  return static_cast<const char*>(base) + elems * elem_bytes(dt);
}

int32_t check_batch(const uint32_t* offsets, uint32_t T, uint32_t B) {
  if (!offsets) return fail(QRP_EINVAL, "input_row_offsets is NULL");
  if (B == 0) return fail(QRP_EINVAL, "batch_size is 0 with total_seq_len > 0");
  if (reinterpret_cast<uintptr_t>(offsets) & 3u) return fail(QRP_EALIGN, "input_row_offsets not 4-byte aligned");
  (void)T;
  return QRP_OK;
}

int32_t check_band(const qrp_band* band, int32_t dtype, uint64_t row_stride, uint32_t layer_idx,
                   const char* what) {
  const std::string w(what);
  if (!band) return fail(QRP_EINVAL, w + " is NULL");
  int32_t st = check_cache(band->cache, dtype, layer_idx, what);
  if (st) return st;
  const uint64_t D = band->cache->head_dim, Hk = band->cache->num_kv_heads;
  const uint32_t ce = chunk_elems(dtype);
  if (band->n_q_heads) {
    if (!band->q_output) return fail(QRP_EINVAL, w + ": q_output is NULL");
    if (!aligned16(band->q_output)) return fail(QRP_EALIGN, w + ": q_output not 16-byte aligned");
    if (band->q_out_row_stride % ce) return fail(QRP_EALIGN, w + ": q_out_row_stride not a multiple of 16 bytes");
    if (band->q_out_row_stride < band->n_q_heads * D) return fail(QRP_EINVAL, w + ": q_out_row_stride < n_q_heads * head_dim");
    if (band->q_col % ce) return fail(QRP_EALIGN, w + ": q_col not a multiple of 16 bytes");
    if (band->q_col + band->n_q_heads * D > row_stride) return fail(QRP_EINVAL, w + ": Q columns exceed the row");
  }
  if (band->k_col >= 0) {
    if ((uint64_t)band->k_col % ce) return fail(QRP_EALIGN, w + ": k_col not a multiple of 16 bytes");
    if ((uint64_t)band->k_col + Hk * D > row_stride) return fail(QRP_EINVAL, w + ": K columns exceed the row");
  }
  if (band->v_col >= 0) {
    if (band->k_col < 0) return fail(QRP_EINVAL, w + ": v_col needs k_col >= 0");
    if (band->cache->kv_planes != 2) return fail(QRP_EINVAL, w + ": v_col needs a cache with a V plane");
    if ((uint64_t)band->v_col % ce) return fail(QRP_EALIGN, w + ": v_col not a multiple of 16 bytes");
    if ((uint64_t)band->v_col + Hk * D > row_stride) return fail(QRP_EINVAL, w + ": V columns exceed the row");
  }
  if ((band->q_gamma && !aligned16(band->q_gamma)) || (band->k_gamma && !aligned16(band->k_gamma)))
    return fail(QRP_EALIGN, w + ": gamma not 16-byte aligned");
  return QRP_OK;
}

void add_band(Builder& b, const qrp_band* band, const void* buf, uint64_t row_stride, int32_t dtype,
              uint32_t cache_slot) {
  const uint64_t D = band->cache->head_dim;
  const uint32_t Hk = band->cache->num_kv_heads;
  b.add_seg(qrp::SEG_Q, elem_ptr(buf, band->q_col, dtype), (int64_t)row_stride, band->q_output,
            (int64_t)band->q_out_row_stride, band->q_gamma, band->epsilon, band->n_q_heads, cache_slot, 0);
  if (band->k_col >= 0)
    b.add_seg(qrp::SEG_K_BUF, elem_ptr(buf, (uint64_t)band->k_col, dtype), (int64_t)row_stride,
              nullptr, 0, band->k_gamma, band->epsilon, Hk, cache_slot, 0);
  else
    b.add_seg(qrp::SEG_K_INPLACE, nullptr, 0, nullptr, 0, band->k_gamma, band->epsilon, Hk,
              cache_slot, 0);
  if (band->v_col >= 0)
    b.add_seg(qrp::SEG_V_COPY, elem_ptr(buf, (uint64_t)band->v_col, dtype), (int64_t)row_stride,
              nullptr, 0, nullptr, 0.f, Hk, cache_slot, 1);
  (void)D;
}

}  // namespace

extern "C" {

const char* qrp_last_error(void) { return g_err.c_str(); }

int32_t qrp_abi_version(void) { return QRP_ABI_VERSION; }

int32_t qrp_set_launch_override(int32_t knob_id, int32_t value, int32_t* previous) {
  g_err.clear();
  if (knob_id < 0 || knob_id >= kKnobs) return fail(QRP_EINVAL, "unknown launch knob");
  if (!knob_value_ok(knob_id, value)) return fail(QRP_EINVAL, "launch knob value out of range");
  const int32_t old = g_knob[knob_id].exchange(value);
  if (previous) *previous = old;
  return QRP_OK;
}

int32_t rope_split_store_paged(const void* qkv, int32_t dtype, uint32_t total_seq_len,
                               uint64_t qkv_row_stride, uint32_t n_q_heads,
                               const uint32_t* input_row_offsets, uint32_t batch_size,
                               const qrp_rope* rope, const qrp_paged_cache* cache,
                               uint32_t layer_idx, void* q_output, int32_t q_out_dtype,
                               uint64_t q_out_row_stride, void* stream) {
  g_err.clear();
  if (!dtype_ok(dtype)) return fail(QRP_EUNSUPPORTED, "dtype must be QRP_F32, QRP_BF16 or QRP_F16");
  if (!dtype_ok(q_out_dtype))
    return fail(QRP_EUNSUPPORTED, "q_out_dtype must be QRP_F32, QRP_BF16 or QRP_F16");
  if (total_seq_len == 0) return QRP_OK;
  int32_t st;
  if ((st = check_batch(input_row_offsets, total_seq_len, batch_size))) return st;
  if ((st = check_cache(cache, dtype, layer_idx, "cache"))) return st;
  if (cache->kv_planes != 2) return fail(QRP_EINVAL, "cache needs K and V planes");
  if ((st = check_rope(rope, dtype, cache->head_dim))) return st;
  if (!qkv || !q_output) return fail(QRP_EINVAL, "qkv / q_output is NULL");
  if (n_q_heads == 0) return fail(QRP_EINVAL, "n_q_heads is 0");
  if (!aligned16(qkv) || !aligned16(q_output)) return fail(QRP_EALIGN, "qkv / q_output not 16-byte aligned");
  if (qkv_row_stride % chunk_elems(dtype) || q_out_row_stride % chunk_elems(q_out_dtype))
    return fail(QRP_EALIGN, "row strides must be multiples of 16 bytes");
  const uint64_t D = cache->head_dim, Hk = cache->num_kv_heads;
  if (qkv_row_stride < (n_q_heads + 2 * Hk) * D) return fail(QRP_EINVAL, "qkv_row_stride < q_dim + k_dim + v_dim");
  if (q_out_row_stride < n_q_heads * D) return fail(QRP_EINVAL, "q_out_row_stride < q_dim");
  if (batch_size > cache->cache_batch) return fail(QRP_EINVAL, "batch_size > cache_batch");

  Builder b;
  b.dtype = dtype;
  b.head_dim = cache->head_dim;
  b.rpp = qrp::rows_per_pass(dtype, cache->head_dim);
  b.a.cache[0] = make_cache(cache, layer_idx);
  b.a.scale[0] = make_scales(cache, layer_idx);
  b.a.fp8_caches = fp8_bit(cache, 0);
  b.a.ncache = 1;
  b.a.offsets = input_row_offsets;
  b.a.batch = batch_size;
  b.a.batch_offset = 0;
  b.a.freqs = rope->freqs_cis;
  b.a.freq_dtype = (uint32_t)rope->freq_dtype;
  b.a.rope_dim = rope->rope_dim;
  b.a.rope_off_chunks = rope->rope_tail ? (b.head_dim - rope->rope_dim) / chunk_elems(dtype) : 0;
  b.a.max_seq_len = rope->max_seq_len;
  b.a.multiply_before_cast = 1;
  b.add_seg(qrp::SEG_Q, qkv, (int64_t)qkv_row_stride, q_output, (int64_t)q_out_row_stride, nullptr,
            0.f, n_q_heads, 0, 0);
  b.add_seg(qrp::SEG_K_BUF, elem_ptr(qkv, n_q_heads * D, dtype), (int64_t)qkv_row_stride, nullptr,
            0, nullptr, 0.f, (uint32_t)Hk, 0, 0);
  b.add_seg(qrp::SEG_V_COPY, elem_ptr(qkv, (n_q_heads + Hk) * D, dtype), (int64_t)qkv_row_stride,
            nullptr, 0, nullptr, 0.f, (uint32_t)Hk, 0, 1);
  if ((st = b.finish(total_seq_len, false, false, true))) return st;
  return launch(b, rope->interleaved != 0, false, stream, false, q_out_dtype);
}

int32_t qk_rmsnorm_rope_paged(const void* qkv, int32_t dtype, uint32_t total_seq_len,
                              uint64_t qkv_row_stride, const qrp_band* band, float weight_offset,
                              int32_t multiply_before_cast, const uint32_t* input_row_offsets,
                              uint32_t batch_size, const qrp_rope* rope, uint32_t layer_idx,
                              void* stream) {
  g_err.clear();
  if (!dtype_ok(dtype)) return fail(QRP_EUNSUPPORTED, "dtype must be QRP_F32, QRP_BF16 or QRP_F16");
  if (total_seq_len == 0) return QRP_OK;
  int32_t st;
  if ((st = check_batch(input_row_offsets, total_seq_len, batch_size))) return st;
  if (!qkv) return fail(QRP_EINVAL, "qkv is NULL");
  if (!aligned16(qkv)) return fail(QRP_EALIGN, "qkv not 16-byte aligned");
  if (qkv_row_stride % chunk_elems(dtype)) return fail(QRP_EALIGN, "qkv_row_stride not a multiple of 16 bytes");
  if ((st = check_band(band, dtype, qkv_row_stride, layer_idx, "band"))) return st;
  if ((st = check_rope(rope, dtype, band->cache->head_dim))) return st;
  if (batch_size > band->cache->cache_batch) return fail(QRP_EINVAL, "batch_size > cache_batch");

  Builder b;
  b.dtype = dtype;
  b.head_dim = band->cache->head_dim;
  b.rpp = qrp::rows_per_pass(dtype, b.head_dim);
  b.a.cache[0] = make_cache(band->cache, layer_idx);
  b.a.scale[0] = make_scales(band->cache, layer_idx);
  b.a.fp8_caches = fp8_bit(band->cache, 0);
  b.a.ncache = 1;
  b.a.offsets = input_row_offsets;
  b.a.batch = batch_size;
  b.a.freqs = rope->freqs_cis;
  b.a.freq_dtype = (uint32_t)rope->freq_dtype;
  b.a.rope_dim = rope->rope_dim;
  b.a.rope_off_chunks = rope->rope_tail ? (b.head_dim - rope->rope_dim) / chunk_elems(dtype) : 0;
  b.a.max_seq_len = rope->max_seq_len;
  b.a.weight_offset = to_dtype(dtype, weight_offset);
  b.a.multiply_before_cast = multiply_before_cast != 0;
  add_band(b, band, qkv, qkv_row_stride, dtype, 0);
  if ((st = b.finish(total_seq_len, false, false, true))) return st;
  return launch(b, rope->interleaved != 0, false, stream);
}

int32_t dual_band(const void* buf, int32_t dtype, uint32_t total_seq_len, uint64_t buf_row_stride,
                  const qrp_band* main_band, const qrp_band* index_band, float weight_offset,
                  int32_t multiply_before_cast, const uint32_t* input_row_offsets,
                  uint32_t batch_size, const qrp_rope* rope, uint32_t layer_idx, void* stream) {
  g_err.clear();
  if (!dtype_ok(dtype)) return fail(QRP_EUNSUPPORTED, "dtype must be QRP_F32, QRP_BF16 or QRP_F16");
  if (!main_band || !index_band || !main_band->cache || !index_band->cache)
    return fail(QRP_EINVAL, "bands and their caches must be non-NULL");
  if (main_band->cache->head_dim != index_band->cache->head_dim)
    return fail(QRP_EGEOMETRY, "main and index bands differ in head_dim");
  if (total_seq_len == 0) return QRP_OK;
  int32_t st;
  if ((st = check_batch(input_row_offsets, total_seq_len, batch_size))) return st;
  if (!buf) return fail(QRP_EINVAL, "buffer is NULL");
  if (!aligned16(buf)) return fail(QRP_EALIGN, "buffer not 16-byte aligned");
  if (buf_row_stride % chunk_elems(dtype)) return fail(QRP_EALIGN, "buf_row_stride not a multiple of 16 bytes");
  if ((st = check_band(main_band, dtype, buf_row_stride, layer_idx, "main_band"))) return st;
  if ((st = check_band(index_band, dtype, buf_row_stride, layer_idx, "index_band"))) return st;
  if (main_band->v_col >= 0 || index_band->v_col >= 0)
    return fail(QRP_EUNSUPPORTED, "dual_band carries no V rows (v_col must be < 0)");
  if ((st = check_rope(rope, dtype, main_band->cache->head_dim))) return st;
  if (batch_size > main_band->cache->cache_batch || batch_size > index_band->cache->cache_batch)
    return fail(QRP_EINVAL, "batch_size > cache_batch");

  Builder b;
  b.dtype = dtype;
  b.head_dim = main_band->cache->head_dim;
  b.rpp = qrp::rows_per_pass(dtype, b.head_dim);
  b.a.cache[0] = make_cache(main_band->cache, layer_idx);
  b.a.scale[0] = make_scales(main_band->cache, layer_idx);
  b.a.cache[1] = make_cache(index_band->cache, layer_idx);
  b.a.scale[1] = make_scales(index_band->cache, layer_idx);
  b.a.fp8_caches = fp8_bit(main_band->cache, 0) | fp8_bit(index_band->cache, 1);
  b.a.ncache = 2;
  b.a.offsets = input_row_offsets;
  b.a.batch = batch_size;
  b.a.freqs = rope->freqs_cis;
  b.a.freq_dtype = (uint32_t)rope->freq_dtype;
  b.a.rope_dim = rope->rope_dim;
  b.a.rope_off_chunks = rope->rope_tail ? (b.head_dim - rope->rope_dim) / chunk_elems(dtype) : 0;
  b.a.max_seq_len = rope->max_seq_len;
  b.a.weight_offset = to_dtype(dtype, weight_offset);
  b.a.multiply_before_cast = multiply_before_cast != 0;
  // rows [q_main | k_main | q_index | k_index]
  add_band(b, main_band, buf, buf_row_stride, dtype, 0);
  add_band(b, index_band, buf, buf_row_stride, dtype, 1);
  // a plain cache beside an FP8 one: the mixed build, per-token layout only
  const bool mixed = (main_band->cache->dtype == QRP_FP8) != (index_band->cache->dtype == QRP_FP8);
  if ((st = b.finish(total_seq_len, false, false, !mixed, mixed))) return st;
  return launch(b, rope->interleaved != 0, false, stream);
}

int32_t kv_cache_radd(const void* a, int32_t dtype, uint32_t total_rows, uint64_t a_row_stride,
                      const uint32_t* input_row_offsets, uint32_t batch_size, uint32_t batch_offset,
                      const qrp_paged_cache* cache, uint32_t layer_idx, void* stream) {
  g_err.clear();
  if (!dtype_ok(dtype)) return fail(QRP_EUNSUPPORTED, "dtype must be QRP_F32, QRP_BF16 or QRP_F16");
  if (total_rows == 0) return QRP_OK;
  int32_t st;
  if ((st = check_batch(input_row_offsets, total_rows, batch_size))) return st;
  if ((st = check_cache(cache, dtype, layer_idx, "cache"))) return st;
  if (cache->kv_planes != 2) return fail(QRP_EINVAL, "cache needs K and V planes");
  if (!a) return fail(QRP_EINVAL, "a is NULL");
  if (!aligned16(a)) return fail(QRP_EALIGN, "a not 16-byte aligned");
  if (a_row_stride % chunk_elems(dtype)) return fail(QRP_EALIGN, "a_row_stride not a multiple of 16 bytes");
  const uint64_t D = cache->head_dim, Hk = cache->num_kv_heads;
  if (a_row_stride < 2 * Hk * D) return fail(QRP_EINVAL, "a_row_stride < 2 * num_kv_heads * head_dim");
  if ((uint64_t)batch_offset + batch_size > cache->cache_batch)
    return fail(QRP_EINVAL, "batch_offset + batch_size > cache_batch");

  Builder b;
  b.dtype = dtype;
  b.head_dim = cache->head_dim;
  b.rpp = qrp::rows_per_pass(dtype, b.head_dim);
  b.a.cache[0] = make_cache(cache, layer_idx);
  b.a.scale[0] = make_scales(cache, layer_idx);
  b.a.fp8_caches = fp8_bit(cache, 0);
  b.a.ncache = 1;
  b.a.offsets = input_row_offsets;
  b.a.batch = batch_size;
  b.a.batch_offset = batch_offset;
  b.a.max_seq_len = 0;
  b.add_seg(qrp::SEG_RADD, a, (int64_t)a_row_stride, nullptr, 0, nullptr, 0.f, (uint32_t)Hk, 0, 0);
  b.add_seg(qrp::SEG_RADD, elem_ptr(a, Hk * D, dtype), (int64_t)a_row_stride, nullptr, 0, nullptr,
            0.f, (uint32_t)Hk, 0, 1);
  if ((st = b.finish(total_rows, true, false, true))) return st;
  return launch(b, true, true, stream);
}

int32_t fused_qk_rope_bshd_continuous_batch(const void* q_proj, int32_t dtype, uint32_t batch_size,
                                            uint32_t seq_len, uint32_t n_q_heads,
                                            const uint32_t* valid_lengths, const qrp_rope* rope,
                                            const qrp_paged_cache* cache, uint32_t layer_idx,
                                            void* output, void* stream) {
  g_err.clear();
  if (!dtype_ok(dtype)) return fail(QRP_EUNSUPPORTED, "dtype must be QRP_F32, QRP_BF16 or QRP_F16");
  if (batch_size == 0 || seq_len == 0) return QRP_OK;
  int32_t st;
  if ((st = check_cache(cache, dtype, layer_idx, "cache"))) return st;
  if ((st = check_rope(rope, dtype, cache->head_dim))) return st;
  if (!q_proj || !output || !valid_lengths)
    return fail(QRP_EINVAL, "q_proj / output / valid_lengths is NULL");
  if (n_q_heads == 0) return fail(QRP_EINVAL, "n_q_heads is 0");
  if (!aligned16(q_proj) || !aligned16(output))
    return fail(QRP_EALIGN, "q_proj / output not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(valid_lengths) & 3u)
    return fail(QRP_EALIGN, "valid_lengths not 4-byte aligned");
  if (batch_size > cache->cache_batch) return fail(QRP_EINVAL, "batch_size > cache_batch");
  const uint64_t tokens = (uint64_t)batch_size * seq_len;
  if (tokens >= (1ull << 31)) return fail(QRP_EINVAL, "batch_size * seq_len too large for one launch");
  const uint64_t row = (uint64_t)n_q_heads * cache->head_dim;

  Builder b;
  b.dtype = dtype;
  b.head_dim = cache->head_dim;
  b.rpp = qrp::rows_per_pass(dtype, cache->head_dim);
  b.a.cache[0] = make_cache(cache, layer_idx);
  b.a.scale[0] = make_scales(cache, layer_idx);
  b.a.fp8_caches = fp8_bit(cache, 0);
  b.a.ncache = 1;
  b.a.offsets = nullptr;
  b.a.batch = batch_size;
  b.a.batch_offset = 0;
  b.a.valid_lengths = valid_lengths;
  b.a.seq_len = seq_len;
  b.a.freqs = rope->freqs_cis;
  b.a.freq_dtype = (uint32_t)rope->freq_dtype;
  b.a.rope_dim = rope->rope_dim;
  b.a.rope_off_chunks = rope->rope_tail ? (b.head_dim - rope->rope_dim) / chunk_elems(dtype) : 0;
  b.a.max_seq_len = rope->max_seq_len;
  b.a.multiply_before_cast = 1;
  b.add_seg(qrp::SEG_Q, q_proj, (int64_t)row, output, (int64_t)row, nullptr, 0.f, n_q_heads, 0, 0);
  b.add_seg(qrp::SEG_K_INPLACE, nullptr, 0, nullptr, 0, nullptr, 0.f, cache->num_kv_heads, 0, 0);
  if ((st = b.finish((uint32_t)tokens, false, true, true))) return st;
  return launch(b, rope->interleaved != 0, false, stream, true);
}

int32_t qrp_validate_host(const uint32_t* off, uint32_t B, uint32_t T, uint32_t batch_offset,
                          const uint32_t* cache_lengths, const uint32_t* table, uint32_t cache_batch,
                          uint32_t max_pages, uint32_t page_size, uint64_t num_pages,
                          uint32_t max_seq_len) {
  g_err.clear();
  if (!off) return fail(QRP_EINVAL, "offsets is NULL");
  if (T > 0 && (!cache_lengths || !table)) return fail(QRP_EINVAL, "cache metadata is NULL");
  if (page_size == 0) return fail(QRP_EINVAL, "page_size is 0");
  if (off[0] != 0) return fail(QRP_EDATA, "input_row_offsets[0] != 0");
  for (uint32_t b = 0; b < B; ++b)
    if (off[b + 1] < off[b])
      return fail(QRP_EDATA, "input_row_offsets decrease at " + std::to_string(b + 1));
  if (off[B] != T) return fail(QRP_EDATA, "input_row_offsets[batch_size] != total_seq_len");
  if ((uint64_t)batch_offset + B > cache_batch) return fail(QRP_EDATA, "batch_offset + batch_size > cache_batch");
  std::vector<uint64_t> rows;
  rows.reserve(T);
  for (uint32_t b = 0; b < B; ++b) {
    const uint32_t s = b + batch_offset;
    for (uint32_t t = off[b]; t < off[b + 1]; ++t) {
      const uint64_t pos = (uint64_t)cache_lengths[s] + (t - off[b]);
      if (max_seq_len && pos >= max_seq_len)
        return fail(QRP_EDATA, "token " + std::to_string(t) + ": position " + std::to_string(pos) +
                                   " >= max_seq_len");
      const uint64_t pidx = pos / page_size;
      if (pidx >= max_pages)
        return fail(QRP_EDATA, "token " + std::to_string(t) + ": page index beyond max_pages_per_seq");
      const uint64_t page = table[(uint64_t)s * max_pages + pidx];
      if (page >= num_pages)
        return fail(QRP_EDATA, "token " + std::to_string(t) + ": page id " + std::to_string(page) +
                                   " >= num_pages");
      rows.push_back(page * page_size + pos % page_size);
    }
  }
  std::sort(rows.begin(), rows.end());
  if (std::adjacent_find(rows.begin(), rows.end()) != rows.end())
    return fail(QRP_EDATA, "two tokens write the same cache row (shared page)");
  return QRP_OK;
}

int32_t qrp_validate(const uint32_t* input_row_offsets, uint32_t batch_size, uint32_t total_seq_len,
                     uint32_t batch_offset, const qrp_paged_cache* cache, uint32_t max_seq_len,
                     void* stream) {
  g_err.clear();
  if (!input_row_offsets || !cache || !cache->cache_lengths || !cache->lookup_table)
    return fail(QRP_EINVAL, "NULL metadata");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::vector<uint32_t> off(batch_size + 1ull), lens(cache->cache_batch),
      table((uint64_t)cache->cache_batch * cache->max_pages_per_seq);
  hipError_t e = hipMemcpyAsync(off.data(), input_row_offsets, off.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(lens.data(), cache->cache_lengths, lens.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(table.data(), cache->lookup_table, table.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(QRP_EHIP, std::string("metadata copy failed: ") + hipGetErrorString(e));
  return qrp_validate_host(off.data(), batch_size, total_seq_len, batch_offset, lens.data(),
                           table.data(), cache->cache_batch, cache->max_pages_per_seq,
                           cache->page_size, cache->num_pages, max_seq_len);
}

}  // extern "C"
