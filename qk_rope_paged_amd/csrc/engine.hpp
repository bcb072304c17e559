// engine.hpp -- launch descriptor of the band engine (internal to the library).
//
// Every operation of the library is one launch of the same kernel family.
// A token's head rows are grouped into at most four SEGMENTS, each a run of
// heads with one role:
//
//   SEG_Q        read from the input buffer, optionally normalised, rotated,
//                written to a dense output row            (Q of every op)
//   SEG_K_BUF    read from the buffer, optionally normalised, rotated,
//                written to the K plane of a paged cache   (store ops)
//   SEG_K_INPLACE read from the K plane of a paged cache, normalised,
//                rotated, written back to the same row     (norm ops, K in cache)
//   SEG_V_COPY   read from the buffer, written bit for bit to the V plane
//   SEG_RADD     read from the buffer, added to a cache row in binary32
//
// A wave processes one token's rows in PASSES of RPP rows (64 lanes, D/16
// lanes per row when rows are bf16 x 128).  Segment s covers passes
// [pass_begin, pass_begin + n_passes) of the token.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace qrp {

enum SegKind : uint32_t {
  SEG_Q = 0,
  SEG_K_BUF = 1,
  SEG_K_INPLACE = 2,
  SEG_V_COPY = 3,
  SEG_RADD = 4,
};

constexpr int kMaxSegs = 4;
constexpr int kMaxCaches = 2;
constexpr int kMaxWavesPerBlock = 4;
constexpr int kThreads = 64 * kMaxWavesPerBlock;  // launch bound; blocks may be smaller
constexpr int kXcds = 8;
constexpr uint32_t kUnitsOnXcd = 0x80000000u;  // BandArgs::per_xcd flag

// Passes (rows of 64 lanes) one wave may hold in registers at once, and
// how many it runs by default.  Waves that each move about 4 KB stream best
// on MI355X (measured with plain copies and with this kernel): 2 passes of
// rope/store rows, 2 or 3 of norm rows (below), 1 of radd rows (each radd
// pass reads two operands).  The per-token store kernels are built for up to 3 passes and
// run 2: that build ran the prefill 1 % faster at 2 passes than a build for
// 2 (same-box A/B, twice), while 3 passes per wave were 7 % slower; the
// token-packed store kernels are built for 2 (the 3-pass build ran them 1 %
// slower).
#ifndef QRP_MAX_PASSES_STORE
#define QRP_MAX_PASSES_STORE 3
#endif
#ifndef QRP_MAX_PASSES_STORE_PACK
#define QRP_MAX_PASSES_STORE_PACK 2
#endif
// The norm kernels hold 3 passes, except per-token launches over plain
// caches, built for 2: that build needs 95 VGPRs against 103, which leaves
// room for a fifth wave per SIMD (dual 53.54 -> 52.39 us); over FP8 caches
// and in the token-packed layout the 2-pass build was 11 % and 6 % slower.
#ifndef QRP_MAX_PASSES_NORM
#define QRP_MAX_PASSES_NORM 3
#endif
#ifndef QRP_MAX_PASSES_NORM_PLAIN
#define QRP_MAX_PASSES_NORM_PLAIN 2
#endif
#ifndef QRP_MAX_PASSES_RADD
#define QRP_MAX_PASSES_RADD 2
#endif
constexpr int kMaxPassesStore = QRP_MAX_PASSES_STORE;
constexpr int kMaxPassesStorePack = QRP_MAX_PASSES_STORE_PACK;
constexpr int kDefaultPassesStore = 2;
constexpr int kMaxPassesNorm = QRP_MAX_PASSES_NORM;
constexpr int kMaxPassesNormPlain = QRP_MAX_PASSES_NORM_PLAIN;
constexpr int kMaxPassesRadd = QRP_MAX_PASSES_RADD;

struct SegDesc {
  // what a wave reads before its first buffer load: one 32-byte scalar load
  const void* src;          // buffer elements, already offset to the segment's first column
  int64_t src_row_stride;   // elements between tokens in src
  uint32_t kind;            // SegKind
  uint32_t pass_begin;
  uint32_t n_heads;
  uint32_t cache;           // cache slot (0 / 1) for the row address and position
  // the rest, read after the metadata chain
  void* dst;                // dense output (SEG_Q)
  int64_t dst_row_stride;   // elements between tokens in dst
  const void* gamma;        // [D] of dtype, or nullptr: no norm
  float eps;
  uint32_t plane;           // cache plane written / read
  uint32_t n_passes;
  uint32_t pad_;
};

struct CacheDesc {
  void* blocks;             // element base
  int64_t page_stride, plane_stride, slot_stride, head_stride;
  int64_t layer_off;        // layer_idx * layer_stride
  const uint32_t* cache_lengths;
  const uint32_t* table;
  uint64_t num_pages;
  uint32_t max_pages;
  uint32_t page_size;
  uint32_t page_shift;      // log2(page_size) when a power of two, else 0xFFFFFFFF
  uint32_t cache_batch;
};

// FP8 caches: one scale per (page, plane, layer, slot, head) row.  Kept
// apart from CacheDesc (at the end of the kernel arguments) so that the
// fields every launch reads keep compact, fixed offsets.
struct ScaleDesc {
  void* scales;
  int64_t s_page_stride, s_plane_stride, s_slot_stride, s_head_stride;
  int64_t s_layer_off;      // layer_idx * scale layer stride
  uint32_t scale_bf16;      // scales stored as bf16 (else binary32)
  uint32_t pad_;
};

struct BandArgs {
  // Everything a wave needs before its segment lookup, in the first 64
  // bytes, so that the prologue is one round of scalar loads.
  uint32_t n_items;         // total_tokens * groups_per_token waves of work
  uint32_t n_blocks;        // blocks holding work
  uint32_t waves_per_block; // 1 .. kMaxWavesPerBlock
  uint32_t per_xcd;         // blocks per XCD after the XCD-contiguous remap (0: no remap);
                            // kUnitsOnXcd | b: each unit's waves in b blocks of one XCD
  uint32_t passes_per_token;
  uint32_t passes_per_group;
  uint32_t groups_per_token;
  uint32_t inplace_segs;    // bit i: segment i reads its rows from the cache (SEG_K_INPLACE)
  uint32_t seg_begin[kMaxSegs - 1];  // seg[i + 1].pass_begin, 0xFFFFFFFF past nseg
  uint32_t rope_dim;
  uint32_t rope_off_chunks; // first rotated 16-byte chunk of a head (0: the leading dims)
  uint32_t batch;
  uint32_t nseg;
  uint32_t ncache;
  SegDesc seg[kMaxSegs];
  CacheDesc cache[kMaxCaches];
  const uint32_t* offsets;  // [batch + 1]
  const void* freqs;        // [max_seq_len][rope_dim] of freq_dtype
  uint32_t total_tokens;
  uint32_t batch_offset;
  uint32_t max_seq_len;     // 0: positions unchecked (no rotation)
  float weight_offset;      // already rounded to the dtype
  uint32_t multiply_before_cast;
  uint64_t guess_mul;       // floor(batch * 2^32 / total_tokens): token -> first sequence guess
  uint32_t freq_dtype;      // DT_F32, DT_BF16 or DT_F16 table entries
  uint32_t fp8_caches;      // bit i: cache i holds FP8 codes (the mixed-cache build reads it)
  // Padded [batch][seq_len] token grid (continuous batching): token t is
  // row t % seq_len of sequence t / seq_len; rows at or past the sequence's
  // valid length pass through.  Unused by the ragged ops.
  const uint32_t* valid_lengths;
  uint32_t seq_len;
  // The launch's last units run one pass per wave: items [tail_item,
  // n_items) are unit tail_unit + r / passes_per_token, pass
  // r % passes_per_token (r = item - tail_item).  Shorter waves at the end
  // of the grid let it drain sooner.  tail_item == n_items: no tail.
  uint32_t tail_item;
  uint32_t tail_unit;
  // Host side only: dynamic LDS reserved per block at launch (unused by the
  // kernel), which caps the blocks resident on a compute unit.
  uint32_t lds_bytes;
  ScaleDesc scale[kMaxCaches];
};
static_assert(offsetof(BandArgs, seg) == 64, "the hot header fills one 64-byte line");

enum DType : int32_t { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2, DT_FP8 = 3 };

// What to launch: the op's element types and shape of work.
struct LaunchSpec {
  int32_t dtype;            // input (and plain cache) dtype
  int32_t q_dtype;          // Q output dtype
  bool cache_fp8;           // caches hold FP8 codes with row scales
  bool cache_mixed;         // two caches, one plain and one FP8 (BandArgs::fp8_caches)
  uint32_t head_dim;
  bool interleaved;
  bool radd;
  bool bshd;                // padded [batch][seq_len] grid
  bool pack;                // token-packed passes (one head of a block of tokens)
};

// Largest passes-per-wave the kernel for this op holds in registers.
// fp8: some cache of the launch holds FP8 codes.
inline uint32_t max_passes(bool radd, bool norm, bool pack, bool fp8) {
  if (radd) return kMaxPassesRadd;
  if (norm) return (pack || fp8) ? kMaxPassesNorm : kMaxPassesNormPlain;
  return pack ? kMaxPassesStorePack : kMaxPassesStore;
}

// Passes per wave a launch runs unless overridden (before it is shrunk to
// give small launches enough waves).
inline uint32_t default_passes(bool radd, bool norm, bool pack, bool fp8) {
  return (radd || norm) ? max_passes(radd, norm, pack, fp8) : (uint32_t)kDefaultPassesStore;
}

// Launch the band engine; returns 0 or a hipError_t value.
int launch_band(const BandArgs& a, const LaunchSpec& s, void* stream);
// The translation units behind it.
int launch_plain(const BandArgs& a, const LaunchSpec& s, void* stream);
int launch_fp8(const BandArgs& a, const LaunchSpec& s, void* stream);
int launch_qout(const BandArgs& a, const LaunchSpec& s, void* stream);
int launch_pack(const BandArgs& a, const LaunchSpec& s, void* stream);
int launch_mixed(const BandArgs& a, const LaunchSpec& s, void* stream);

// Rows handled per 64-lane pass for a dtype / head_dim.
inline uint32_t rows_per_pass(int32_t dtype, uint32_t head_dim) {
  const uint32_t elems_per_chunk = dtype == DT_F32 ? 4u : 8u;  // 16 bytes of 4- or 2-byte elements
  const uint32_t lanes_per_row = head_dim / elems_per_chunk / 2u;
  return 64u / lanes_per_row;
}

}  // namespace qrp
