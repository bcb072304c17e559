// gemv_norm.hpp -- launch descriptor of the fused GEMV + partial RMSNorm
// kernel (MatmulFusedPartialRMSNorm page: Summary, execute, Args).
//
// y = x W^T for up to kGemvMaxRows input rows; the first n_normed columns of
// each row are RMS-normalised as one vector and scaled by gamma, the other
// columns are stored as they are.  One wave computes a group of columns
// over the whole of k; the columns that need the norm go to a binary32
// workspace, and the last block of those to arrive normalises every row.
#pragma once

#include <stdint.h>

namespace qrp {

constexpr uint32_t kGemvMaxRows = 8;

// Workspace layout: the arrival counters (the norm's in the first 256
// bytes; with W stored [k][n], one per column tile of a launch that splits
// k, in the next 1024), then the binary32 y values [m][n_normed], then (W
// stored [k][n] only) the binary32 partial sums of the split launch.
constexpr uint64_t kGemvCounterBytes = 1280;
constexpr uint64_t kGemvTileCounterOffset = 256;
constexpr uint32_t kGemvMaxSplitBlocks = 256;  // blocks of a launch that splits k
constexpr uint32_t kGemvMaxTileCols = 64;      // columns of a [k][n] tile (128 bytes)
constexpr uint64_t kGemvPartialBytesPerRow = 4ull * kGemvMaxSplitBlocks * kGemvMaxTileCols;

// Offset of the partial sums: after the y values, on a 256-byte boundary.
constexpr uint64_t gemv_partials_offset(uint64_t m, uint64_t n_normed) {
  return kGemvCounterBytes + (4 * m * n_normed + 255) / 256 * 256;
}

// Bytes of workspace a call needs (0: none).
constexpr uint64_t gemv_workspace_bytes(uint64_t m, uint64_t n_normed, bool transpose_b) {
  return transpose_b ? (n_normed ? kGemvCounterBytes + 4 * m * n_normed : 0)
                     : gemv_partials_offset(m, n_normed) + kGemvPartialBytesPerRow * m;
}

struct GemvArgs {
  const void* x;          // [m][x_stride] elements
  const void* w;          // [n][w_stride] elements (W stored row-major, y = x W^T)
  const void* gamma;      // [n_normed]
  void* normed;           // [m][normed_stride]
  void* unnormed;         // [m][unnormed_stride]
  float* ybuf;            // workspace: [m][n_normed] binary32 values of y
  uint32_t* counter;      // workspace: arrival counter, zero between calls
  uint32_t* tile_counter; // workspace ([k][n]): per-tile arrival counters, zero between calls
  float* partials;        // workspace ([k][n]): [tile][split][m][tile columns] partial sums
  int64_t x_stride, w_stride, normed_stride, unnormed_stride;
  uint32_t m, n, kc;      // kc: 16-byte chunks per row of x and W
  uint32_t n_normed;
  float eps;
  uint32_t transpose_b;    // 1: W stored [n][w_stride]; 0: W stored [k][w_stride]
  // launch shape (set by launch_gemv_norm)
  uint32_t n_groups;       // column groups: ceil(n / columns per group)
  uint32_t n_norm_groups;  // groups holding a normed column (the leading ones)
  uint32_t n_norm_blocks;  // blocks holding a normed group: the arrivals
  uint32_t k_splits;       // W stored [k][n]: blocks sharing a column tile, each a slice of k
  uint32_t split_rows;     // W stored [k][n]: rows of k per slice
  uint32_t single_arrival; // W stored [k][n]: blocks of normed tiles arrive at the norm's counter
};

// Enqueue the kernel (its launch shape is chosen from the sizes and the
// device's compute-unit count); returns a hipError_t value (0: launched).
int launch_gemv_norm(GemvArgs& a, int32_t dtype, void* stream);

// The library's own scratch for callers that cannot allocate: per GPU, the
// workspace of the largest call it serves, m * n_normed <= kGemvScratchFloats
// y values and (W stored [k][n]) the partial sums of 8 rows.
constexpr uint64_t kGemvScratchFloats = 131072;
constexpr uint64_t kGemvScratchBytes =
    kGemvCounterBytes + 4 * kGemvScratchFloats + kGemvPartialBytesPerRow * kGemvMaxRows;

// Device address of the current device's scratch (set up on the first call
// for that device: its address looked up, its counter cleared on `stream`).
// Returns a hipError_t value (0: *out is set).
int gemv_scratch(void** out, void* stream);

}  // namespace qrp
