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
constexpr uint64_t kGemvCounterBytes = 256;  // the arrival counter's own line(s)

struct GemvArgs {
  const void* x;          // [m][x_stride] elements
  const void* w;          // [n][w_stride] elements (W stored row-major, y = x W^T)
  const void* gamma;      // [n_normed]
  void* normed;           // [m][normed_stride]
  void* unnormed;         // [m][unnormed_stride]
  float* ybuf;            // workspace: [m][n_normed] binary32 values of y
  uint32_t* counter;      // workspace: arrival counter, zero between calls
  int64_t x_stride, w_stride, normed_stride, unnormed_stride;
  uint32_t m, n, kc;      // kc: 16-byte chunks per row of x and W
  uint32_t n_normed;
  float eps;
  uint32_t transpose_b;    // 1: W stored [n][w_stride]; 0: W stored [k][w_stride]
  // launch shape (set by launch_gemv_norm)
  uint32_t n_groups;       // column groups: ceil(n / columns per group)
  uint32_t n_norm_groups;  // groups holding a normed column (the leading ones)
  uint32_t n_norm_blocks;  // blocks holding a normed group: the arrivals
  uint32_t units_per_xcd;  // W stored [k][n]: column units each XCD takes, in turn
};

// Enqueue the kernel (its launch shape is chosen from the sizes and the
// device's compute-unit count); returns a hipError_t value (0: launched).
int launch_gemv_norm(GemvArgs& a, int32_t dtype, void* stream);

// The library's own scratch for callers that cannot allocate: per GPU, the
// counter's line and then at most kGemvScratchFloats binary32 y values
// (m * n_normed of them per call).
constexpr uint64_t kGemvScratchFloats = 131072;
constexpr uint64_t kGemvScratchBytes = kGemvCounterBytes + 4 * kGemvScratchFloats;

// Device address of the current device's scratch (set up on the first call
// for that device: its address looked up, its counter cleared on `stream`).
// Returns a hipError_t value (0: *out is set).
int gemv_scratch(void** out, void* stream);

}  // namespace qrp
