// gemv_norm.hpp -- launch descriptor of the fused GEMV + partial RMSNorm
// kernel (MatmulFusedPartialRMSNorm page: Summary, execute, Args).
//
// y = x W^T for up to kGemvMaxRows input rows; the first n_normed columns of
// each row are RMS-normalised as one vector and scaled by gamma, the other
// columns are stored as they are.  One wave computes cols_per_wave columns
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
  uint32_t n_waves;        // ceil(n / cols_per_wave)
  uint32_t n_norm_blocks;  // blocks holding a normed column: the arrivals
  float eps;
};

// Columns one wave computes for m input rows, and waves per block.  A block
// arrives once, so larger blocks mean fewer releases and fewer increments
// of the one counter (each is serialised), but fewer blocks leave compute
// units idle.  Measured at one row of 7168 into 2112 columns (1536 normed):
// 2 columns x 8 waves 12.8 us; 1 x 16: 14.4; 2 x 16: 18.7; 2 x 4: 14.3;
// 4 x 4: 14.6; 3 x 8: 15.0; at two rows 2 x 8: 15.0, 1 x 8: 17.4.  Every
// build has at least the four waves the norm uses.
inline uint32_t gemv_cols_per_wave(uint32_t) { return 2u; }
inline uint32_t gemv_waves_per_block(uint32_t m) { return m <= 2 ? 8u : 4u; }

// Enqueue the kernel; returns a hipError_t value (0: launched).
int launch_gemv_norm(const GemvArgs& a, int32_t dtype, void* stream);

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
