// gemv_norm.hip -- fused GEMV + partial RMSNorm for gfx950
// (MatmulFusedPartialRMSNorm page: Summary, execute, Args).
//
// A GEMV reads every element of W once, so the kernel is bound by HBM
// bandwidth, not by the matrix cores: it streams W with 16-byte
// non-temporal loads and does the products on the vector ALUs.
//
// Work mapping.  One wave64 owns a group of CPW consecutive output columns
// and sweeps the whole of k: lane l takes the 16-byte chunks l, l + 64,
// l + 128, ... of each W row (a wave reads 1 KB of a row per load
// instruction, fully coalesced) and the same chunks of every x row (from
// the L1 for one row; several rows are copied to LDS once per block when
// they fit 63 KB).  U chunks per lane are loaded before any is used, so a
// wave keeps U * CPW KB of W in flight.  Each lane sums its own terms in k
// order -- for fp32 one fused multiply-add per term, for bf16 and f16 one
// packed dot product per pair of terms (v_dot2, whose two products are
// exact in binary32) -- then an xor butterfly over the 64 lanes adds the
// partial sums; every lane ends with the same bits (each step adds the same
// two values, and binary32 addition commutes).  The order of additions is
// therefore fixed: the result does not depend on the launch shape, and a
// row gives the same bits alone or among others.
//
// Launch shape.  At most one block of 8 waves per compute unit.  Blocks
// [0, nbn) take the groups that hold normed columns, the others the
// passed-through groups; within each set the groups go round-robin over
// the blocks (see run()).
//
// The partial norm.  A row's norm needs all n_normed columns, which many
// blocks produce.  Their waves store binary32 y values in a workspace; then
// each normed block meets at a barrier, and one thread releases the block's
// values at agent scope and takes a ticket from an arrival counter (an
// atomic increment that wraps to zero, so the counter is zero again after
// every call).  Arrivals are serialised -- each release writes back its
// XCD's L2 (about 130 ns apart on one XCD, measured) and the increments of
// the one counter follow each other -- so they are taken per block, not
// per wave.  The block that draws the last ticket acquires, and its first
// four waves read the whole of y back and normalise every row:
//   ss = sum y_j^2 (per-thread fused multiply-adds in j order over every
//        256th column, the butterfly, then the four wave sums in order),
//   r = 1 / sqrt(ss / n_normed + eps),
//   out_j = (y_j * r) * gamma_j, rounded to the storage dtype.
// No wave waits for another, so nothing can hang on a missing arrival.
// The columns past n_normed are rounded and stored by the wave that made
// them.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "gemv_norm.hpp"
#include "qk_rope_paged.h"

namespace qrp {
namespace {

typedef unsigned int gv4u __attribute__((ext_vector_type(4)));
typedef _Float16 gh2 __attribute__((ext_vector_type(2)));

template <int DT>
constexpr int chunk_elems() {
  return DT == QRP_F32 ? 4 : 8;
}

// one 16-byte chunk -> binary32 values (every conversion is exact)
template <int DT>
__device__ __forceinline__ void widen(const gv4u v, float* f) {
  if constexpr (DT == QRP_F32) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  } else if constexpr (DT == QRP_BF16) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const gh2 h = __builtin_bit_cast(gh2, w[i]);
      f[2 * i] = (float)h.x;
      f[2 * i + 1] = (float)h.y;
    }
  }
}

// v rounded to the dtype (nearest even) and stored as element i
template <int DT>
__device__ __forceinline__ void store_elem(void* base, int64_t i, float v) {
  if constexpr (DT == QRP_F32) {
    reinterpret_cast<float*>(base)[i] = v;
  } else if constexpr (DT == QRP_BF16) {
    reinterpret_cast<__bf16*>(base)[i] = (__bf16)v;
  } else {
    reinterpret_cast<_Float16*>(base)[i] = (_Float16)v;
  }
}

typedef __bf16 gbf2 __attribute__((ext_vector_type(2)));

// acc + x.lo * w.lo + x.hi * w.hi for two packed 16-bit values per word
template <int DT>
__device__ __forceinline__ float dot2(uint32_t x, uint32_t w, float acc) {
  if constexpr (DT == QRP_BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(gbf2, x),
                                           __builtin_bit_cast(gbf2, w), acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(gh2, x), __builtin_bit_cast(gh2, w), acc,
                                  false);
}

// sum over the wave's 64 lanes; every lane gets the same bits
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// y values were stored by other compute units (other L2s): agent-scope loads
__device__ __forceinline__ float load_y(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// element i of a dtype array as raw bits, and those bits widened (exact)
template <int DT>
__device__ __forceinline__ uint32_t load_bits(const void* base, int64_t i) {
  if constexpr (DT == QRP_F32)
    return reinterpret_cast<const uint32_t*>(base)[i];
  else
    return reinterpret_cast<const uint16_t*>(base)[i];
}
template <int DT>
__device__ __forceinline__ float bits_value(uint32_t b) {
  if constexpr (DT == QRP_F32)
    return __uint_as_float(b);
  else if constexpr (DT == QRP_BF16)
    return __uint_as_float(b << 16);
  else
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// element i of a dtype array, widened (exact)
template <int DT>
__device__ __forceinline__ float load_elem_bits(const void* base, uint32_t i) {
  return bits_value<DT>(load_bits<DT>(base, (int64_t)i));
}

// y values of row r, column j (< n_normed): from the workspace, stored by
// other compute units ...
struct YFromWorkspace {
  const float* y;
  uint32_t nn;
  __device__ float operator()(uint32_t r, uint32_t j) const {
    return load_y(y + (uint64_t)r * nn + j);
  }
};
// ... or from this block's LDS
struct YFromLds {
  const float* y;
  uint32_t nn;
  __device__ float operator()(uint32_t r, uint32_t j) const { return y[r * nn + j]; }
};

// The norm is done by the first 256 threads (four waves, present in every
// launch) of the last block; each holds up to kNormHeld of a row's y values
// and gammas, so a row of up to 2048 normed columns is read in one round.
constexpr uint32_t kNormThreads = 256;
constexpr int kNormHeld = 8;

// RMSNorm of the n_normed leading columns of every row, by the last block
// (every thread of it calls this: the barriers need them all).  Thread t
// sums columns t, t + 256, ... in order (padding terms add exact zeros),
// each wave adds its 64 sums in the butterfly, and the four wave sums are
// added in wave order, so the order does not depend on the launch shape, on
// how many rounds a row takes or on how many rows are normalised together.
//
// The loads are what this tail waits on, so they are issued together and
// unconditionally: indexes past the end are clamped to the last column (a
// value read and then replaced by zero), the raw gamma bits are widened
// after every load has been issued, and with up to 2048 normed columns all
// the rows' y values and the gammas (shared by the rows) are read in one
// round before any is used.
template <int DT, int MB, class Y>
__device__ void norm_rows(const GemvArgs& a, const Y& y_at) {
  __shared__ float wave_part[MB][kNormThreads / 64];
  const uint32_t t = threadIdx.x;
  const bool worker = t < kNormThreads;  // wave-uniform
  const uint32_t nn = a.n_normed;
  const int64_t out_row = a.normed_stride;
  if (nn <= kNormThreads * (uint32_t)kNormHeld) {
    float v[MB][kNormHeld], g[kNormHeld];
    if (worker) {
      uint32_t gb[kNormHeld];
#pragma unroll
      for (int i = 0; i < kNormHeld; ++i) {
        const uint32_t jc = min(t + kNormThreads * (uint32_t)i, nn - 1);
        gb[i] = load_bits<DT>(a.gamma, jc);
#pragma unroll
        for (int r = 0; r < MB; ++r) {
          const uint32_t rc = min((uint32_t)r, a.m - 1);
          v[r][i] = y_at(rc, jc);
        }
      }
#pragma unroll
      for (int i = 0; i < kNormHeld; ++i) {
        const bool in = t + kNormThreads * (uint32_t)i < nn;
        g[i] = in ? bits_value<DT>(gb[i]) : 0.f;
#pragma unroll
        for (int r = 0; r < MB; ++r) v[r][i] = in ? v[r][i] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < MB; ++r) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < kNormHeld; ++i) ss = __builtin_fmaf(v[r][i], v[r][i], ss);
        ss = wave_sum(ss);
        if ((t & 63u) == 0) wave_part[r][t >> 6] = ss;
      }
    }
    __syncthreads();
    if (worker) {
#pragma unroll
      for (int r = 0; r < MB; ++r) {
        if ((uint32_t)r >= a.m) break;
        const float total =
            ((wave_part[r][0] + wave_part[r][1]) + wave_part[r][2]) + wave_part[r][3];
        const float rs = 1.0f / __builtin_sqrtf(total / (float)nn + a.eps);
#pragma unroll
        for (int i = 0; i < kNormHeld; ++i) {
          const uint32_t j = t + kNormThreads * (uint32_t)i;
          if (j < nn) store_elem<DT>(a.normed, (int64_t)r * out_row + j, (v[r][i] * rs) * g[i]);
        }
      }
    }
    return;
  }
  // longer rows: one row at a time, kNormHeld columns per thread per round
  for (uint32_t r = 0; r < a.m; ++r) {
    float ss = 0.f;
    if (worker) {
      for (uint32_t base = 0; base < nn; base += kNormThreads * (uint32_t)kNormHeld) {
        float v[kNormHeld];
#pragma unroll
        for (int i = 0; i < kNormHeld; ++i)
          v[i] = y_at(r, min(base + t + kNormThreads * (uint32_t)i, nn - 1));
#pragma unroll
        for (int i = 0; i < kNormHeld; ++i) {
          const float x = base + t + kNormThreads * (uint32_t)i < nn ? v[i] : 0.f;
          ss = __builtin_fmaf(x, x, ss);
        }
      }
      ss = wave_sum(ss);
      if ((t & 63u) == 0) wave_part[0][t >> 6] = ss;
    }
    __syncthreads();
    if (worker) {
      const float total =
          ((wave_part[0][0] + wave_part[0][1]) + wave_part[0][2]) + wave_part[0][3];
      const float rs = 1.0f / __builtin_sqrtf(total / (float)nn + a.eps);
      for (uint32_t base = 0; base < nn; base += kNormThreads * (uint32_t)kNormHeld) {
        float v[kNormHeld];
        uint32_t gb[kNormHeld];
#pragma unroll
        for (int i = 0; i < kNormHeld; ++i) {
          const uint32_t jc = min(base + t + kNormThreads * (uint32_t)i, nn - 1);
          v[i] = y_at(r, jc);
          gb[i] = load_bits<DT>(a.gamma, jc);
        }
#pragma unroll
        for (int i = 0; i < kNormHeld; ++i) {
          const uint32_t j = base + t + kNormThreads * (uint32_t)i;
          if (j < nn)
            store_elem<DT>(a.normed, (int64_t)r * out_row + j,
                           (v[i] * rs) * bits_value<DT>(gb[i]));
        }
      }
    }
    __syncthreads();  // wave_part is reused by the next row
  }
}

// Columns [g * CPW, g * CPW + CPW) of every row, by one wave: the wave's
// dot products, then lane m * CPW + j stores (row m, column g * CPW + j) --
// into the workspace for a normed column, rounded to the output otherwise.
// Columns and rows past the ends are clamped so every load stays in bounds,
// and their results are never stored.
template <int DT, int MB, int CPW, int U, bool XL>
__device__ __forceinline__ void column_group(const GemvArgs& a, uint32_t g, uint32_t lane,
                                             const gv4u* x_lds) {
  const uint32_t n0 = g * CPW;
  const gv4u* wrow[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const uint32_t col = min(n0 + (uint32_t)j, a.n - 1);
    wrow[j] = reinterpret_cast<const gv4u*>(
        reinterpret_cast<const char*>(a.w) +
        (int64_t)col * a.w_stride * (int64_t)(16 / chunk_elems<DT>()));
  }
  const gv4u* xrow[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const uint32_t row = min((uint32_t)m, a.m - 1);
    xrow[m] = reinterpret_cast<const gv4u*>(
        reinterpret_cast<const char*>(a.x) +
        (int64_t)row * a.x_stride * (int64_t)(16 / chunk_elems<DT>()));
  }

  constexpr int E = chunk_elems<DT>();
  float acc[MB][CPW];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < CPW; ++j) acc[m][j] = 0.f;

  const gv4u zero = {0u, 0u, 0u, 0u};
  const uint32_t kc = a.kc;
  for (uint32_t base = 0; base < kc; base += 64u * U) {
    gv4u wv[U][CPW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t c = base + (uint32_t)u * 64u + lane;
      const bool in = c < kc;
#pragma unroll
      for (int j = 0; j < CPW; ++j)
        wv[u][j] = in ? __builtin_nontemporal_load(wrow[j] + c) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t c = base + (uint32_t)u * 64u + lane;
      const bool in = c < kc;
      float wf[CPW][E];
      if constexpr (DT == QRP_F32) {
#pragma unroll
        for (int j = 0; j < CPW; ++j) widen<DT>(wv[u][j], wf[j]);
      }
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        gv4u xv = zero;
        if constexpr (XL) {
          if (in) xv = x_lds[m * kc + c];
        } else {
          if (in) xv = xrow[m][c];
        }
        if constexpr (DT == QRP_F32) {
          float xf[E];
          widen<DT>(xv, xf);
#pragma unroll
          for (int j = 0; j < CPW; ++j)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[m][j] = __builtin_fmaf(xf[e], wf[j][e], acc[m][j]);
        } else {
          // 16-bit types: one packed dot product per pair of elements, on
          // the loaded words (the two products are exact in binary32)
#pragma unroll
          for (int j = 0; j < CPW; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][j] = dot2<DT>(xv[i], wv[u][j][i], acc[m][j]);
        }
      }
    }
  }

  float mine = 0.f;
  uint32_t my_row = 0, my_col = 0;
  bool store = false;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const float t = wave_sum(acc[m][j]);
      if (lane == (uint32_t)(m * CPW + j)) {
        mine = t;
        my_row = (uint32_t)m;
        my_col = n0 + (uint32_t)j;
        store = true;
      }
    }
  if (store && my_row < a.m && my_col < a.n) {
    if (my_col < a.n_normed)
      __hip_atomic_store(a.ybuf + (uint64_t)my_row * a.n_normed + my_col, mine,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      store_elem<DT>(a.unnormed, (int64_t)my_row * a.unnormed_stride + (my_col - a.n_normed),
                     mine);
  }
}

// chunk c of x row m (rows past the last are clamped to it)
template <int DT>
__device__ __forceinline__ gv4u xrow_chunk(const GemvArgs& a, int m, uint32_t c) {
  const uint32_t row = min((uint32_t)m, a.m - 1);
  return reinterpret_cast<const gv4u*>(reinterpret_cast<const char*>(a.x) +
                                       (int64_t)row * a.x_stride *
                                           (int64_t)(16 / chunk_elems<DT>()))[c];
}

// Waves per block.
constexpr uint32_t kGemvMaxWaves = 8;
// Bytes of W each block of normed groups streams (the launch shape).
constexpr uint64_t kGemvNormBlockBytes = 200 * 1024;

template <int DT, int MB, int CPW, int U, bool XL>
__global__ void __launch_bounds__(64 * kGemvMaxWaves) gemv_norm_kernel(const GemvArgs a) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t w = threadIdx.x >> 6;
  const uint32_t nw = blockDim.x >> 6;
  const uint32_t nb = gridDim.x;
  const uint32_t b = blockIdx.x;

  // several x rows (XL): the block copies them to LDS once, row m at
  // x_lds + m * kc; every wave would otherwise re-read them all from global
  // memory, which overflows the L1
  extern __shared__ gv4u x_lds[];
  if constexpr (XL) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
      for (uint32_t c = threadIdx.x; c < a.kc; c += blockDim.x)
        x_lds[m * a.kc + c] = xrow_chunk<DT>(a, m, c);
    __syncthreads();
  }

  // Blocks [0, nbn) compute the normed groups, the others the passed-through
  // ones; within each set wave w of block b takes groups w * nbs + b, then
  // every (nw * nbs)-th after it (nbs blocks in the set), so consecutive
  // groups go to different compute units.
  const uint32_t nbn = a.n_norm_blocks;
  const uint32_t ng = a.n_norm_groups;
  if (b >= nbn) {
    const uint32_t nbu = nb - nbn;
    for (uint32_t g = ng + w * nbu + (b - nbn); g < a.n_groups; g += nw * nbu)
      column_group<DT, MB, CPW, U, XL>(a, g, lane, x_lds);
    return;
  }
  for (uint32_t g = w * nbn + b; g < ng; g += nw * nbn)
    column_group<DT, MB, CPW, U, XL>(a, g, lane, x_lds);

  // arrive once per block; the block that draws the last ticket normalises
  __shared__ uint32_t block_last;
  __syncthreads();  // every wave's y values are stored
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    block_last = __builtin_amdgcn_atomic_inc32(a.counter, nbn - 1, __ATOMIC_RELAXED, "agent") ==
                 nbn - 1;
  }
  // with no block of their own, the passed-through groups come after
  if (nb == nbn)
    for (uint32_t g = ng + w * nb + b; g < a.n_groups; g += nw * nb)
      column_group<DT, MB, CPW, U, XL>(a, g, lane, x_lds);
  __syncthreads();  // block_last is set
  if (!block_last) return;  // block-uniform
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  norm_rows<DT, MB>(a, YFromWorkspace{a.ybuf, a.n_normed});
}

// W stored [k][n] (transpose_b = 0): y_j = sum_k x_k W[k][j].  A row of W
// holds many columns, so a column's k values lie a row apart.  A compute
// unit issues only about one line request every 8 cycles (measured), so
// every request should bring a whole 128-byte line: the columns are cut
// into tiles of 128 bytes of a row (64 bf16 or f16 columns, 32 fp32), and 8
// lanes read one row's tile, 16 bytes each.  A tile is narrow, so k is cut
// too: block b takes tile b % tiles and slice b / tiles of split_rows rows
// of k, and the chip streams W with whole lines from every compute unit.
//
// In a block of 512 threads, thread t reads chunk t % 8 of the tile and
// belongs to row group t / 8 (64 groups); each round a group takes RG
// consecutive rows (the block RG * 64), loading RG chunks of W and, for each
// x row, the x values of those rows as whole 16-byte chunks.  Per column the
// sum runs: each thread's terms in k order (one fused multiply-add per
// term), the xor butterfly over its wave's 8 groups, the 8 wave sums in wave
// order, then the slices' sums in slice order.  The order is fixed by the
// sizes and the slice count, which depends on n, k, the dtype and the
// device's compute-unit count, not on the row count: a row gives the same
// bits alone or among others.
//
// With k cut, each block stores its sums in the workspace and releases
// them.  Normally it then takes a ticket from its tile's counter (an
// increment that wraps to zero); the tile's last block acquires and adds
// the slices' sums, and, as in the [n][k] kernel, each tile holding normed
// columns stores its y values, releases them and arrives once at the norm's
// counter; the last one normalises every row.  When the normed columns'
// slice sums are few, the blocks of normed tiles take their ticket from the
// norm's counter at once (single arrival), and the last of them adds every
// normed column's slices itself (in the same order) before normalising;
// only tiles with passed-through columns still meet at their own counter.
// Without k cut, a block's sums are y itself.
constexpr uint32_t kTileLanes = 8;  // lanes reading one row's tile (128 bytes)
constexpr uint32_t kTWaves = 8;     // waves per block
constexpr uint32_t kTGroups = kTWaves * 64 / kTileLanes;  // row groups per block

// 16-byte chunk v, element i, widened (exact)
template <int DT>
__device__ __forceinline__ float chunk_elem(const gv4u v, int i) {
  if constexpr (DT == QRP_F32) {
    return __uint_as_float(v[i]);
  } else if constexpr (DT == QRP_BF16) {
    return __uint_as_float((i & 1) ? (v[i >> 1] & 0xFFFF0000u) : (v[i >> 1] << 16));
  } else {
    const gh2 h = __builtin_bit_cast(gh2, (uint32_t)v[i >> 1]);
    return (float)((i & 1) ? h.y : h.x);
  }
}

// With the single arrival (few slice sums in all), the last block to arrive
// adds the slices of every normed column in slice order -- the same sums
// as a tile's last block makes -- into LDS, and normalises from there.  Each
// thread takes every 512th (row, column) pair; the loads of four pairs and
// four slices are issued together.
constexpr uint32_t kGemvSingleMaxY = 8192;         // m * n_normed held in LDS
constexpr uint32_t kGemvSingleMaxSlices = 16384;  // k_splits * m * n_normed read

template <int DT, int MB>
__device__ void norm_from_slices(const GemvArgs& a) {
  constexpr uint32_t CT = kTileLanes * chunk_elems<DT>();
  constexpr uint32_t NT = 64 * kTWaves;
  __shared__ float y_lds[kGemvSingleMaxY];
  const uint32_t t = threadIdx.x;
  const uint32_t nn = a.n_normed, total = a.m * nn, S = a.k_splits;
  const uint64_t slice_stride = (uint64_t)a.m * CT;
  for (uint32_t base = t; base < total; base += 4 * NT) {
    const float* src[4];
#pragma unroll
    for (uint32_t h = 0; h < 4; ++h) {
      const uint32_t idx = min(base + h * NT, total - 1);
      const uint32_t r = idx / nn, j = idx % nn;
      src[h] = a.partials + ((uint64_t)(j / CT) * S * a.m + r) * CT + j % CT;
    }
    float y[4];
    for (uint32_t s0 = 0; s0 < S; s0 += 4) {
      float v[4][4];
#pragma unroll
      for (uint32_t h = 0; h < 4; ++h)
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i) v[h][i] = load_y(src[h] + min(s0 + i, S - 1) * slice_stride);
#pragma unroll
      for (uint32_t h = 0; h < 4; ++h)
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i)
          if (s0 + i < S) y[h] = (s0 + i == 0) ? v[h][i] : y[h] + v[h][i];
    }
#pragma unroll
    for (uint32_t h = 0; h < 4; ++h)
      if (base + h * NT < total) y_lds[base + h * NT] = y[h];
  }
  __syncthreads();
  norm_rows<DT, MB>(a, YFromLds{y_lds, nn});
}

template <int DT, int MB, int RG>
__global__ void __launch_bounds__(64 * kTWaves) gemv_norm_t_kernel(const GemvArgs a) {
  constexpr int E = chunk_elems<DT>();
  constexpr uint32_t CT = kTileLanes * E;  // columns per tile
  constexpr int XC = RG / E;               // x chunks per row group and x row
  static_assert(RG % 8 == 0 && MB * CT <= 64 * kTWaves, "tile shape");
  const uint32_t t = threadIdx.x;
  const uint32_t w = t >> 6;
  const uint32_t p = t & (kTileLanes - 1u);
  const uint32_t grp = t / kTileLanes;
  const uint32_t tile = blockIdx.x % a.n_groups;
  const uint32_t split = blockIdx.x / a.n_groups;
  const uint32_t n0 = tile * CT;
  const int64_t es = 16 / E;  // element bytes
  const uint32_t k = a.kc * (uint32_t)E;
  const uint32_t kb = split * a.split_rows;
  const uint32_t ke = min(k, kb + a.split_rows);
  // a chunk past the row's stride (the last tile of a ragged n) is never
  // read; one inside it but past n is read and its columns never stored
  const bool col_in = n0 + p * (uint32_t)E < (uint64_t)a.w_stride;
  const char* wp = reinterpret_cast<const char*>(a.w) + (int64_t)(n0 + p * E) * es;
  const int64_t wrow = a.w_stride * es;
  const char* xp[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
    xp[m] = reinterpret_cast<const char*>(a.x) +
            (int64_t)min((uint32_t)m, a.m - 1) * a.x_stride * es;

  float acc[MB][E];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[m][e] = 0.f;

  const gv4u zero = {0u, 0u, 0u, 0u};
  for (uint32_t base = kb + grp * RG; base < ke; base += kTGroups * RG) {
    // rows base .. base + RG - 1; k and ke are multiples of E, so each x
    // chunk (E rows) is wholly inside or wholly past the slice
    gv4u wv[RG];
    gv4u xv[MB][XC];
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const uint32_t r = base + (uint32_t)i;
      wv[i] = (r < ke && col_in)
                  ? __builtin_nontemporal_load(reinterpret_cast<const gv4u*>(wp + (int64_t)r * wrow))
                  : zero;
    }
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int c = 0; c < XC; ++c) {
        const uint32_t r = base + (uint32_t)(c * E);
        xv[m][c] = r < ke ? *reinterpret_cast<const gv4u*>(xp[m] + (int64_t)r * es) : zero;
      }
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      float wf[E];
      widen<DT>(wv[i], wf);
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const float xm = chunk_elem<DT>(xv[m][i / E], i % E);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[m][e] = __builtin_fmaf(xm, wf[e], acc[m][e]);
      }
    }
  }

  // the butterfly over the wave's 8 groups (lanes p, p + 8, ..., p + 56),
  // then the 8 wave sums in order; thread t < MB * CT holds (row t / CT,
  // column n0 + t % CT)
  __shared__ float part[kTWaves][MB * CT];
  __shared__ uint32_t tile_flag, norm_flag;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float v = acc[m][e];
      v += __shfl_xor(v, 8, 64);
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if ((t & 63u) < kTileLanes) part[w][m * CT + p * E + e] = v;
    }
  __syncthreads();
  const bool holder = t < MB * CT;
  const uint32_t my_row = t / CT, tc = t % CT, my_col = n0 + tc;
  float y = 0.f;
  if (holder) {
    y = part[0][t];
#pragma unroll
    for (uint32_t v = 1; v < kTWaves; ++v) y += part[v][t];
  }

  const bool normed_tile = tile < a.n_norm_groups;
  bool norm_last = false;  // this block normalises
  if (a.k_splits > 1) {
    // This slice's sums go to the workspace.  Blocks of a tile with
    // passed-through columns (every tile, without the single arrival) take
    // a ticket from the tile's counter: the last adds the slices for them.
    // With the single arrival, blocks of normed tiles also take one from the
    // norm's counter: the last of all adds the normed columns' slices.
    const uint64_t slice_stride = (uint64_t)a.m * CT;
    float* tile_part = a.partials + (uint64_t)tile * a.k_splits * slice_stride;
    if (holder && my_row < a.m)
      __hip_atomic_store(tile_part + split * slice_stride + (uint64_t)my_row * CT + tc, y,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool tile_arrives =
        !a.single_arrival || max(n0, a.n_normed) < min(n0 + CT, a.n);  // passed-through columns
    const bool norm_arrives = a.single_arrival && normed_tile;
    __syncthreads();  // every thread's sums are stored
    if (t == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      tile_flag = tile_arrives && __builtin_amdgcn_atomic_inc32(a.tile_counter + tile,
                                                                a.k_splits - 1, __ATOMIC_RELAXED,
                                                                "agent") == a.k_splits - 1;
      const uint32_t last = a.n_norm_groups * a.k_splits - 1;
      norm_flag = norm_arrives && __builtin_amdgcn_atomic_inc32(a.counter, last, __ATOMIC_RELAXED,
                                                                "agent") == last;
    }
    __syncthreads();
    const bool tile_last = tile_flag;  // block-uniform
    norm_last = norm_flag;
    if (!tile_last && !norm_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (tile_last && holder && my_row < a.m) {
      const float* src = tile_part + (uint64_t)my_row * CT + tc;
      // the slices in order, their loads issued eight at a time
      y = 0.f;
      for (uint32_t s0 = 0; s0 < a.k_splits; s0 += 8) {
        float v[8];
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i)
          v[i] = load_y(src + min(s0 + i, a.k_splits - 1) * slice_stride);
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i)
          if (s0 + i < a.k_splits) y = (s0 + i == 0) ? v[i] : y + v[i];
      }
    }
    if (!tile_last) y = 0.f;  // nothing of this tile is stored below
  }

  // the tile's outputs: y values of normed columns to the workspace (not
  // with the single arrival: the normalising block reads the slices),
  // passed-through columns rounded to the output
  const bool store_y = a.k_splits == 1 || tile_flag;
  if (store_y && holder && my_row < a.m && my_col < a.n) {
    if (my_col >= a.n_normed)
      store_elem<DT>(a.unnormed, (int64_t)my_row * a.unnormed_stride + (my_col - a.n_normed), y);
    else if (!a.single_arrival)
      __hip_atomic_store(a.ybuf + (uint64_t)my_row * a.n_normed + my_col, y, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  if (a.single_arrival) {
    if (norm_last) norm_from_slices<DT, MB>(a);
    return;
  }
  if (!normed_tile) return;  // block-uniform: no normed column here

  // arrive once per tile; the tile that draws the last ticket normalises
  __syncthreads();  // every thread's y values are stored (and the flags read)
  if (t == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    norm_flag = __builtin_amdgcn_atomic_inc32(a.counter, a.n_norm_groups - 1, __ATOMIC_RELAXED,
                                              "agent") == a.n_norm_groups - 1;
  }
  __syncthreads();
  if (!norm_flag) return;  // block-uniform
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  norm_rows<DT, MB>(a, YFromWorkspace{a.ybuf, a.n_normed});
}

// Largest LDS copy of the x rows (more rows go through global memory); 1 KB
// of a 64 KB block allocation is left for the kernel's own LDS.
constexpr uint64_t kGemvMaxLdsBytes = 63 * 1024;

// compute units of the current device (looked up once per device)
std::mutex g_cu_mu;
std::vector<uint32_t> g_cu_count;

int device_cus(uint32_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  std::lock_guard<std::mutex> lock(g_cu_mu);
  if ((size_t)dev >= g_cu_count.size()) g_cu_count.resize((size_t)dev + 1, 0u);
  if (!g_cu_count[dev]) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    g_cu_count[dev] = cus > 0 ? (uint32_t)cus : 1u;
  }
  *out = g_cu_count[dev];
  return 0;
}

// Bytes of W each block of a [k][n] launch streams (the slice count).
constexpr uint64_t kGemvTSliceBytes = 256 * 1024;

// The [k][n] launch: tiles x slices blocks.  With fewer tiles than compute
// units, k is cut into slices of about kGemvTSliceBytes of W each, with at
// most one block per compute unit and at least one round of a block's row
// groups per slice; the slice length is a multiple of 8 rows.  Every block
// arrives once (a release and an increment, about 1.2 us measured), so
// fewer, longer slices can finish sooner: at one row of 7168 into 2112 (33
// tiles), 4 slices of 1792 rows took 13.2 us, against 13.6 with 5, 14.6
// with 7 and 14.5 with 3.  When the normed columns' slice sums are few
// (kGemvSingleMaxY, kGemvSingleMaxSlices) the blocks of normed tiles arrive
// at the norm's counter directly; otherwise each tile's last block adds its
// slices first and arrives in its turn, one more release and increment in
// the chain (17.6 us instead of 13.2 at the shape above).
template <int DT, int MB, int RG>
int run_t(GemvArgs& a, hipStream_t s) {
  uint32_t cus = 0;
  const int e = device_cus(&cus);
  if (e != 0) return e;
  constexpr uint64_t E = chunk_elems<DT>();
  constexpr uint64_t CT = kTileLanes * E;
  const uint64_t tiles = ((uint64_t)a.n + CT - 1) / CT;
  const uint64_t k = (uint64_t)a.kc * E;
  const uint64_t limit = std::min<uint64_t>(cus, kGemvMaxSplitBlocks);
  uint64_t splits = 1;
  if (tiles < limit && k) {
    const uint64_t tile_row = kTileLanes * 16;  // bytes of a tile in one row of W
    const uint64_t by_bytes = (k * tile_row + kGemvTSliceBytes - 1) / kGemvTSliceBytes;
    const uint64_t by_rounds = (k + kTGroups * RG - 1) / (kTGroups * RG);
    splits = std::max<uint64_t>(1, std::min(limit / tiles, std::min(by_bytes, by_rounds)));
  }
  uint64_t rows = (k + splits - 1) / splits;
  rows = (rows + 7) / 8 * 8;
  splits = rows ? (k + rows - 1) / rows : 1;
  a.n_groups = (uint32_t)tiles;
  a.n_norm_groups = (uint32_t)(((uint64_t)a.n_normed + CT - 1) / CT);
  a.n_norm_blocks = a.n_norm_groups;
  a.k_splits = (uint32_t)splits;
  a.split_rows = (uint32_t)rows;
  const uint64_t ys = (uint64_t)a.m * a.n_normed;
  a.single_arrival = splits > 1 && ys && ys <= kGemvSingleMaxY &&
                     splits * ys <= kGemvSingleMaxSlices;
  hipLaunchKernelGGL((gemv_norm_t_kernel<DT, MB, RG>), dim3((uint32_t)(tiles * splits)),
                     dim3(64 * kTWaves), 0, s, a);
  return (int)hipGetLastError();
}

// rows per launch -> rows held (8 rows of k per row group and round)
template <int DT>
int run_t_rows(GemvArgs& a, hipStream_t s) {
  if (a.m <= 1) return run_t<DT, 1, 8>(a, s);
  if (a.m <= 2) return run_t<DT, 2, 8>(a, s);
  if (a.m <= 4) return run_t<DT, 4, 8>(a, s);
  return run_t<DT, 8, 8>(a, s);
}

template <int DT, int MB, int CPW, int U>
int launch(const GemvArgs& a, uint32_t blocks, uint32_t waves, hipStream_t s) {
  const uint64_t lds = (uint64_t)MB * a.kc * 16;
  if (MB > 1 && lds <= kGemvMaxLdsBytes)
    hipLaunchKernelGGL((gemv_norm_kernel<DT, MB, CPW, U, (MB > 1)>), dim3(blocks),
                       dim3(64 * waves), (uint32_t)lds, s, a);
  else
    hipLaunchKernelGGL((gemv_norm_kernel<DT, MB, CPW, U, false>), dim3(blocks), dim3(64 * waves),
                       0, s, a);
  return (int)hipGetLastError();
}

// The launch shape.  At most one block per compute unit: every compute
// unit draws about the same share of HBM bandwidth, so one given two blocks
// finishes last, at twice the time.  The normed groups get blocks of their
// own, each streaming about kGemvNormBlockBytes of W (and at most two
// rounds of its waves): every such block arrives once, and the arrivals
// are serialised (a release writes back the XCD's L2, about 130 ns apart on
// one XCD, and the increments of the one counter follow each other), so
// more normed blocks stream the normed columns faster but arrive more
// slowly; at one row of 7168 into 1536 normed columns the time is flat
// between 96 and 128 such blocks.  The passed-through groups take few of
// the remaining compute units (one round of their waves where they fit),
// which leaves the normed blocks a larger share of the bandwidth.
template <int DT, int MB, int CPW, int U>
int run(GemvArgs& a, hipStream_t s) {
  uint32_t cus = 0;
  const int e = device_cus(&cus);
  if (e != 0) return e;
  const uint64_t groups = ((uint64_t)a.n + CPW - 1) / CPW;
  const uint64_t norm_groups = ((uint64_t)a.n_normed + CPW - 1) / CPW;
  a.n_groups = (uint32_t)groups;
  a.n_norm_groups = (uint32_t)norm_groups;
  const uint64_t nw = kGemvMaxWaves;
  uint64_t nbn = 0, nbu;
  if (norm_groups) {
    const uint64_t bytes = norm_groups * CPW * (uint64_t)a.kc * 16;
    nbn = std::max((bytes + kGemvNormBlockBytes - 1) / kGemvNormBlockBytes,
                   (norm_groups + 2 * nw - 1) / (2 * nw));
    nbn = std::max<uint64_t>(1, std::min<uint64_t>(nbn, std::min<uint64_t>(norm_groups,
                                                                            cus * 3 / 4)));
    nbu = std::min<uint64_t>(cus - std::min<uint64_t>(cus, nbn),
                             (groups - norm_groups + nw - 1) / nw);
  } else {
    // nothing to arrive for: every compute unit streams (about 5 % faster
    // than one round of 8 waves per block at one row of 7168 into 2112)
    nbu = std::max<uint64_t>(1, std::min<uint64_t>(cus, groups));
  }
  a.n_norm_blocks = (uint32_t)nbn;
  return launch<DT, MB, CPW, U>(a, (uint32_t)(nbn + nbu), (uint32_t)nw, s);
}

// rows per launch -> (rows held, columns per group, chunks in flight per lane)
template <int DT>
int run_rows(GemvArgs& a, hipStream_t s) {
  if (a.m <= 1) return run<DT, 1, 2, 16>(a, s);
  if (a.m <= 2) return run<DT, 2, 2, 8>(a, s);
  if (a.m <= 4) return run<DT, 4, 2, 4>(a, s);
  return run<DT, 8, 2, 4>(a, s);
}

// Clears the arrival counter's line of a scratch buffer.
__global__ void __launch_bounds__(64) clear_counter(uint32_t* c) {
  for (uint32_t i = threadIdx.x; i < kGemvCounterBytes / 4; i += 64) c[i] = 0u;
}

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device; null until that device is set up

}  // namespace

// Scratch of the entry point that allocates nothing: the arrival counter's
// line, then the y values.  Each GPU the library runs on holds its own copy
// until the process ends.  Host code never uses this name as an address: it
// stands for the host-side shadow of the variable; gemv_scratch() looks up
// each device's copy.
static __device__ __align__(256) unsigned char scratch[kGemvScratchBytes];

int gemv_scratch(void** out, void* stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    // the counter must be zero before the first call (every call leaves it
    // at zero); a kernel, not a memset, so that a captured first call
    // records it as a kernel node
    hipLaunchKernelGGL(clear_counter, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<uint32_t*>(p));
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

int launch_gemv_norm(GemvArgs& a, int32_t dtype, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!a.transpose_b) {
    if (dtype == QRP_F32) return run_t_rows<QRP_F32>(a, s);
    if (dtype == QRP_F16) return run_t_rows<QRP_F16>(a, s);
    return run_t_rows<QRP_BF16>(a, s);
  }
  if (dtype == QRP_F32) return run_rows<QRP_F32>(a, s);
  if (dtype == QRP_F16) return run_rows<QRP_F16>(a, s);
  return run_rows<QRP_BF16>(a, s);
}

}  // namespace qrp
