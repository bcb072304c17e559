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
template <int DT, int MB>
__device__ void norm_rows(const GemvArgs& a) {
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
          v[r][i] = load_y(a.ybuf + (uint64_t)rc * nn + jc);
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
    const float* yr = a.ybuf + (uint64_t)r * nn;
    float ss = 0.f;
    if (worker) {
      for (uint32_t base = 0; base < nn; base += kNormThreads * (uint32_t)kNormHeld) {
        float v[kNormHeld];
#pragma unroll
        for (int i = 0; i < kNormHeld; ++i)
          v[i] = load_y(yr + min(base + t + kNormThreads * (uint32_t)i, nn - 1));
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
          v[i] = load_y(yr + jc);
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
  norm_rows<DT, MB>(a);
}

// W stored [k][n] (transpose_b = 0): y_j = sum_k x_k W[k][j].  A row of W
// now holds many columns, so a wave cannot stream one column's k values
// contiguously.  Instead a block of 256 threads owns a unit of TP 16-byte
// column chunks (TP * E columns) over the whole of k: thread t takes the
// rows t, t + 256, t + 512, ... and loads, for each, the unit's 16 bytes
// of that row and the row's x value of every input row (a wave's load
// instruction covers 64 consecutive rows).  Each W access is 16 bytes of a
// different line; the line's other chunks belong to neighbouring units, which the
// grid places on the same XCD at the same time (unit u on XCD u / per), so
// the L2 serves them and HBM sees each line once -- the loads are ordinary
// ones, so that the lines stay in the L2.
//
// Summation order per column: thread t adds its rows' terms in k order
// (one fused multiply-add per term, so each term rounds once), then the
// butterfly over its wave's 64 lanes, then the four wave sums in wave
// order -- fixed, and the same for every row count.
// The partial norm is the one of the [n][k] kernel: one arrival per block
// holding a normed column, and the last block normalises.
template <int DT, int MB, int TP, int UT>
__global__ void __launch_bounds__(256) gemv_norm_t_kernel(const GemvArgs a) {
  constexpr int E = chunk_elems<DT>();
  constexpr int NC = TP * E;  // columns per unit
  const uint32_t t = threadIdx.x;
  const uint32_t lane = t & 63u;
  const uint32_t w = t >> 6;
  // blocks are dealt to the XCDs in turn (block b on XCD b % 8): XCD x takes
  // units [x * per, (x + 1) * per), so neighbouring units share its L2
  const uint32_t unit = (blockIdx.x % 8u) * a.units_per_xcd + blockIdx.x / 8u;
  if (unit >= a.n_groups) return;  // block-uniform, before any barrier
  const uint32_t n0 = unit * NC;
  const int64_t es = 16 / E;  // element bytes
  const char* wcol = reinterpret_cast<const char*>(a.w) + (int64_t)n0 * es;
  const int64_t wrow = a.w_stride * es;
  const char* xb = reinterpret_cast<const char*>(a.x);
  const int64_t xrow = a.x_stride * es;

  float acc[MB][NC];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[m][c] = 0.f;

  // thread t takes rows t, t + 256, t + 512, ...: a wave's load instruction
  // reads 64 consecutive rows, so its addresses stay close together
  const gv4u zero = {0u, 0u, 0u, 0u};
  const uint32_t k = a.kc * (uint32_t)E;
  constexpr int RT = UT * E;  // rows per thread per round
  for (uint32_t base = 0; base < k; base += 256u * RT) {
    gv4u wv[RT][TP];
    float xs[RT][MB];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const uint32_t row = base + (uint32_t)i * 256u + t;
      const bool in = row < k;
      const uint32_t rc = in ? row : 0u;
#pragma unroll
      for (int p = 0; p < TP; ++p) {
        // a chunk past the row's stride (the last unit of a ragged n) is
        // never read: its columns are never stored
        const bool inp = in && n0 + (uint32_t)(p * E) < (uint64_t)a.w_stride;
        wv[i][p] = inp ? *reinterpret_cast<const gv4u*>(wcol + (int64_t)rc * wrow + p * 16) : zero;
      }
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const uint32_t xr = min((uint32_t)m, a.m - 1);
        xs[i][m] = in ? load_elem_bits<DT>(xb + (int64_t)xr * xrow, rc) : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      float wf[TP][E];
#pragma unroll
      for (int p = 0; p < TP; ++p) widen<DT>(wv[i][p], wf[p]);
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int p = 0; p < TP; ++p)
#pragma unroll
          for (int e = 0; e < E; ++e)
            acc[m][p * E + e] = __builtin_fmaf(xs[i][m], wf[p][e], acc[m][p * E + e]);
    }
  }

  // each column's 256 thread sums: the butterfly in each wave, then the four
  // wave sums in order; thread m * NC + c stores (row m, column n0 + c)
  __shared__ float part[4][MB * NC];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float v = wave_sum(acc[m][c]);
      if (lane == 0) part[w][m * NC + c] = v;
    }
  __syncthreads();
  if (t < (uint32_t)(MB * NC)) {
    const uint32_t my_row = t / NC, my_col = n0 + t % NC;
    const float y = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
    if (my_row < a.m && my_col < a.n) {
      if (my_col < a.n_normed)
        __hip_atomic_store(a.ybuf + (uint64_t)my_row * a.n_normed + my_col, y, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      else
        store_elem<DT>(a.unnormed,
                       (int64_t)my_row * a.unnormed_stride + (my_col - a.n_normed), y);
    }
  }
  if (unit >= a.n_norm_blocks) return;  // block-uniform: no normed column here

  // arrive once per block; the block that draws the last ticket normalises
  __shared__ uint32_t block_last;
  __syncthreads();  // every thread's y values are stored
  if (t == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    block_last = __builtin_amdgcn_atomic_inc32(a.counter, a.n_norm_blocks - 1, __ATOMIC_RELAXED,
                                               "agent") == a.n_norm_blocks - 1;
  }
  __syncthreads();
  if (!block_last) return;  // block-uniform
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  norm_rows<DT, MB>(a);
}

// The [k][n] launch: one block per unit of TP column chunks, the units of
// each XCD contiguous.  One chunk per unit (one block per 8 bf16 columns)
// measured fastest at one row of 7168 into 2112: 26.9 us, against 29.2 with
// two chunks (half the blocks) and 40-131 us with a unit's chunks spread
// over 2-8 neighbouring lanes (a quarter to an eighth of the blocks).
template <int DT, int MB, int TP, int UT>
int run_t(GemvArgs& a, hipStream_t s) {
  constexpr uint64_t NC = (uint64_t)TP * chunk_elems<DT>();
  const uint64_t units = ((uint64_t)a.n + NC - 1) / NC;
  const uint64_t per = (units + 7) / 8;
  a.n_groups = (uint32_t)units;
  a.n_norm_groups = (uint32_t)(((uint64_t)a.n_normed + NC - 1) / NC);
  a.n_norm_blocks = a.n_norm_groups;  // units [0, n_norm_groups) arrive
  a.units_per_xcd = (uint32_t)per;
  hipLaunchKernelGGL((gemv_norm_t_kernel<DT, MB, TP, UT>), dim3((uint32_t)(8 * per)), dim3(256), 0,
                     s, a);
  return (int)hipGetLastError();
}

template <int DT>
int run_t_rows(GemvArgs& a, hipStream_t s) {
  if (a.m <= 1) return run_t<DT, 1, 1, 2>(a, s);
  if (a.m <= 2) return run_t<DT, 2, 1, 2>(a, s);
  if (a.m <= 4) return run_t<DT, 4, 1, 1>(a, s);
  return run_t<DT, 8, 1, 1>(a, s);
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
  if (threadIdx.x < kGemvCounterBytes / 4) c[threadIdx.x] = 0u;
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
