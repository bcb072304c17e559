// gemv_norm.hip -- fused GEMV + partial RMSNorm for gfx950
// (MatmulFusedPartialRMSNorm page: Summary, execute, Args).
//
// A GEMV reads every element of W once, so the kernel is bound by HBM
// bandwidth, not by the matrix cores: it streams W with 16-byte
// non-temporal loads and does the products on the vector ALUs.
//
// Work mapping.  One wave64 owns `CPW` consecutive output columns and sweeps
// the whole of k: lane l takes the 16-byte chunks l, l + 64, l + 128, ... of
// each W row (a wave reads 1 KB of a row per load instruction, fully
// coalesced) and the same chunks of every x row (from the L1 for one row;
// several rows are copied to LDS once per block when they fit 63 KB).  U chunks per lane are loaded before any is used, so a wave keeps
// U * CPW KB of W in flight.  Each lane sums its own terms in k order with
// one fused multiply-add per term, then an xor butterfly over the 64 lanes
// adds the partial sums; every lane ends with the same bits (each step adds
// the same two values, and binary32 addition commutes), so the order of
// additions is fixed and the result does not depend on the launch.
//
// The partial norm.  A row's norm needs all n_normed columns, which many
// waves produce.  Those waves store their binary32 y values in a workspace;
// then each block that holds a normed column meets at a barrier, and one
// thread releases the block's values at agent scope and takes a ticket from
// an arrival counter (an atomic increment that wraps to zero, so the counter
// is zero again after every call).  Releases and increments of one counter
// are serialised by the memory system (about 10 ns each, measured), so they
// are taken per block of waves, not per wave.  The block that draws
// the last ticket acquires, and its first four waves read the whole of y
// back and normalise every row:
//   ss = sum y_j^2 (per-thread fused multiply-adds in j order over every
//        256th column, the butterfly, then the four wave sums in order),
//   r = 1 / sqrt(ss / n_normed + eps),
//   out_j = (y_j * r) * gamma_j, rounded to the storage dtype.
// No wave waits for another, so nothing can hang on a missing arrival.
// The columns past n_normed are rounded and stored by the wave that made
// them.  Waves of the normed columns come first in the grid, so their
// arrival overlaps the streaming of the rest.
#include <hip/hip_runtime.h>

#include <stdint.h>

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

// element i of a dtype array, widened
template <int DT>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
  if constexpr (DT == QRP_F32) {
    return reinterpret_cast<const float*>(base)[i];
  } else if constexpr (DT == QRP_BF16) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
  } else {
    return (float)reinterpret_cast<const _Float16*>(base)[i];
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

// The norm is done by the first 256 threads (four waves, present in every
// build) of the last block; each holds up to kNormHeld of a row's y values
// and gammas, so a row of up to 2048 normed columns is read in one round.
constexpr uint32_t kNormThreads = 256;
constexpr int kNormHeld = 8;

// RMSNorm of the n_normed leading columns of every row, by the last block
// (every thread of it calls this: the barriers need them all).  Thread t
// sums columns t, t + 256, ... in order (padding terms add exact zeros),
// each wave adds its 64 sums in the butterfly, and the four wave sums are
// added in wave order, so the order does not depend on the block size or on
// how many rounds a row takes.
template <int DT>
__device__ void norm_rows(const GemvArgs& a) {
  __shared__ float wave_part[kNormThreads / 64];
  const uint32_t t = threadIdx.x;
  const bool worker = t < kNormThreads;
  const uint32_t nn = a.n_normed;
  const bool one_round = nn <= kNormThreads * (uint32_t)kNormHeld;
  for (uint32_t m = 0; m < a.m; ++m) {
    const float* yr = a.ybuf + (uint64_t)m * nn;
    void* out = reinterpret_cast<char*>(a.normed) +
                (int64_t)m * a.normed_stride * (int64_t)(16 / chunk_elems<DT>());
    float v[kNormHeld], g[kNormHeld];
    float ss = 0.f;
    for (uint32_t base = 0; base < nn; base += kNormThreads * (uint32_t)kNormHeld) {
#pragma unroll
      for (int i = 0; i < kNormHeld; ++i) {
        const uint32_t j = base + t + kNormThreads * (uint32_t)i;
        const bool in = worker && j < nn;
        v[i] = in ? load_y(yr + j) : 0.f;
        g[i] = in ? load_elem<DT>(a.gamma, j) : 0.f;
      }
#pragma unroll
      for (int i = 0; i < kNormHeld; ++i) ss = __builtin_fmaf(v[i], v[i], ss);
    }
    ss = wave_sum(ss);
    if (worker && (t & 63u) == 0) wave_part[t >> 6] = ss;
    __syncthreads();
    const float total = ((wave_part[0] + wave_part[1]) + wave_part[2]) + wave_part[3];
    const float r = 1.0f / __builtin_sqrtf(total / (float)nn + a.eps);
    if (one_round) {
#pragma unroll
      for (int i = 0; i < kNormHeld; ++i) {
        const uint32_t j = t + kNormThreads * (uint32_t)i;
        if (worker && j < nn) store_elem<DT>(out, j, (v[i] * r) * g[i]);
      }
    } else if (worker) {
      for (uint32_t j = t; j < nn; j += kNormThreads)
        store_elem<DT>(out, j, (load_y(yr + j) * r) * load_elem<DT>(a.gamma, j));
    }
    __syncthreads();  // wave_part is reused by the next row
  }
}

template <int DT, int MB, int CPW, int U, int WPB, bool XL>
__global__ void __launch_bounds__(64 * WPB) gemv_norm_kernel(const GemvArgs a) {
  const uint32_t lane = threadIdx.x & 63u;
  // the grid's last block may hold waves past the end: they skip the work
  // but still meet the block at its barrier
  const uint32_t wave_raw = blockIdx.x * WPB + (threadIdx.x >> 6);
  const bool live = wave_raw < a.n_waves;
  const uint32_t wave = live ? wave_raw : a.n_waves - 1;
  const uint32_t n0 = wave * CPW;

  // operand rows; columns and rows past the ends are clamped so every load
  // stays in bounds, and their results are never stored
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

  // several x rows (XL): the block copies them to LDS once, row m at
  // x_lds + m * kc; every wave would otherwise re-read them all from global
  // memory, which overflows the L1
  extern __shared__ gv4u x_lds[];
  if constexpr (XL) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
      for (uint32_t c = threadIdx.x; c < a.kc; c += 64u * WPB) x_lds[m * a.kc + c] = xrow[m][c];
    __syncthreads();
  }

  const gv4u zero = {0u, 0u, 0u, 0u};
  const uint32_t kc = live ? a.kc : 0u;
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
          if (in) xv = x_lds[m * a.kc + c];
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

  // totals, then lane m * CPW + j stores (row m, column n0 + j)
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
  store = store && live && my_row < a.m && my_col < a.n;
  if (store) {
    if (my_col < a.n_normed)
      __hip_atomic_store(a.ybuf + (uint64_t)my_row * a.n_normed + my_col, mine,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      store_elem<DT>(a.unnormed, (int64_t)my_row * a.unnormed_stride + (my_col - a.n_normed),
                     mine);
  }
  // block-uniform: blocks past the normed columns are done
  if (blockIdx.x * (uint32_t)(WPB * CPW) >= a.n_normed) return;

  // arrive once per block; the block holding the last ticket normalises
  __shared__ uint32_t block_ticket;
  __syncthreads();  // every wave's y values are stored
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    block_ticket = __builtin_amdgcn_atomic_inc32(a.counter, a.n_norm_blocks - 1,
                                                 __ATOMIC_RELAXED, "agent");
  }
  __syncthreads();
  if (block_ticket != a.n_norm_blocks - 1) return;  // block-uniform
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  norm_rows<DT>(a);
}

// Largest LDS copy of the x rows (more rows go through global memory); 1 KB
// of a 64 KB block allocation is left for the kernel's own LDS.
constexpr uint64_t kGemvMaxLdsBytes = 63 * 1024;

template <int DT, int MB, int CPW, int U, int WPB>
int run(const GemvArgs& a, hipStream_t s) {
  const uint32_t blocks = (a.n_waves + WPB - 1) / WPB;
  const uint64_t lds = (uint64_t)MB * a.kc * 16;
  if (MB > 1 && lds <= kGemvMaxLdsBytes)
    hipLaunchKernelGGL((gemv_norm_kernel<DT, MB, CPW, U, WPB, (MB > 1)>), dim3(blocks),
                       dim3(64 * WPB), (uint32_t)lds, s, a);
  else
    hipLaunchKernelGGL((gemv_norm_kernel<DT, MB, CPW, U, WPB, false>), dim3(blocks),
                       dim3(64 * WPB), 0, s, a);
  return (int)hipGetLastError();
}

// rows per launch -> (rows held, columns per wave, chunks in flight per lane,
// waves per block); the columns and waves must match gemv_cols_per_wave()
// and gemv_waves_per_block()
template <int DT>
int run_rows(const GemvArgs& a, hipStream_t s) {
  if (a.m <= 1) return run<DT, 1, 2, 8, 8>(a, s);
  if (a.m <= 2) return run<DT, 2, 2, 8, 8>(a, s);
  if (a.m <= 4) return run<DT, 4, 2, 4, 4>(a, s);
  return run<DT, 8, 2, 4, 4>(a, s);
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

int launch_gemv_norm(const GemvArgs& a, int32_t dtype, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == QRP_F32) return run_rows<QRP_F32>(a, s);
  if (dtype == QRP_F16) return run_rows<QRP_F16>(a, s);
  return run_rows<QRP_BF16>(a, s);
}

}  // namespace qrp
