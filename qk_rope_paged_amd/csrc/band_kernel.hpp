// band_kernel.hpp -- the band engine: ragged RoPE / split / paged store, the
// fused per-head RMSNorm + RoPE (single and dual band) and the K/V radd,
// hand-written for gfx950 (CDNA4, wave64).
//
// What is computed (Modular MAX kernel documentation):
//   * rope_split_store_paged_ragged page, Summary and Args: a ragged flat
//     QKV buffer is split into Q, K and V heads; Q and K are rotated at the
//     token's position (Parameters: interleaved), Q goes to a dense output,
//     K and V go into the paged cache of layer layer_idx;
//   * fused_dual_qk_rms_norm_rope_ragged_paged page, Description: per-head
//     RMSNorm before the rotation, K updated in place in its cache, two bands
//     of rows in one launch with per-row band selection;
//   * generic_kv_cache_radd_dispatch page, Summary and Description: the K and
//     V halves of `a` accumulated into the cache rows of the batch;
//   * generic_fused_qk_rope_bshd_continuous_batch page, Args: the padded
//     [batch][seq_len] grid, rotation only below each valid length;
//   * rope_split_store_paged_ragged page, Parameters (freq_dtype,
//     q_out_dtype) and Args (kv_collection with a scale dtype and a
//     quantization granularity): tables, Q outputs and caches of other
//     element types, FP8 caches with one scale per written row.
//
// The kernel template is instantiated by four translation units (plain
// caches; FP8 caches; Q outputs in another dtype; the token-packed layout)
// that build in parallel.
//
// How it maps onto the chip.  The pass is HBM-bound (about one flop per byte
// moved), so there is no MFMA and no LDS staging of bulk data:
//   * one wave per (token, group of passes); a pass is 64 lanes over RPP head
//     rows, D/16 lanes per bf16x128 row, every lane owning two 16-byte chunks
//     (one dwordx4 load and store each).  The chunk pairing is chosen so that
//     a RoPE pair never leaves its lane: half-split lanes hold chunk c and
//     chunk c + rope_dim/16 (bf16), interleaved lanes hold two chunks whose
//     pairs are inside the chunk;
//   * when segments have fewer heads than a pass has rows, the token-packed
//     layout instead gives a wave a block of RPP consecutive tokens: a pass is
//     one head of one segment, one row per token, and the metadata below is
//     resolved per row;
//   * every wave fetches each 64-byte line of the argument block in one round
//     at entry (the block is written just before the launch, so its lines
//     start cold);
//   * all buffer loads of a wave's passes are issued before the token's
//     metadata chain (offsets -> cache length -> page table) resolves, so the
//     chain overlaps the data fetch; the metadata is wave-uniform and read
//     with scalar loads;
//   * the freqs row of the token's position lives in registers and serves
//     every head of the token (each lane always needs the same columns);
//   * the per-head sum of squares is reduced across the row's lanes with DPP
//     (quad_perm, row_half_mirror, row_mirror); gammas are staged in LDS, one
//     copy per wave, with no block barrier;
//   * an XCD-contiguous block remap is available (QRP_XCD_REMAP=1) but off by
//     default: blocks are dealt to the 8 XCDs round-robin.
#ifndef QRP_BAND_KERNEL_HPP
#define QRP_BAND_KERNEL_HPP

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "engine.hpp"

namespace qrp {
namespace {

typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// Element types: float (binary32), Bf16 and F16 (16-bit words), Fp8 (OCP
// E4M3 codes, cache rows only, each row with a binary32 or bf16 scale).
struct Bf16 {
  uint16_t bits;
};
struct F16 {
  uint16_t bits;
};
struct Fp8 {
  uint8_t bits;
};
// Cache type of a launch whose two caches differ: one holds the op's dtype,
// the other FP8 codes (BandArgs::fp8_caches says which).
struct MixFp8 {};

// elements per 16-byte chunk
template <typename T>
struct Fmt {
  static constexpr int E = 16 / (int)sizeof(T);
};

// Streamed rows (read once / written once) may bypass cache retention with
// nontemporal accesses; the switches exist to measure both forms.
#ifndef QRP_NT_LOADS
#define QRP_NT_LOADS 1
#endif
#ifndef QRP_NT_STORES
#define QRP_NT_STORES 1
#endif


typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// a head-row chunk that is read exactly once
__device__ __forceinline__ uint4 ld16s(const void* p) {
#if QRP_NT_LOADS
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return ld16(p);
#endif
}

// a head-row chunk that is written exactly once
__device__ __forceinline__ void st16s(void* p, const uint4 v) {
#if QRP_NT_STORES
  const v4u w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<v4u*>(p));
#else
  *reinterpret_cast<uint4*>(p) = v;
#endif
}

typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// 8- and 4-byte parts of streamed rows (FP8 cache chunks, narrow Q outputs)
__device__ __forceinline__ uint2 ld8s(const void* p) {
  const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ld4s(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ void st8s(void* p, uint32_t a, uint32_t b) {
  const v2u w = {a, b};
  __builtin_nontemporal_store(w, reinterpret_cast<v2u*>(p));
}
__device__ __forceinline__ void st4s(void* p, uint32_t a) {
  __builtin_nontemporal_store(a, reinterpret_cast<uint32_t*>(p));
}

template <typename T>
__device__ __forceinline__ void unpack(const uint4 v, float* f) {
  if constexpr (std::is_same_v<T, float>) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  } else if constexpr (std::is_same_v<T, Bf16>) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);  // a bf16 is the top half of a binary32
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const h2v h = __builtin_bit_cast(h2v, w[i]);  // binary16 -> binary32 is exact
      f[2 * i] = (float)h.x;
      f[2 * i + 1] = (float)h.y;
    }
  }
}

// two binary32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const f2v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2v));
}

// two binary32 -> packed binary16, round to nearest even
__device__ __forceinline__ uint32_t pack2_f16(float lo, float hi) {
  const f2v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2v));
}

template <typename T>
__device__ __forceinline__ uint4 pack(const float* f) {
  uint4 v;
  if constexpr (std::is_same_v<T, F16>) {
    v.x = pack2_f16(f[0], f[1]);
    v.y = pack2_f16(f[2], f[3]);
    v.z = pack2_f16(f[4], f[5]);
    v.w = pack2_f16(f[6], f[7]);
  } else if constexpr (std::is_same_v<T, float>) {
    v.x = __float_as_uint(f[0]);
    v.y = __float_as_uint(f[1]);
    v.z = __float_as_uint(f[2]);
    v.w = __float_as_uint(f[3]);
  } else {
    v.x = pack2_bf16(f[0], f[1]);
    v.y = pack2_bf16(f[2], f[3]);
    v.z = pack2_bf16(f[4], f[5]);
    v.w = pack2_bf16(f[6], f[7]);
  }
  return v;
}

// value rounded to the storage dtype, back in binary32
template <typename T>
__device__ __forceinline__ float to_dtype(float x) {
  if constexpr (std::is_same_v<T, float>) {
    return x;
  } else if constexpr (std::is_same_v<T, F16>) {
    return (float)(_Float16)x;
  } else {
    return (float)(__bf16)x;
  }
}

// E binary32 values -> the words of E elements of U, nearest-even.  Fp8
// values must already lie in [-448, 448] (the conversion gives NaN past the
// largest finite code instead of saturating).
template <typename U, int E>
__device__ __forceinline__ void to_words(const float* f, uint32_t* w) {
  if constexpr (std::is_same_v<U, float>) {
#pragma unroll
    for (int e = 0; e < E; ++e) w[e] = __float_as_uint(f[e]);
  } else if constexpr (std::is_same_v<U, Bf16>) {
#pragma unroll
    for (int i = 0; i < E / 2; ++i) w[i] = pack2_bf16(f[2 * i], f[2 * i + 1]);
  } else if constexpr (std::is_same_v<U, F16>) {
#pragma unroll
    for (int i = 0; i < E / 2; ++i) w[i] = pack2_f16(f[2 * i], f[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * i], f[4 * i + 1], 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * i + 2], f[4 * i + 3], v, true);
      w[i] = (uint32_t)v;
    }
  }
}

// Store the words of E elements of U (4, 8, 16 or 32 bytes) at p.
template <typename U, int E>
__device__ __forceinline__ void st_chunk(U* p, const uint32_t* w) {
  constexpr int B = E * (int)sizeof(U);
  if constexpr (B == 32) {
    st16s(p, make_uint4(w[0], w[1], w[2], w[3]));
    st16s(reinterpret_cast<char*>(p) + 16, make_uint4(w[4], w[5], w[6], w[7]));
  } else if constexpr (B == 16) {
    st16s(p, make_uint4(w[0], w[1], w[2], w[3]));
  } else if constexpr (B == 8) {
    st8s(p, w[0], w[1]);
  } else {
    static_assert(B == 4, "chunk size");
    st4s(p, w[0]);
  }
}

// E codes of an FP8 chunk (in the low words of v) times the row's scale, in
// binary32.  The product is rounded on its own: contracting it into a
// following add (an FMA) would skip that rounding.
template <int E>
__device__ __forceinline__ void fp8_values(const uint4 v, float s, float* f) {
#pragma clang fp contract(off)
  const uint32_t w[2] = {v.x, v.y};
#pragma unroll
  for (int i = 0; i < E / 4; ++i) {
    const int q = (int)w[i];
    f[4 * i] = __builtin_amdgcn_cvt_f32_fp8(q, 0) * s;
    f[4 * i + 1] = __builtin_amdgcn_cvt_f32_fp8(q, 1) * s;
    f[4 * i + 2] = __builtin_amdgcn_cvt_f32_fp8(q, 2) * s;
    f[4 * i + 3] = __builtin_amdgcn_cvt_f32_fp8(q, 3) * s;
  }
}

// One FP8 chunk (E bytes) of a cache row, in the low words of a uint4.
template <int E>
__device__ __forceinline__ uint4 ld_fp8_chunk(const uint8_t* p) {
  if constexpr (E == 8) {
    const uint2 v = ld8s(p);
    return make_uint4(v.x, v.y, 0, 0);
  } else {
    return make_uint4(ld4s(p), 0, 0, 0);
  }
}

// The scale of one FP8 cache row (binary32 or bf16 storage).
__device__ __forceinline__ float load_scale(const ScaleDesc& cd, int64_t idx) {
  if (cd.scale_bf16)
    return __uint_as_float((uint32_t)(reinterpret_cast<const uint16_t*>(cd.scales)[idx]) << 16);
  return reinterpret_cast<const float*>(cd.scales)[idx];
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the LPR consecutive lanes holding one head row.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LPR >= 8) v += dpp<0x141>(v);  // row_half_mirror: the other quad of 8
  if constexpr (LPR >= 16) v += dpp<0x140>(v);  // row_mirror: the other half of 16
  if constexpr (LPR >= 32) v += __shfl_xor(v, 16);
  return v;
}

// Largest value over the LPR consecutive lanes holding one head row.
template <int LPR>
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  if constexpr (LPR >= 8) v = fmaxf(v, dpp<0x141>(v));
  if constexpr (LPR >= 16) v = fmaxf(v, dpp<0x140>(v));
  if constexpr (LPR >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  return v;
}

// Quantize one head row, held as v0/v1 by the LPR lanes of the row, to FP8
// codes with one scale: every step in binary32 -- amax over the row,
// s = amax / 448 (rounded to bf16 for a bf16 scale), r = 1 / s (0 for an
// all-zero row), code = nearest-even of clamp(v * r, +-448).  Stores the
// lane's two chunks at row + c*E and, from the row's first lane, the scale.
template <int LPR, int E>
__device__ __forceinline__ void quantize_store(float* v0, float* v1, Fp8* row, uint32_t c0,
                                               uint32_t c1, const ScaleDesc& cd, int64_t sidx,
                                               bool active, bool first) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) m = fmaxf(m, fmaxf(fabsf(v0[e]), fabsf(v1[e])));
  m = row_max<LPR>(m);
  float s = m / 448.0f;
  uint32_t sbits = __float_as_uint(s);
  if (cd.scale_bf16) {
    sbits = pack2_bf16(s, s) & 0xFFFFu;
    s = __uint_as_float(sbits << 16);
  }
  const float r = s > 0.0f ? 1.0f / s : 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v0[e] = fminf(fmaxf(v0[e] * r, -448.0f), 448.0f);
    v1[e] = fminf(fmaxf(v1[e] * r, -448.0f), 448.0f);
  }
  uint32_t w0[E / 4], w1[E / 4];
  to_words<Fp8, E>(v0, w0);
  to_words<Fp8, E>(v1, w1);
  if (active) {
    st_chunk<Fp8, E>(row + c0 * E, w0);
    st_chunk<Fp8, E>(row + c1 * E, w1);
    if (first) {
      if (cd.scale_bf16)
        __builtin_nontemporal_store((uint16_t)sbits, reinterpret_cast<uint16_t*>(cd.scales) + sidx);
      else
        __builtin_nontemporal_store(sbits, reinterpret_cast<uint32_t*>(cd.scales) + sidx);
    }
  }
}

// Rotate a lane's two chunks by its (cos, sin) entries fl: interleaved
// chunks hold their pairs inside each chunk; half-split lanes hold element e
// of the real half in v0 and its partner in v1.  rot0 / rot1 say whether the
// chunk rotates at all.
template <bool IL, int E>
__device__ __forceinline__ void rope_chunks(float* v0, float* v1, const float* fl, bool rot0,
                                            bool rot1) {
  if constexpr (IL) {
#pragma unroll
    for (int m = 0; m < E / 2; ++m) {
      const float a0 = v0[2 * m], b0 = v0[2 * m + 1];
      const float cs = fl[2 * m], sn = fl[2 * m + 1];
      v0[2 * m] = rot0 ? a0 * cs - b0 * sn : a0;
      v0[2 * m + 1] = rot0 ? a0 * sn + b0 * cs : b0;
      const float a1 = v1[2 * m], b1 = v1[2 * m + 1];
      const float cs1 = fl[E + 2 * m], sn1 = fl[E + 2 * m + 1];
      v1[2 * m] = rot1 ? a1 * cs1 - b1 * sn1 : a1;
      v1[2 * m + 1] = rot1 ? a1 * sn1 + b1 * cs1 : b1;
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float re = v0[e], im = v1[e];
      const float cs = fl[2 * e], sn = fl[2 * e + 1];
      v0[e] = rot0 ? re * cs - im * sn : re;
      v1[e] = rot0 ? re * sn + im * cs : im;
    }
  }
}

// Largest b < B with off[b] <= t, for batches of kSmallBatch sequences or
// more.  The guess g = t * B / T (a host-computed 32.32 fixed-point factor) is
// exact for one-token-per-sequence decode: its two offsets are loaded
// together and checked, and a miss falls back to a binary search over the
// side the guess left open.  Every index read is <= B.  `hit` reports a
// resolved guess.
constexpr uint32_t kSmallBatch = 16;

__device__ __forceinline__ uint32_t find_seq(const uint32_t* __restrict__ off, uint32_t B,
                                             uint32_t g, uint32_t t, uint32_t& start,
                                             uint32_t& end, bool& hit) {
  const uint32_t lo_v = off[g];
  const uint32_t hi_v = off[g + 1];
  hit = (lo_v <= t) & (t < hi_v);
  if (hit) {
    start = lo_v;
    end = hi_v;
    return g;
  }
  uint32_t lo = 0, hi = B;
  if (lo_v <= t)
    lo = g;
  else
    hi = g;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) >> 1;
    if (off[mid] <= t)
      lo = mid;
    else
      hi = mid;
  }
  start = off[lo];
  end = off[lo + 1];
  return lo;
}

// The small-batch metadata (17 offsets, 16 cache lengths of each cache)
// through one empty asm statement: no instruction, but the compiler must have
// every value in an SGPR at that point, which keeps all 49 loads ahead of it
// (issued together, waited for once).  The values are uniform.
__device__ __forceinline__ void pin49(uint32_t* o, uint32_t* c, uint32_t* d) {
#pragma unroll
  for (int i = 0; i < 17; ++i) o[i] = __builtin_amdgcn_readfirstlane(o[i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    c[i] = __builtin_amdgcn_readfirstlane(c[i]);
    d[i] = __builtin_amdgcn_readfirstlane(d[i]);
  }
  asm(""
      : "+s"(o[0]), "+s"(o[1]), "+s"(o[2]), "+s"(o[3]), "+s"(o[4]), "+s"(o[5]), "+s"(o[6]),
        "+s"(o[7]), "+s"(o[8]), "+s"(o[9]), "+s"(o[10]), "+s"(o[11]), "+s"(o[12]), "+s"(o[13]),
        "+s"(o[14]), "+s"(o[15]), "+s"(o[16]), "+s"(c[0]), "+s"(c[1]), "+s"(c[2]), "+s"(c[3]),
        "+s"(c[4]), "+s"(c[5]), "+s"(c[6]), "+s"(c[7]), "+s"(c[8]), "+s"(c[9]), "+s"(c[10]),
        "+s"(c[11]), "+s"(c[12]), "+s"(c[13]), "+s"(c[14]), "+s"(c[15]), "+s"(d[0]), "+s"(d[1]),
        "+s"(d[2]), "+s"(d[3]), "+s"(d[4]), "+s"(d[5]), "+s"(d[6]), "+s"(d[7]), "+s"(d[8]),
        "+s"(d[9]), "+s"(d[10]), "+s"(d[11]), "+s"(d[12]), "+s"(d[13]), "+s"(d[14]),
        "+s"(d[15]));
}

__device__ __forceinline__ uint32_t seg_of(const BandArgs& a, uint32_t kp) {
  uint32_t s = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i)
    if (kp >= a.seg_begin[i - 1]) s = (uint32_t)i;
  return s;
}

// N consecutive freqs table entries of type FDT, widened (exactly) to binary32.
template <int FDT, int N>
__device__ __forceinline__ void table_entries(const void* base, int64_t idx, float* out) {
  if constexpr (FDT == DT_F32) {
    const float* p = static_cast<const float*>(base) + idx;
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const uint4 v = ld16(p + 4 * q);
      out[4 * q] = __uint_as_float(v.x);
      out[4 * q + 1] = __uint_as_float(v.y);
      out[4 * q + 2] = __uint_as_float(v.z);
      out[4 * q + 3] = __uint_as_float(v.w);
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + idx;
    uint32_t w[N / 2];
    if constexpr (N == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x;
      w[1] = v.y;
    } else {
#pragma unroll
      for (int q = 0; q < N / 8; ++q) {
        const uint4 v = ld16(p + 8 * q);
        w[4 * q] = v.x;
        w[4 * q + 1] = v.y;
        w[4 * q + 2] = v.z;
        w[4 * q + 3] = v.w;
      }
    }
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      if constexpr (FDT == DT_BF16) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      } else {
        const h2v h = __builtin_bit_cast(h2v, w[i]);
        out[2 * i] = (float)h.x;
        out[2 * i + 1] = (float)h.y;
      }
    }
  }
}

// The loads are unconditional: a chunk that does not rotate reads the
// table's first entries instead (every table has at least rope_dim >= 2E
// columns and one row), and its values go unused.  A load under a lane
// condition would be compiled into a branch that waits for every load in
// flight before the next one issues.
template <int FDT, typename T, bool IL>
__device__ __forceinline__ void load_freqs_t(const void* __restrict__ freqs, int64_t row,
                                             uint32_t c0, uint32_t c1, uint32_t j, bool rot0,
                                             bool rot1, float* fl) {
  constexpr int E = Fmt<T>::E;
  if constexpr (IL) {
    // chunk c holds pairs c*E/2 .. c*E/2 + E/2 - 1: table columns c*E .. c*E + E - 1
    table_entries<FDT, E>(freqs, rot0 ? row + c0 * E : 0, fl);
    table_entries<FDT, E>(freqs, rot1 ? row + c1 * E : 0, fl + E);
  } else {
    // a half-split lane j < rope_dim/(2E) rotates frequencies j*E .. j*E + E - 1
    table_entries<FDT, 2 * E>(freqs, rot0 ? row + 2 * j * E : 0, fl);
  }
}

// This lane's (cos, sin) entries of freqs row `pos`: the 2E table values of
// the frequencies its chunks rotate (table values of no meaning where a
// chunk is not rotated: the rotation selects the unrotated value there).
// c0 / c1 are the chunks' places within the rotated dims.
// The table's entry type is uniform over the launch.
template <typename T, bool IL>
__device__ __forceinline__ void load_freqs(const BandArgs& a, uint32_t pos, uint32_t c0,
                                           uint32_t c1, uint32_t j, bool rot0, bool rot1,
                                           float* fl) {
  const int64_t row = (int64_t)pos * a.rope_dim;
  if (a.freq_dtype == DT_F32)
    load_freqs_t<DT_F32, T, IL>(a.freqs, row, c0, c1, j, rot0, rot1, fl);
  else if (a.freq_dtype == DT_BF16)
    load_freqs_t<DT_BF16, T, IL>(a.freqs, row, c0, c1, j, rot0, rot1, fl);
  else
    load_freqs_t<DT_F16, T, IL>(a.freqs, row, c0, c1, j, rot0, rot1, fl);
}

// Bring every 64-byte line of the first BYTES bytes of the argument block
// into the scalar cache at once: one dword load per line, all in flight
// together, taken as operands by one empty asm statement (no instruction, no
// memory access, so the loads complete before it and nothing else is
// ordered by it).  The block is written just before the launch, so its lines
// start cold: fetched this way they cost one miss latency per wave on the
// launch's ramp, instead of one per line in the order the code first reads
// them.  Returns the block's first dword, passed through the asm, so that
// the caller's work depends on the fetch.
template <uint32_t BYTES>
__device__ __forceinline__ void line_words(uint32_t (&v)[12]) {
  using kptr = const uint32_t __attribute__((address_space(4)))*;
  const kptr k = (kptr)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr uint32_t N = (BYTES + 63) / 64;
  static_assert(N >= 1 && N <= 12, "one asm operand per line");
#pragma unroll
  for (uint32_t i = 0; i < 12; ++i) {
    const uint32_t l = i < N ? i : N - 1;
    v[i] = k[l + 1 < N ? l * 16 : (BYTES - 4) / 4];  // the last line: the block's last dword
  }
}

template <uint32_t BYTES>
__device__ __forceinline__ uint32_t touch_args() {
  uint32_t v[12];
  line_words<BYTES>(v);
  asm("" : "+s"(v[0]) : "s"(v[1]), "s"(v[2]), "s"(v[3]), "s"(v[4]), "s"(v[5]), "s"(v[6]),
      "s"(v[7]), "s"(v[8]), "s"(v[9]), "s"(v[10]), "s"(v[11]));
  return v[0];
}

// The same, also passing four 64-bit values through the statement (the norm
// kernels' gamma pointers, their first loads' addresses), so that they are
// loaded in the same round.
template <uint32_t BYTES>
__device__ __forceinline__ uint32_t touch_args(uint64_t (&p)[4]) {
  uint32_t v[12];
  line_words<BYTES>(v);
  asm("" : "+s"(v[0]), "+s"(p[0]), "+s"(p[1]), "+s"(p[2]), "+s"(p[3])
      : "s"(v[1]), "s"(v[2]), "s"(v[3]), "s"(v[4]), "s"(v[5]), "s"(v[6]), "s"(v[7]), "s"(v[8]),
        "s"(v[9]), "s"(v[10]), "s"(v[11]));
  return v[0];
}

// T: input (and norm / plain cache) element type; QT: Q output element type;
// CT: cache element type (T, or Fp8 with a scale per row).
template <typename T, typename QT, typename CT, int D, bool IL, int NPMAX, bool RADD, bool NORM,
          bool BSHD, bool PACK = false>
__global__ void __launch_bounds__(kThreads) band_kernel(const BandArgs a) {
  // QUANT: every cache holds FP8 codes; MIX: the caches differ (a per-cache
  // run-time bit); QANY: FP8 rows may occur.
  constexpr bool QUANT = std::is_same_v<CT, Fp8>;
  constexpr bool MIX = std::is_same_v<CT, MixFp8>;
  constexpr bool QANY = QUANT || MIX;
  static_assert(QANY || std::is_same_v<CT, T>, "a cache holds the op dtype or FP8");
  static_assert(!MIX || (NORM && !RADD && !BSHD && !PACK), "mixed caches: the norm ops' build");
  // does cache ci hold FP8 codes
  auto fp8_cache = [&](uint32_t ci) -> bool {
    if constexpr (MIX) return (a.fp8_caches >> ci) & 1u;
    return QUANT;
  };
  constexpr int E = Fmt<T>::E;
  constexpr int CH = D / E;      // 16-byte chunks per head row
  constexpr int LPR = CH / 2;    // lanes per head row
  constexpr int RPP = 64 / LPR;  // head rows per pass
  static_assert(LPR >= 4 && LPR <= 32, "unsupported head_dim / dtype");

  static_assert(offsetof(BandArgs, n_items) == 0, "the fetch returns n_items");
  constexpr uint32_t ARG_BYTES =
      QANY ? (uint32_t)sizeof(BandArgs) : (uint32_t)offsetof(BandArgs, scale);
  // norm kernels: every segment's gamma pointer (null for unused segments,
  // whose descriptors are zero), fetched with the argument lines
  uint64_t gpv[kMaxSegs] = {0, 0, 0, 0};
  uint32_t n_items;
  if constexpr (NORM) {
#pragma unroll
    for (int q = 0; q < kMaxSegs; ++q) gpv[q] = (uint64_t)a.seg[q].gamma;
    n_items = touch_args<ARG_BYTES>(gpv);
  } else {
    n_items = touch_args<ARG_BYTES>();
  }
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Waves past the work (a last block's spare waves, blocks the XCD remap
  // adds) run on a clamped item and leave at the metadata check: no branch
  // before the first loads, so the header's fields arrive in one round.
  uint32_t blk = blockIdx.x;
  uint32_t item_raw;
  bool dead;
  if (a.per_xcd & kUnitsOnXcd) {
    // Blocks are dealt to the XCDs round-robin (block b runs on XCD b % 8).
    // Give each unit (token, or token block) bpu consecutive blocks of one
    // XCD -- blocks x, x + 8, x + 16, ... -- so that its waves share that
    // XCD's L2 (one fetch of its freqs row and metadata), while the units
    // at work at any moment stay neighbours, spread over all XCDs.
    const uint32_t bpu = a.per_xcd & ~kUnitsOnXcd;
    const uint32_t x = blk % kXcds, sl = blk / kXcds;
    const uint32_t jq = sl / bpu;
    const uint32_t g = (sl - jq * bpu) * a.waves_per_block + wave;  // group within the unit
    item_raw = (jq * kXcds + x) * a.groups_per_token + g;
    dead = g >= a.groups_per_token || item_raw >= n_items;
  } else {
    blk = a.per_xcd ? (blk % kXcds) * a.per_xcd + blk / kXcds : blk;
    item_raw = blk * a.waves_per_block + wave;
    dead = blk >= a.n_blocks || item_raw >= n_items;
  }
  const uint32_t item = dead ? n_items - 1 : item_raw;

  // Gammas of every segment, per wave, in LDS.  Reading them there keeps the
  // store loop free of vector-memory loads (vmcnt counts stores as well as
  // loads, so a load issued after a store would wait for it).  The gamma
  // loads issue first, ahead of the buffer loads; each wave writes its own
  // copy when phase E starts (it waits for its data there anyway), so no
  // barrier holds the metadata chain.  LDS operations of one wave execute in
  // order: the reads that follow see the write.
  __shared__ uint4 lds_gamma[NORM ? kMaxWavesPerBlock : 1][NORM ? kMaxSegs : 1][NORM ? CH : 1];
  constexpr uint32_t GPT = NORM ? (kMaxSegs * CH + 63) / 64 : 1;  // chunks per lane
  uint4 gst[GPT];
  if constexpr (NORM) {
#pragma unroll
    for (uint32_t k = 0; k < GPT; ++k) {
      const uint32_t i = lane + 64 * k;
      const uint32_t si = i / CH, c = i % CH;
      // the segment differs across lanes: select among the uniform
      // (scalar-loaded) pointers rather than index the argument array
      uint64_t gp = 0;
#pragma unroll
      for (uint32_t q = 0; q < (uint32_t)kMaxSegs; ++q)
        if (si == q) gp = gpv[q];
      gst[k] = make_uint4(0, 0, 0, 0);
      // a global-memory pointer again (an integer cast would give a flat
      // load, which also counts against the scalar loads' wait counter)
      using v4u = unsigned int __attribute__((ext_vector_type(4)));
      using gptr = const v4u __attribute__((address_space(1)))*;
      if (i < kMaxSegs * CH && gp != 0) {
        const v4u w = ((gptr)gp)[c];
        gst[k] = make_uint4(w.x, w.y, w.z, w.w);
      }
    }
  }

  // A wave's unit: one token (its passes cover the token's head rows, RPP
  // heads of one segment per pass), or with PACK a block of RPP consecutive
  // tokens (a pass is one head of one segment, one row per token: nothing
  // idles when segments have fewer heads than a pass has rows).
  uint32_t unit, p0, np;
  if (item < a.tail_item) {
    unit = item / a.groups_per_token;
    p0 = (item - unit * a.groups_per_token) * a.passes_per_group;
    np = min(a.passes_per_group, a.passes_per_token - p0);
  } else {
    // the launch's last units: one pass per wave
    const uint32_t r = item - a.tail_item;
    const uint32_t q = r / a.passes_per_token;
    unit = a.tail_unit + q;
    p0 = r - q * a.passes_per_token;
    np = 1;
  }

  // this lane's row within a pass and its two chunks within the row
  const uint32_t row = lane / LPR;
  const uint32_t j = lane % LPR;
  // this row's token: wave-uniform, or per row with PACK (rows past the last
  // token read the last one's rows and write nothing)
  uint32_t t = unit;
  bool tok_ok = true;
  if constexpr (PACK) {
    const uint32_t tr = unit * RPP + row;
    tok_ok = tr < a.total_tokens;
    t = tok_ok ? tr : a.total_tokens - 1;
  }
  // The rotated dims are chunks oc .. oc + rope_dim/E - 1 (oc = 0, or the
  // last rope_dim dims of the head).  Half-split, leading dims: lanes j < hh
  // hold rotated chunk j and its partner j + hh, the other lanes two of the
  // chunks 2hh .. that pass through.  The trailing layout is that list turned
  // by oc chunks (mod D/E, a power of two): rotated chunks land on oc.., the
  // pass-through ones on 0 .. oc - 1.  Branch-free, so the lanes stay
  // converged while the first loads issue.
  constexpr uint32_t NC = D / E;
  static_assert((NC & (NC - 1)) == 0, "chunks per head must be a power of two");
  const uint32_t oc = a.rope_off_chunks;
  const uint32_t hh = (IL || RADD) ? (uint32_t)LPR : a.rope_dim / (2 * E);
  uint32_t c0, c1;
  if constexpr (IL || RADD) {
    c0 = j;
    c1 = j + LPR;
  } else {
    const bool lead = j < hh;
    c0 = (j + (lead ? 0u : hh) + oc) & (NC - 1);
    c1 = (j + (lead ? hh : (uint32_t)LPR) + oc) & (NC - 1);
  }
  // interleaved: a chunk rotates when c - oc < rope_dim/E (unsigned, so the
  // chunks before oc wrap past the bound)
  const uint32_t rot_chunks = a.rope_dim / E;
  bool rot0 = !RADD && (IL ? c0 - oc < rot_chunks : j < hh);
  bool rot1 = !RADD && (IL ? c1 - oc < rot_chunks : j < hh);

  uint4 x[NPMAX][2];
  uint4 y[RADD ? NPMAX : 1][2];

  // ---- A: loads from the input buffer (no metadata needed) ----
#pragma unroll
  for (int p = 0; p < NPMAX; ++p) {
    x[p][0] = x[p][1] = make_uint4(0, 0, 0, 0);
    if ((uint32_t)p < np) {
      const uint32_t kp = p0 + p;
      const SegDesc& sd = a.seg[seg_of(a, kp)];
      // the address before the branch: one scalar-load round for the fields
      const uint32_t h = min(PACK ? kp - sd.pass_begin : (kp - sd.pass_begin) * RPP + row,
                             sd.n_heads - 1);
      const T* src = reinterpret_cast<const T*>(sd.src) + (int64_t)t * sd.src_row_stride +
                     (int64_t)h * D;
      if (!((a.inplace_segs >> seg_of(a, kp)) & 1u)) {
        x[p][0] = ld16s(src + c0 * E);
        x[p][1] = ld16s(src + c1 * E);
      }
    }
  }

  // ---- B: token -> sequence -> position -> page (wave-uniform) ----
  uint32_t start, end, b;
  uint32_t clen[kMaxCaches] = {0, 0};
  bool pass = false;  // padded grid: a row past its sequence's valid length
  if constexpr (BSHD) {
    b = t / a.seq_len;
    start = b * a.seq_len;
    end = start + a.seq_len;
    const uint32_t vl = a.valid_lengths[b];
    clen[0] = a.cache[0].cache_lengths[b];
    pass = t - start >= vl;
  } else if (a.batch < kSmallBatch) {
    // Small batch: every offset and every sequence's cache length in one
    // round of independent scalar loads (indices clamped in range), then a
    // scan -- one load latency before the page-table lookup.  Every load is
    // unconditional: a load guarded by the cache count would be compiled
    // into a branch of its own that waits for the loads before it (16
    // dependent rounds).  With one cache the second pointer names the first
    // cache's array (valid loads, values unused).  The batch size and
    // offset, and then the loaded values, pass through empty asm statements:
    // the compiler must hold them in SGPRs there, so those fields are read
    // (scalar-cache hits) before the first metadata load, and every metadata
    // load is issued before the first wait on one.
    uint32_t B = a.batch, boff = a.batch_offset;
    const uint32_t* offp = a.offsets;
    const uint32_t* clp0 = a.cache[0].cache_lengths;
    const uint32_t* clp1 = a.ncache > 1 ? a.cache[1].cache_lengths : clp0;
    asm("" : "+s"(B), "+s"(boff));
    uint32_t o[kSmallBatch + 1];
    uint32_t cl[kMaxCaches][kSmallBatch];
#pragma unroll
    for (uint32_t i = 0; i <= kSmallBatch; ++i) o[i] = offp[i < B ? i : B];
#pragma unroll
    for (uint32_t i = 0; i < kSmallBatch; ++i) {
      cl[0][i] = clp0[(i < B ? i : B - 1) + boff];
      cl[1][i] = clp1[(i < B ? i : B - 1) + boff];
    }
    pin49(o, cl[0], cl[1]);
    b = 0;
#pragma unroll
    for (uint32_t i = 1; i < kSmallBatch; ++i)
      if (i < B && o[i] <= t) b = i;
    start = o[0];
    end = o[1];
    clen[0] = cl[0][0];
    clen[1] = cl[1][0];
#pragma unroll
    for (uint32_t i = 1; i < kSmallBatch; ++i) {
      if (i == b) {
        start = o[i];
        end = o[i + 1];
        clen[0] = cl[0][i];
        clen[1] = cl[1][i];
      }
    }
  } else {
    // The guess's offsets and both caches' lengths in one round (pointers
    // first; with one cache the second pointer names the first cache's
    // array, a valid load whose value goes unused), so a decode wave pays one
    // load latency before its page-table lookup.
    const uint32_t B = a.batch;
    const uint32_t* const cl0 = a.cache[0].cache_lengths + a.batch_offset;
    const uint32_t* const cl1 =
        (a.ncache > 1 ? a.cache[1].cache_lengths : a.cache[0].cache_lengths) + a.batch_offset;
    uint32_t g = (uint32_t)(((uint64_t)t * a.guess_mul) >> 32);
    g = g < B ? g : B - 1;
    const uint32_t cg0 = cl0[g], cg1 = cl1[g];
    bool hit;
    b = find_seq(a.offsets, B, g, t, start, end, hit);
    clen[0] = hit ? cg0 : cl0[b];
    clen[1] = hit ? cg1 : cl1[b];
  }
  bool ok = !dead && tok_ok && start <= t && t < end;
  const uint32_t local = t - start;
  const uint32_t cseq = b + a.batch_offset;
  uint32_t pos[kMaxCaches] = {0, 0};
  int64_t base[kMaxCaches] = {0, 0};
  int64_t sbase[kMaxCaches] = {0, 0};  // FP8: the row's scale index before plane and head
  uint64_t pidx_c[kMaxCaches] = {0, 0}, slot_c[kMaxCaches] = {0, 0};
#pragma unroll
  for (int ci = 0; ci < kMaxCaches; ++ci) {
    if ((uint32_t)ci < a.ncache) {
      const CacheDesc& cd = a.cache[ci];
      const uint64_t p64 = (uint64_t)clen[ci] + local;
      const uint64_t pidx = cd.page_shift != 0xFFFFFFFFu ? (p64 >> cd.page_shift)
                                                         : p64 / cd.page_size;
      slot_c[ci] = p64 - pidx * cd.page_size;
      pidx_c[ci] = pidx;
      ok = ok && (pass || ((a.max_seq_len == 0 || p64 < a.max_seq_len) && pidx < cd.max_pages));
      pos[ci] = (uint32_t)p64;
    }
  }
  // One-pass waves (decode-sized launches, the padded grid) and the store
  // op over FP8 caches load the freqs row as soon as the position is known:
  // its address needs no page-table entry, so the two lookups overlap
  // (measured: decode 3.17 -> 3.09 us per launch, prefill over an FP8
  // cache 35.12 -> 34.50; the plain prefill and the dual band ran 0.6 and
  // 1.2 % slower with it, so they keep the freqs load after the lookup).
  constexpr bool EARLY_FREQS = (NPMAX == 1 || (QUANT && !NORM)) && !RADD;
  float fl[RADD ? 1 : 2 * E];
  uint32_t fl_pos = pos[0];
  if constexpr (EARLY_FREQS) {
    const bool fok = ok && !pass;
    load_freqs<T, IL>(a, fl_pos, c0 - oc, c1 - oc, j, rot0 && fok, rot1 && fok, fl);
  }
#pragma unroll
  for (int ci = 0; ci < kMaxCaches; ++ci) {
    if ((uint32_t)ci < a.ncache) {
      const CacheDesc& cd = a.cache[ci];
      const uint64_t pidx = pidx_c[ci];
      const uint64_t slot = slot_c[ci];
      uint64_t page = 0;
      if (ok && !pass) page = cd.table[(uint64_t)cseq * cd.max_pages + pidx];
      ok = ok && (pass || page < cd.num_pages);
      base[ci] = (int64_t)page * cd.page_stride + cd.layer_off + (int64_t)slot * cd.slot_stride;
      if constexpr (QANY)
        sbase[ci] = (int64_t)page * a.scale[ci].s_page_stride + a.scale[ci].s_layer_off +
                    (int64_t)slot * a.scale[ci].s_slot_stride;
    }
  }
  // out-of-range metadata: this token writes nothing.  With PACK the rows of
  // one wave belong to different tokens: such rows stay (their wave's LDS
  // gamma copy and row reductions need every lane) and are masked below.
  if constexpr (!PACK) {
    if (!ok) return;
  }
  // a passed-through row is copied as it is; a row that writes nothing
  // (PACK) reads no freqs row either: its position is unchecked
  if (pass || !ok) rot0 = rot1 = false;

  // ---- C: loads from the cache (in-place K, radd accumulator) ----
  float rsc[QANY ? NPMAX : 1];  // FP8: scale of the row read
#pragma unroll
  for (int p = 0; p < NPMAX; ++p) {
    if constexpr (RADD) y[p][0] = y[p][1] = make_uint4(0, 0, 0, 0);
    if constexpr (QANY) rsc[p] = 0.f;
    if ((uint32_t)p < np) {
      const uint32_t kp = p0 + p;
      const SegDesc& sd = a.seg[seg_of(a, kp)];
      if (((sd.kind == SEG_K_INPLACE && !pass) || (RADD && sd.kind == SEG_RADD)) && ok) {
        const CacheDesc& cd = a.cache[sd.cache];
        const uint32_t h = min(PACK ? kp - sd.pass_begin : (kp - sd.pass_begin) * RPP + row,
                               sd.n_heads - 1);
        const int64_t roff =
            base[sd.cache] + (int64_t)sd.plane * cd.plane_stride + (int64_t)h * cd.head_stride;
        uint4 r0, r1;
        if (QANY && fp8_cache(sd.cache)) {
          const uint8_t* src = reinterpret_cast<const uint8_t*>(cd.blocks) + roff;
          r0 = ld_fp8_chunk<E>(src + c0 * E);
          r1 = ld_fp8_chunk<E>(src + c1 * E);
          const ScaleDesc& sdsc = a.scale[sd.cache];
          if constexpr (QANY)
            rsc[p] = load_scale(sdsc, sbase[sd.cache] + (int64_t)sd.plane * sdsc.s_plane_stride +
                                          (int64_t)h * sdsc.s_head_stride);
        } else {
          const T* src = reinterpret_cast<const T*>(cd.blocks) + roff;
          r0 = ld16s(src + c0 * E);
          r1 = ld16s(src + c1 * E);
        }
        if constexpr (RADD) {
          y[p][0] = r0;
          y[p][1] = r1;
        } else {
          x[p][0] = r0;
          x[p][1] = r1;
        }
      }
    }
  }

  // ---- D: this lane's (cos, sin) entries of the token's freqs row ----
  if constexpr (!RADD && !EARLY_FREQS) load_freqs<T, IL>(a, fl_pos, c0 - oc, c1 - oc, j, rot0, rot1, fl);


  // ---- E: arithmetic and stores ----
  if constexpr (NORM) {
#pragma unroll
    for (uint32_t k = 0; k < GPT; ++k) {
      const uint32_t i = lane + 64 * k;
      if (i < kMaxSegs * CH) lds_gamma[wave][i / CH][i % CH] = gst[k];
    }
  }
#pragma unroll
  for (int p = 0; p < NPMAX; ++p) {
    if ((uint32_t)p < np) {
      const uint32_t kp = p0 + p;
      const uint32_t si = seg_of(a, kp);
      const SegDesc& sd = a.seg[si];
      const uint32_t kind = sd.kind;
      const uint32_t h = PACK ? kp - sd.pass_begin : (kp - sd.pass_begin) * RPP + row;
      const bool active = ok && h < sd.n_heads && !(BSHD && pass && kind != SEG_Q);
      T* dst;
      if (kind == SEG_Q) {
        dst = reinterpret_cast<T*>(sd.dst) + (int64_t)t * sd.dst_row_stride + (int64_t)h * D;
      } else {
        const CacheDesc& cd = a.cache[sd.cache];
        dst = reinterpret_cast<T*>(cd.blocks) + base[sd.cache] + (int64_t)sd.plane * cd.plane_stride +
              (int64_t)h * cd.head_stride;
      }
      uint4 o0, o1;
      if constexpr (RADD) {
        if constexpr (QUANT) {
          // dequantize, one binary32 add, quantize the row again
          const CacheDesc& cd = a.cache[sd.cache];
          float va0[E], va1[E], vc0[E], vc1[E];
          unpack<T>(x[p][0], va0);
          unpack<T>(x[p][1], va1);
          fp8_values<E>(y[p][0], rsc[p], vc0);
          fp8_values<E>(y[p][1], rsc[p], vc1);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            vc0[e] = vc0[e] + va0[e];
            vc1[e] = vc1[e] + va1[e];
          }
          quantize_store<LPR, E>(
              vc0, vc1,
              reinterpret_cast<Fp8*>(cd.blocks) + base[sd.cache] +
                  (int64_t)sd.plane * cd.plane_stride + (int64_t)h * cd.head_stride,
              c0, c1, a.scale[sd.cache],
              sbase[sd.cache] + (int64_t)sd.plane * a.scale[sd.cache].s_plane_stride +
                  (int64_t)h * a.scale[sd.cache].s_head_stride,
              active, j == 0);
          continue;
        } else {
          float va[E], vc[E];
          unpack<T>(x[p][0], va);
          unpack<T>(y[p][0], vc);
#pragma unroll
          for (int e = 0; e < E; ++e) vc[e] = vc[e] + va[e];  // one binary32 add
          o0 = pack<T>(vc);
          unpack<T>(x[p][1], va);
          unpack<T>(y[p][1], vc);
#pragma unroll
          for (int e = 0; e < E; ++e) vc[e] = vc[e] + va[e];
          o1 = pack<T>(vc);
        }
      } else {
        if (kind == SEG_V_COPY) {
          if (QANY && fp8_cache(sd.cache)) {
            // V bits cannot move into an FP8 row as they are: quantize them
            const CacheDesc& cd = a.cache[sd.cache];
            float v0[E], v1[E];
            unpack<T>(x[p][0], v0);
            unpack<T>(x[p][1], v1);
            quantize_store<LPR, E>(
                v0, v1,
                reinterpret_cast<Fp8*>(cd.blocks) + base[sd.cache] +
                    (int64_t)sd.plane * cd.plane_stride + (int64_t)h * cd.head_stride,
                c0, c1, a.scale[sd.cache],
                sbase[sd.cache] + (int64_t)sd.plane * a.scale[sd.cache].s_plane_stride +
                    (int64_t)h * a.scale[sd.cache].s_head_stride,
                active, j == 0);
            continue;
          } else {
            o0 = x[p][0];
            o1 = x[p][1];
          }
        } else {
          const bool fp8_row = QANY && kind != SEG_Q && fp8_cache(sd.cache);
          float v0[E], v1[E];
          if (fp8_row && kind == SEG_K_INPLACE) {
            fp8_values<E>(x[p][0], rsc[QANY ? p : 0], v0);
            fp8_values<E>(x[p][1], rsc[QANY ? p : 0], v1);
          } else {
            unpack<T>(x[p][0], v0);
            unpack<T>(x[p][1], v1);
          }
          const bool norm = NORM && sd.gamma != nullptr;
          if constexpr (NORM) {
            if (norm) {
              float ss = 0.f;
#pragma unroll
              for (int e = 0; e < E; ++e) ss += v0[e] * v0[e] + v1[e] * v1[e];
              ss = row_sum<LPR>(ss);
              const float r = __builtin_amdgcn_rsqf(ss * (1.0f / D) + sd.eps);
              float g0[E], g1[E];
              unpack<T>(lds_gamma[wave][si][c0], g0);
              unpack<T>(lds_gamma[wave][si][c1], g1);
              const float w = a.weight_offset;
              if (a.multiply_before_cast) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                  v0[e] = v0[e] * r * (g0[e] + w);
                  v1[e] = v1[e] * r * (g1[e] + w);
                }
              } else {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                  v0[e] = to_dtype<T>(to_dtype<T>(v0[e] * r) * to_dtype<T>(g0[e] + w));
                  v1[e] = to_dtype<T>(to_dtype<T>(v1[e] * r) * to_dtype<T>(g1[e] + w));
                }
              }
            }
          }
          // Segments run cache 0 first, then cache 1; a second cache whose
          // cache length differs for this sequence needs the freqs row of its
          // own position (uniform, taken at most once per wave).
          if (pos[sd.cache] != fl_pos) {
            fl_pos = pos[sd.cache];
            load_freqs<T, IL>(a, fl_pos, c0 - oc, c1 - oc, j, rot0, rot1, fl);
          }
          rope_chunks<IL, E>(v0, v1, fl, rot0, rot1);
          if constexpr (!std::is_same_v<QT, T>) {
            if (kind == SEG_Q) {
              // Q in its own dtype: one rounding (un-roped elements converted)
              constexpr int W = E * (int)sizeof(QT) / 4;
              uint32_t w0[W], w1[W];
              to_words<QT, E>(v0, w0);
              to_words<QT, E>(v1, w1);
              QT* qd = reinterpret_cast<QT*>(sd.dst) + (int64_t)t * sd.dst_row_stride +
                       (int64_t)h * D;
              if (active) {
                st_chunk<QT, E>(qd + c0 * E, w0);
                st_chunk<QT, E>(qd + c1 * E, w1);
              }
              continue;
            }
          }
          if constexpr (QANY) {
            if (fp8_row) {
              const CacheDesc& cd = a.cache[sd.cache];
              quantize_store<LPR, E>(
                  v0, v1,
                  reinterpret_cast<Fp8*>(cd.blocks) + base[sd.cache] +
                      (int64_t)sd.plane * cd.plane_stride + (int64_t)h * cd.head_stride,
                  c0, c1, a.scale[sd.cache],
                  sbase[sd.cache] + (int64_t)sd.plane * a.scale[sd.cache].s_plane_stride +
                      (int64_t)h * a.scale[sd.cache].s_head_stride,
                  active, j == 0);
              continue;
            }
          }
          o0 = (norm || rot0) ? pack<T>(v0) : x[p][0];
          o1 = (norm || rot1) ? pack<T>(v1) : x[p][1];
        }
      }
      if (active) {
        st16s(dst + c0 * E, o0);
        st16s(dst + c1 * E, o1);
      }
    }
  }
}

template <typename T, typename QT, typename CT, int D, bool IL, int NPMAX, bool RADD, bool NORM,
          bool BSHD, bool PACK>
int launch_np(const BandArgs& a, void* stream) {
  const uint32_t grid =
      (a.per_xcd && !(a.per_xcd & kUnitsOnXcd)) ? a.per_xcd * kXcds : a.n_blocks;
  hipLaunchKernelGGL((band_kernel<T, QT, CT, D, IL, NPMAX, RADD, NORM, BSHD, PACK>), dim3(grid),
                     dim3(64 * a.waves_per_block), a.lds_bytes,
                     reinterpret_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

// Store kernels built for one pass per wave hold fewer registers (more
// waves resident); they run whenever the launch gives each wave one pass.
template <typename T, typename QT, typename CT, int D, bool IL, bool RADD, bool NORM, bool BSHD,
          bool PACK>
int launch_t(const BandArgs& a, void* stream) {
  constexpr bool FP8 = std::is_same_v<CT, Fp8> || std::is_same_v<CT, MixFp8>;
  constexpr int NPMAX =
      RADD ? kMaxPassesRadd
           : (NORM ? ((PACK || FP8) ? kMaxPassesNorm : kMaxPassesNormPlain)
                   : (PACK ? kMaxPassesStorePack : kMaxPassesStore));
  if constexpr (!RADD && !NORM && NPMAX > 1) {
    if (a.passes_per_group == 1)
      return launch_np<T, QT, CT, D, IL, 1, RADD, NORM, BSHD, PACK>(a, stream);
  }
  return launch_np<T, QT, CT, D, IL, NPMAX, RADD, NORM, BSHD, PACK>(a, stream);
}

template <typename T, typename QT, typename CT, bool IL, bool RADD, bool NORM, bool BSHD,
          bool PACK = false>
int launch_d(const BandArgs& a, uint32_t head_dim, void* stream) {
  switch (head_dim) {
    case 64: return launch_t<T, QT, CT, 64, IL, RADD, NORM, BSHD, PACK>(a, stream);
    case 128: return launch_t<T, QT, CT, 128, IL, RADD, NORM, BSHD, PACK>(a, stream);
    case 256: return launch_t<T, QT, CT, 256, IL, RADD, NORM, BSHD, PACK>(a, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

inline bool has_norm(const BandArgs& a) {
  bool norm = false;
  for (uint32_t s = 0; s < a.nseg; ++s) norm = norm || a.seg[s].gamma != nullptr;
  return norm;
}

// Every op for one (input, cache) element-type pair; Q in the input dtype.
// PACK: the token-packed layout.
template <typename T, typename CT, bool PACK = false>
int launch_ops(const BandArgs& a, const LaunchSpec& s, void* stream) {
  if (s.radd) return launch_d<T, T, CT, true, true, false, false, PACK>(a, s.head_dim, stream);
  if (s.bshd)
    return s.interleaved
               ? launch_d<T, T, CT, true, false, false, true, PACK>(a, s.head_dim, stream)
               : launch_d<T, T, CT, false, false, false, true, PACK>(a, s.head_dim, stream);
  if (has_norm(a))
    return s.interleaved
               ? launch_d<T, T, CT, true, false, true, false, PACK>(a, s.head_dim, stream)
               : launch_d<T, T, CT, false, false, true, false, PACK>(a, s.head_dim, stream);
  return s.interleaved ? launch_d<T, T, CT, true, false, false, false, PACK>(a, s.head_dim, stream)
                       : launch_d<T, T, CT, false, false, false, false, PACK>(a, s.head_dim, stream);
}

// The rope / split / store op with Q in its own dtype (PACK: token-packed).
template <typename T, typename QT, typename CT, bool PACK = false>
int launch_store(const BandArgs& a, const LaunchSpec& s, void* stream) {
  return s.interleaved
             ? launch_d<T, QT, CT, true, false, false, false, PACK>(a, s.head_dim, stream)
             : launch_d<T, QT, CT, false, false, false, false, PACK>(a, s.head_dim, stream);
}

}  // namespace
}  // namespace qrp

#endif  // QRP_BAND_KERNEL_HPP
