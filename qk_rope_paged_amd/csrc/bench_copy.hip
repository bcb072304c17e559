// bench_copy.hip -- a plain streaming device copy, built as its own small
// library (libqrp_bench_copy.so) so the benchmark can measure the chip's
// practical read+write bandwidth at the same byte count as one pass.  It is
// not part of the qk_rope_paged C ABI.
//
// Each thread moves U 16-byte chunks, 256 threads apart, loads first and
// stores after, with nontemporal (streaming) accesses: the form that measured
// fastest among the plain copies tried on MI355X.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <int U>
__global__ void __launch_bounds__(256) stream_copy(v4u* __restrict__ dst, const v4u* __restrict__ src,
                                                   uint64_t n16) {
  const uint64_t base = (uint64_t)blockIdx.x * 256 * U + threadIdx.x;
  v4u v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t i = base + (uint64_t)u * 256;
    if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t i = base + (uint64_t)u * 256;
    if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
  }
}

template <int U>
void launch_copy(v4u* dst, const v4u* src, uint64_t n16, hipStream_t s) {
  const uint64_t grid = (n16 + 256 * U - 1) / (256 * U);
  hipLaunchKernelGGL(stream_copy<U>, dim3((uint32_t)grid), dim3(256), 0, s, dst, src, n16);
}

}  // namespace

// Copy nbytes (a multiple of 16; both pointers 16-byte aligned) from src to
// dst on `stream` with U = chunks per thread (1, 2, 4 or 8).  Returns a
// hipError_t.
extern "C" int32_t qrp_bench_stream_copy(void* dst, const void* src, uint64_t nbytes,
                                         int32_t chunks_per_thread, void* stream) {
  if (nbytes % 16 || (reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15u)
    return (int32_t)hipErrorInvalidValue;
  const uint64_t n16 = nbytes / 16;
  if (n16 == 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  v4u* d = static_cast<v4u*>(dst);
  const v4u* r = static_cast<const v4u*>(src);
  switch (chunks_per_thread) {
    case 1: launch_copy<1>(d, r, n16, s); break;
    case 2: launch_copy<2>(d, r, n16, s); break;
    case 4: launch_copy<4>(d, r, n16, s); break;
    case 8: launch_copy<8>(d, r, n16, s); break;
    default: return (int32_t)hipErrorInvalidValue;
  }
  return (int32_t)hipGetLastError();
}
