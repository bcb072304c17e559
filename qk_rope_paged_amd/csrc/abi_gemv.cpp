// abi_gemv.cpp -- the extern "C" entry point of the fused GEMV + partial
// RMSNorm (MatmulFusedPartialRMSNorm page): argument checks, the launch
// descriptor and the workspace size.  The kernel is in gemv_norm.hip.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "errors.hpp"
#include "gemv_norm.hpp"
#include "qk_rope_paged.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
uint32_t elem_bytes(int32_t dt) { return dt == QRP_F32 ? 4u : 2u; }
uint32_t chunk_elems(int32_t dt) { return 16u / elem_bytes(dt); }
bool dtype_ok(int32_t dt) { return dt == QRP_F32 || dt == QRP_BF16 || dt == QRP_F16; }

}  // namespace

extern "C" uint64_t qrp_gemv_norm_workspace_bytes(uint32_t m, uint32_t n_normed,
                                                  int32_t transpose_b) {
  return qrp::gemv_workspace_bytes(m, n_normed, transpose_b != 0);
}

namespace {

// Both entry points.  no_alloc: the scratch is the library's own (the
// workspace arguments are unused), sized for m * n_normed <= kGemvScratchFloats.
int32_t gemv_call(void* normed_output, uint64_t normed_row_stride, void* unnormed_output,
                  uint64_t unnormed_row_stride, const void* input, uint64_t input_row_stride,
                  uint32_t m, const void* weight, uint64_t weight_row_stride, uint32_t n,
                  uint32_t k, const void* gamma, uint32_t n_normed, float epsilon,
                  float weight_offset, int32_t dtype, int32_t transpose_b, void* workspace,
                  uint64_t workspace_bytes, void* stream, bool no_alloc) {
  qrp::clear_error();
  (void)weight_offset;  // not consumed by this op (its page's Args)
  if (!dtype_ok(dtype)) return qrp::set_error(QRP_EUNSUPPORTED, "dtype must be QRP_F32, QRP_BF16 or QRP_F16");
  if (transpose_b != 0 && transpose_b != 1)
    return qrp::set_error(QRP_EINVAL, "transpose_b must be 0 (W stored [k][n]) or 1 (W stored [n][k])");
  if (n_normed > n) return qrp::set_error(QRP_EINVAL, "n_normed > n");
  if (m > qrp::kGemvMaxRows) return qrp::set_error(QRP_EUNSUPPORTED, "m > 8 rows per call");
  if (m == 0 || n == 0) return QRP_OK;
  if (n >= (1u << 31)) return qrp::set_error(QRP_EINVAL, "n >= 2^31 columns in one launch");
  if (!input || !weight) return qrp::set_error(QRP_EINVAL, "input / weight is NULL");
  if (n_normed && (!gamma || !normed_output))
    return qrp::set_error(QRP_EINVAL, "gamma and normed_output are needed when n_normed > 0");
  const uint64_t ws_need = qrp::gemv_workspace_bytes(m, n_normed, transpose_b != 0);
  if (ws_need && !workspace && !no_alloc)
    return qrp::set_error(QRP_EINVAL, transpose_b ? "workspace is needed when n_normed > 0"
                                                  : "workspace is needed with W stored [k][n]");
  if (n_normed < n && !unnormed_output)
    return qrp::set_error(QRP_EINVAL, "unnormed_output is NULL with columns past n_normed");
  const uint32_t ce = chunk_elems(dtype);
  const uintptr_t eb = elem_bytes(dtype) - 1;
  if (!aligned16(input) || !aligned16(weight) || (workspace && !aligned16(workspace)))
    return qrp::set_error(QRP_EALIGN, "input, weight and workspace must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(normed_output) | reinterpret_cast<uintptr_t>(unnormed_output) |
       reinterpret_cast<uintptr_t>(gamma)) & eb)
    return qrp::set_error(QRP_EALIGN, "outputs and gamma must be aligned to their element size");
  if (k % ce || input_row_stride % ce || weight_row_stride % ce)
    return qrp::set_error(QRP_EALIGN, "k and the input / weight row strides must be multiples of 16 bytes");
  if (input_row_stride < k) return qrp::set_error(QRP_EINVAL, "input row stride < k");
  if (weight_row_stride < (transpose_b ? k : n))
    return qrp::set_error(QRP_EINVAL, transpose_b ? "weight row stride < k (W stored [n][k])"
                                                  : "weight row stride < n (W stored [k][n])");
  if (n_normed && normed_row_stride < n_normed)
    return qrp::set_error(QRP_EINVAL, "normed_row_stride < n_normed");
  if (n_normed < n && unnormed_row_stride < n - n_normed)
    return qrp::set_error(QRP_EINVAL, "unnormed_row_stride < n - n_normed");
  if (no_alloc) {
    if ((uint64_t)m * n_normed > qrp::kGemvScratchFloats)
      return qrp::set_error(QRP_EINVAL, "m * n_normed exceeds the library's scratch (" +
                                            std::to_string(qrp::kGemvScratchFloats) +
                                            " values); use matmul_fused_partial_rmsnorm");
    workspace = nullptr;
    if (ws_need) {
      const int e = qrp::gemv_scratch(&workspace, stream);
      if (e != 0)
        return qrp::set_error(QRP_EHIP, std::string("scratch set-up failed: ") +
                                            hipGetErrorString(static_cast<hipError_t>(e)));
    }
  } else if (workspace_bytes < ws_need) {
    return qrp::set_error(QRP_EINVAL,
                          "workspace smaller than qrp_gemv_norm_workspace_bytes(m, n_normed, transpose_b)");
  }

  qrp::GemvArgs a{};
  a.x = input;
  a.w = weight;
  a.gamma = gamma;
  a.normed = normed_output;
  a.unnormed = unnormed_output;
  char* ws = static_cast<char*>(workspace);
  a.counter = reinterpret_cast<uint32_t*>(ws);
  a.tile_counter = ws ? reinterpret_cast<uint32_t*>(ws + qrp::kGemvTileCounterOffset) : nullptr;
  a.ybuf = ws ? reinterpret_cast<float*>(ws + qrp::kGemvCounterBytes) : nullptr;
  a.partials = ws && !transpose_b
                   ? reinterpret_cast<float*>(ws + qrp::gemv_partials_offset(m, n_normed))
                   : nullptr;
  a.x_stride = (int64_t)input_row_stride;
  a.w_stride = (int64_t)weight_row_stride;
  a.normed_stride = (int64_t)normed_row_stride;
  a.unnormed_stride = (int64_t)unnormed_row_stride;
  a.m = m;
  a.n = n;
  a.kc = k / ce;
  a.n_normed = n_normed;
  a.eps = epsilon;
  a.transpose_b = (uint32_t)transpose_b;
  const int e = qrp::launch_gemv_norm(a, dtype, stream);
  if (e != 0)
    return qrp::set_error(QRP_EHIP, std::string("kernel launch failed: ") +
                              hipGetErrorString(static_cast<hipError_t>(e)));
  return QRP_OK;
}

}  // namespace

extern "C" {

int32_t matmul_fused_partial_rmsnorm(void* normed_output, uint64_t normed_row_stride,
                                     void* unnormed_output, uint64_t unnormed_row_stride,
                                     const void* input, uint64_t input_row_stride, uint32_t m,
                                     const void* weight, uint64_t weight_row_stride, uint32_t n,
                                     uint32_t k, const void* gamma, uint32_t n_normed,
                                     float epsilon, float weight_offset, int32_t dtype,
                                     int32_t transpose_b, void* workspace,
                                     uint64_t workspace_bytes, void* stream) {
  return gemv_call(normed_output, normed_row_stride, unnormed_output, unnormed_row_stride, input,
                   input_row_stride, m, weight, weight_row_stride, n, k, gamma, n_normed,
                   epsilon, weight_offset, dtype, transpose_b, workspace, workspace_bytes, stream,
                   false);
}

int32_t matmul_fused_partial_rmsnorm_noalloc(void* normed_output, uint64_t normed_row_stride,
                                             void* unnormed_output, uint64_t unnormed_row_stride,
                                             const void* input, uint64_t input_row_stride,
                                             uint32_t m, const void* weight,
                                             uint64_t weight_row_stride, uint32_t n, uint32_t k,
                                             const void* gamma, uint32_t n_normed, float epsilon,
                                             float weight_offset, int32_t dtype,
                                             int32_t transpose_b, void* stream) {
  return gemv_call(normed_output, normed_row_stride, unnormed_output, unnormed_row_stride, input,
                   input_row_stride, m, weight, weight_row_stride, n, k, gamma, n_normed,
                   epsilon, weight_offset, dtype, transpose_b, nullptr, 0, stream, true);
}

}  // extern "C"
