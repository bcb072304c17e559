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

extern "C" {

uint64_t qrp_gemv_norm_workspace_bytes(uint32_t m, uint32_t n_normed) {
  if (n_normed == 0) return 0;
  return qrp::kGemvCounterBytes + 4ull * m * n_normed;
}

int32_t matmul_fused_partial_rmsnorm(void* normed_output, uint64_t normed_row_stride,
                                     void* unnormed_output, uint64_t unnormed_row_stride,
                                     const void* input, uint64_t input_row_stride, uint32_t m,
                                     const void* weight, uint64_t weight_row_stride, uint32_t n,
                                     uint32_t k, const void* gamma, uint32_t n_normed,
                                     float epsilon, float weight_offset, int32_t dtype,
                                     int32_t transpose_b, void* workspace,
                                     uint64_t workspace_bytes, void* stream) {
  qrp::clear_error();
  (void)weight_offset;  // not consumed by this op (its page's Args)
  if (!dtype_ok(dtype)) return qrp::set_error(QRP_EUNSUPPORTED, "dtype must be QRP_F32, QRP_BF16 or QRP_F16");
  if (transpose_b != 1)
    return qrp::set_error(QRP_EUNSUPPORTED, "only transpose_b = 1 (W stored [n][k]) is built");
  if (n_normed > n) return qrp::set_error(QRP_EINVAL, "n_normed > n");
  if (m > qrp::kGemvMaxRows) return qrp::set_error(QRP_EUNSUPPORTED, "m > 8 rows per call");
  if (m == 0 || n == 0) return QRP_OK;
  if (n >= (1u << 31)) return qrp::set_error(QRP_EINVAL, "n >= 2^31 columns in one launch");
  if (!input || !weight) return qrp::set_error(QRP_EINVAL, "input / weight is NULL");
  if (n_normed && (!gamma || !normed_output || !workspace))
    return qrp::set_error(QRP_EINVAL, "gamma, normed_output and workspace are needed when n_normed > 0");
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
  if (input_row_stride < k || weight_row_stride < k)
    return qrp::set_error(QRP_EINVAL, "input / weight row stride < k");
  if (n_normed && normed_row_stride < n_normed)
    return qrp::set_error(QRP_EINVAL, "normed_row_stride < n_normed");
  if (n_normed < n && unnormed_row_stride < n - n_normed)
    return qrp::set_error(QRP_EINVAL, "unnormed_row_stride < n - n_normed");
  if (workspace_bytes < qrp_gemv_norm_workspace_bytes(m, n_normed))
    return qrp::set_error(QRP_EINVAL, "workspace smaller than qrp_gemv_norm_workspace_bytes(m, n_normed)");

  qrp::GemvArgs a{};
  a.x = input;
  a.w = weight;
  a.gamma = gamma;
  a.normed = normed_output;
  a.unnormed = unnormed_output;
  a.counter = static_cast<uint32_t*>(workspace);
  a.ybuf = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                qrp::kGemvCounterBytes)
                     : nullptr;
  a.x_stride = (int64_t)input_row_stride;
  a.w_stride = (int64_t)weight_row_stride;
  a.normed_stride = (int64_t)normed_row_stride;
  a.unnormed_stride = (int64_t)unnormed_row_stride;
  a.m = m;
  a.n = n;
  a.kc = k / ce;
  a.n_normed = n_normed;
  const uint32_t cpw = qrp::gemv_cols_per_wave(m);
  a.n_waves = (uint32_t)(((uint64_t)n + cpw - 1) / cpw);
  const uint64_t norm_waves = ((uint64_t)n_normed + cpw - 1) / cpw;
  const uint32_t wpb = qrp::gemv_waves_per_block(m);
  a.n_norm_blocks = (uint32_t)((norm_waves + wpb - 1) / wpb);
  a.eps = epsilon;
  const int e = qrp::launch_gemv_norm(a, dtype, stream);
  if (e != 0)
    return qrp::set_error(QRP_EHIP, std::string("kernel launch failed: ") +
                              hipGetErrorString(static_cast<hipError_t>(e)));
  return QRP_OK;
}

}  // extern "C"
