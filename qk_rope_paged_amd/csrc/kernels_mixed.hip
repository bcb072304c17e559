// kernels_mixed.hip -- the dual band's launches when its two caches differ
// in element type, one holding the op's dtype and the other FP8 codes with a
// scale per row (fused_dual_qk_rms_norm_rope_ragged_paged page, Signature:
// main_cache_dtype and index_cache_dtype are separate parameters).  Each row
// picks its cache's form at run time (BandArgs::fp8_caches); the per-token
// layout and the norm build serve every such launch (segments without a
// gamma skip the norm in it).
#include "band_kernel.hpp"

namespace qrp {

int launch_mixed(const BandArgs& a, const LaunchSpec& s, void* stream) {
  if (s.radd || s.bshd || s.pack || s.q_dtype != s.dtype) return (int)hipErrorInvalidValue;
  if (s.dtype == DT_F32)
    return s.interleaved ? launch_d<float, float, MixFp8, true, false, true, false>(a, s.head_dim, stream)
                         : launch_d<float, float, MixFp8, false, false, true, false>(a, s.head_dim, stream);
  if (s.dtype == DT_F16)
    return s.interleaved ? launch_d<F16, F16, MixFp8, true, false, true, false>(a, s.head_dim, stream)
                         : launch_d<F16, F16, MixFp8, false, false, true, false>(a, s.head_dim, stream);
  return s.interleaved ? launch_d<Bf16, Bf16, MixFp8, true, false, true, false>(a, s.head_dim, stream)
                       : launch_d<Bf16, Bf16, MixFp8, false, false, true, false>(a, s.head_dim, stream);
}

}  // namespace qrp
