// kernels_pack.hip -- every op in the token-packed layout, for plain and FP8
// caches with Q in the op's dtype: a pass is one head of a block of
// consecutive tokens (grid rows, for the padded grid), one row per token, so
// launches whose segments have fewer heads than a pass has rows (a GPU's
// share of the heads under head parallelism) keep every lane busy.
#include "band_kernel.hpp"

namespace qrp {

int launch_pack(const BandArgs& a, const LaunchSpec& s, void* stream) {
  if (s.q_dtype != s.dtype) return (int)hipErrorInvalidValue;
  if (s.cache_fp8) {
    if (s.dtype == DT_F32) return launch_ops<float, Fp8, true>(a, s, stream);
    if (s.dtype == DT_F16) return launch_ops<F16, Fp8, true>(a, s, stream);
    return launch_ops<Bf16, Fp8, true>(a, s, stream);
  }
  if (s.dtype == DT_F32) return launch_ops<float, float, true>(a, s, stream);
  if (s.dtype == DT_F16) return launch_ops<F16, F16, true>(a, s, stream);
  return launch_ops<Bf16, Bf16, true>(a, s, stream);
}

}  // namespace qrp
