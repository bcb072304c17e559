// kernels.hip -- the band engine's launches for caches of the op's own
// dtype, and the dispatch to the FP8-cache, Q-dtype, token-packed and
// mixed-cache translation units.
#include "band_kernel.hpp"

namespace qrp {

int launch_plain(const BandArgs& a, const LaunchSpec& s, void* stream) {
  if (s.dtype == DT_F32) return launch_ops<float, float>(a, s, stream);
  if (s.dtype == DT_F16) return launch_ops<F16, F16>(a, s, stream);
  return launch_ops<Bf16, Bf16>(a, s, stream);
}

int launch_band(const BandArgs& a, const LaunchSpec& s, void* stream) {
  if (s.cache_mixed) return launch_mixed(a, s, stream);
  if (s.q_dtype != s.dtype) return launch_qout(a, s, stream);
  if (s.pack) return launch_pack(a, s, stream);
  if (s.cache_fp8) return launch_fp8(a, s, stream);
  return launch_plain(a, s, stream);
}

}  // namespace qrp
