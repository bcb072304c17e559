// kernels_fp8.hip -- the band engine's launches for FP8 (OCP E4M3) caches
// with one scale per written row; Q stays in the op's dtype.
#include "band_kernel.hpp"

namespace qrp {

int launch_fp8(const BandArgs& a, const LaunchSpec& s, void* stream) {
  if (s.dtype == DT_F32) return launch_ops<float, Fp8>(a, s, stream);
  if (s.dtype == DT_F16) return launch_ops<F16, Fp8>(a, s, stream);
  return launch_ops<Bf16, Fp8>(a, s, stream);
}

}  // namespace qrp
