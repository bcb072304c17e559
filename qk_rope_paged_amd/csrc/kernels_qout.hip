// kernels_qout.hip -- the rope / split / store launches whose Q output has
// a dtype of its own (rope_split_store_paged_ragged page, Parameters:
// q_out_dtype), for plain and FP8 caches, in both layouts.
#include "band_kernel.hpp"

namespace qrp {
namespace {

template <typename T, typename QT>
int launch_q(const BandArgs& a, const LaunchSpec& s, void* stream) {
  if (s.pack)
    return s.cache_fp8 ? launch_store<T, QT, Fp8, true>(a, s, stream)
                       : launch_store<T, QT, T, true>(a, s, stream);
  return s.cache_fp8 ? launch_store<T, QT, Fp8>(a, s, stream) : launch_store<T, QT, T>(a, s, stream);
}

template <typename T>
int launch_t_q(const BandArgs& a, const LaunchSpec& s, void* stream) {
  if (s.q_dtype == DT_F32) {
    if constexpr (!std::is_same_v<T, float>) return launch_q<T, float>(a, s, stream);
  } else if (s.q_dtype == DT_F16) {
    if constexpr (!std::is_same_v<T, F16>) return launch_q<T, F16>(a, s, stream);
  } else {
    if constexpr (!std::is_same_v<T, Bf16>) return launch_q<T, Bf16>(a, s, stream);
  }
  return (int)hipErrorInvalidValue;  // same dtype: not this unit's launch
}

}  // namespace

int launch_qout(const BandArgs& a, const LaunchSpec& s, void* stream) {
  if (s.radd || s.bshd || has_norm(a)) return (int)hipErrorInvalidValue;
  if (s.dtype == DT_F32) return launch_t_q<float>(a, s, stream);
  if (s.dtype == DT_F16) return launch_t_q<F16>(a, s, stream);
  return launch_t_q<Bf16>(a, s, stream);
}

}  // namespace qrp
