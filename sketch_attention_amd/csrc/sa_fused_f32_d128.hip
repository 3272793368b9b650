// Fused compression kernels for f32 inputs, d = 128.  One translation unit
// per (dtype, d) so the instantiations compile in parallel.
#include "sa_fused.hpp"

namespace sa {

hipError_t launch_fused_f32_d128(const Plan& p, const FusedArgs& a, int groups, hipStream_t st) {
  return dispatch_fused<float, 128>(p, a, groups, st, nullptr);
}

hipError_t occupancy_f32_d128(const Plan& p, int* n) {
  static const FusedArgs unused{};
  return dispatch_fused<float, 128>(p, unused, 0, nullptr, n);
}

}  // namespace sa
