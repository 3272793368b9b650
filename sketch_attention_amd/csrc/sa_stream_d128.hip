// Streamed compression plans, bf16, d = 128: the two 32x32x16 passes (eight
// waves of 32 prototypes; sa_wide.hpp with the prototypes along the lanes, the
// one-pass default for 128 < k <= 256, and sa_stream32.hpp, which runs the
// two phases beyond k = 512) and the 16x16x32 plans of sa_stream.hpp: 32
// prototypes per wave with the folded matrix in registers (four waves per
// group for k <= 128), 64 per wave with the folded matrix in LDS up to k = 512.
#include "sa_wide.hpp"

namespace sa {

#define SA_PLANS(X) X(128, 32, 8, 1, 4, 1, 2) X(128, 32, 4, 1, 4, 1, 2) X(128, 32, 8, 1, 2, 1, 2) X(128, 32, 4, 2, 2, 1, 2) X(128, 32, 2, 2, 2, 1, 2) X(128, 64, 8, 1, 2, 1, 1)

hipError_t dispatch_stream_d128(const Plan& p, const FusedArgs& a, const Launch& l, int* occ) {
  if (p.kind == 2) {
    if (p.kw != 32 || p.waves_k != 8 || p.waves_rows != 1) return hipErrorInvalidValue;
    const bool pad = p.k != p.k_pad;
    if (occ)
      return pad ? hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, sa_stream32_kernel<true, false, 0>, 512, 0)
                 : hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, sa_stream32_kernel<false, false, 0>, 512, 0);
    return pad ? launch_stream32_pad<true>(a, l) : launch_stream32_pad<false>(a, l);
  }
  if (p.kind == 3) {
    if (p.kw != 32 || p.waves_k != 8 || p.waves_rows != 1) return hipErrorInvalidValue;
    const bool pad = p.k != p.k_pad;
    if (occ)
      return pad ? hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, sa_wide_kernel<true, false>, 512, 0)
                 : hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, sa_wide_kernel<false, false>, 512, 0);
    return pad ? launch_wide_pad<true>(a, l) : launch_wide_pad<false>(a, l);
  }
  SA_PLANS(SA_STREAM_PLAN)
  return hipErrorInvalidValue;
}

}  // namespace sa
