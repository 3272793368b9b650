// Streamed compression plans, bf16, d = 128: the 32x32x16 pass (sa_stream32.hpp,
// eight waves of 32 prototypes) and the 16x16x32 plans of sa_stream.hpp: 32 prototypes per
// wave with the folded matrix in registers up to k = 256 (four waves per
// group for k <= 64, eight otherwise), 64 per wave with the folded matrix in
// LDS up to k = 512.
#include "sa_stream32.hpp"

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
  SA_PLANS(SA_STREAM_PLAN)
  return hipErrorInvalidValue;
}

}  // namespace sa
