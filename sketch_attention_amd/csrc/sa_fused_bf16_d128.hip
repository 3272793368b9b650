// Fused compression plans, d = 128: bf16 inputs; eight waves per group, folded matrix in LDS, accumulators of at most 128 registers per lane.
// Each plan group is its own translation unit so groups compile in parallel
// and can take their own code-generation options.
#include "sa_fused.hpp"

namespace sa {

hipError_t dispatch_bf16_d128(const Plan& p, const FusedArgs& a, const Launch& l, int* occ) {
  SA_PLAN(bf16, 128, 16, 1, 8, true)
  SA_PLAN(bf16, 128, 32, 1, 8, true)
  SA_PLAN(bf16, 128, 64, 1, 8, true)
  SA_PLAN(bf16, 128, 64, 2, 4, true)
  SA_PLAN(bf16, 128, 64, 4, 2, true)
  SA_PLAN(bf16, 128, 64, 8, 1, true)
  return hipErrorInvalidValue;
}

}  // namespace sa
