// Fused compression plans, d = 128: float32 inputs; four waves per group, folded matrix in registers
// (four waves over 16, 32 or 64 prototypes each also run the comparator).
// Each plan group is its own translation unit so groups compile in parallel
// and can take their own code-generation options.
#include "sa_fused.hpp"

namespace sa {

hipError_t dispatch_f32_d128(const Plan& p, const FusedArgs& a, const Launch& l, int* occ) {
  SA_PLAN(float, 128, 16, 1, 4, false)
  SA_PLAN(float, 128, 32, 1, 4, false)
  SA_PLAN(float, 128, 64, 1, 4, false)
  SA_PLAN(float, 128, 64, 2, 2, false)
  SA_PLAN(float, 128, 64, 4, 1, false)
  SA_PLAN(float, 128, 16, 4, 1, false)  // comparator plans (with 4 x 64 above)
  SA_PLAN(float, 128, 32, 4, 1, false)
  return hipErrorInvalidValue;
}

}  // namespace sa
