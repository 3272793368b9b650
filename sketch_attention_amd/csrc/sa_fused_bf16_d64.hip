// Fused compression plans for bf16 inputs, d = 64: accumulators of at most 128 registers per lane.
// Each plan group is its own translation unit so groups compile in parallel
// and can take their own code-generation options.
#include "sa_fused.hpp"

namespace sa {

hipError_t dispatch_bf16_d64(const Plan& p, const FusedArgs& a, int groups, hipStream_t st, int* occ) {
  SA_PLAN(bf16, 64, 16, 1, false)
  SA_PLAN(bf16, 64, 32, 1, false)
  SA_PLAN(bf16, 64, 64, 1, false)
  SA_PLAN(bf16, 64, 64, 2, false)
  SA_PLAN(bf16, 64, 64, 4, false)
  SA_PLAN(bf16, 64, 16, 1, true)
  SA_PLAN(bf16, 64, 32, 1, true)
  SA_PLAN(bf16, 64, 64, 1, true)
  SA_PLAN(bf16, 64, 64, 2, true)
  SA_PLAN(bf16, 64, 64, 4, true)
  SA_PLAN(bf16, 64, 128, 2, true)
  SA_PLAN(bf16, 64, 128, 4, true)
  return hipErrorInvalidValue;
}

}  // namespace sa
