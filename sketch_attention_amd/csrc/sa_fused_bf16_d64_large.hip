// Fused compression plans for bf16 inputs, d = 64: accumulators wider than 128 registers per lane (AGPR-resident).
// Each plan group is its own translation unit so groups compile in parallel
// and can take their own code-generation options.
#include "sa_fused.hpp"

namespace sa {

hipError_t dispatch_bf16_d64_large(const Plan& p, const FusedArgs& a, int groups, hipStream_t st, int* occ) {
  SA_PLAN(bf16, 64, 256, 4, true)
  return hipErrorInvalidValue;
}

}  // namespace sa
