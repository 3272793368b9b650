// Streamed compression plans, bf16, d = 128 (sa_stream.hpp): 32 prototypes per
// wave, folded matrix in registers, eight waves per group.
#include "sa_stream.hpp"

namespace sa {

hipError_t dispatch_stream_d128(const Plan& p, const FusedArgs& a, int groups, hipStream_t st, int* occ) {
  SA_STREAM_PLAN(128, 32, 8, 1, 4, 1)
  SA_STREAM_PLAN(128, 32, 8, 1, 4, 2)
  SA_STREAM_PLAN(128, 32, 8, 1, 2, 1)
  SA_STREAM_PLAN(128, 32, 4, 2, 2, 1)
  SA_STREAM_PLAN(128, 32, 2, 4, 2, 1)
  return hipErrorInvalidValue;
}

}  // namespace sa
