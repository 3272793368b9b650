// Streamed compression plans, bf16, d = 128 (sa_stream.hpp): 32 prototypes per
// wave, folded matrix in registers, eight waves per group (four for k <= 64).
#include "sa_stream.hpp"

namespace sa {

#define SA_PLANS(X) X(128, 32, 8, 1, 4, 1) X(128, 32, 8, 1, 2, 1) X(128, 32, 4, 2, 2, 1) X(128, 32, 2, 2, 2, 1)

hipError_t dispatch_stream_d128(const Plan& p, const FusedArgs& a, int groups, hipStream_t st, int* occ) {
  SA_PLANS(SA_STREAM_PLAN)
  return hipErrorInvalidValue;
}

}  // namespace sa
