// Streamed compression plans, bf16, d = 128 (sa_stream.hpp): 32 prototypes per
// wave with the folded matrix in registers up to k = 256 (four waves per
// group for k <= 64, eight otherwise), 64 per wave with the folded matrix in
// LDS up to k = 512.
#include "sa_stream.hpp"

namespace sa {

#define SA_PLANS(X) X(128, 32, 8, 1, 4, 1, 2) X(128, 64, 4, 1, 4, 1, 2) X(128, 64, 4, 1, 2, 1, 2) X(128, 32, 4, 1, 4, 1, 2) X(128, 32, 8, 1, 2, 1, 2) X(128, 32, 4, 2, 2, 1, 2) X(128, 32, 2, 2, 2, 1, 2) X(128, 64, 8, 1, 2, 1, 1)

hipError_t dispatch_stream_d128(const Plan& p, const FusedArgs& a, const Launch& l, int* occ) {
  SA_PLANS(SA_STREAM_PLAN)
  return hipErrorInvalidValue;
}

}  // namespace sa
