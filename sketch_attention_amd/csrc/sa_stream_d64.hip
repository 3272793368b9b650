// Streamed compression plans, bf16, d = 64 (sa_stream.hpp): 32 prototypes per
// wave (64 above k = 256) with the folded matrix in registers up to k = 512,
// 128 per wave with the folded matrix in LDS up to k = 1024; eight waves.
#include "sa_stream.hpp"

namespace sa {

#define SA_PLANS(X) X(64, 64, 8, 1, 2, 1, 2) X(64, 32, 4, 1, 4, 1, 2) X(64, 32, 8, 1, 4, 1, 2) X(64, 32, 4, 2, 4, 1, 2) X(64, 32, 2, 4, 2, 1, 2) X(64, 128, 8, 1, 2, 1, 1)

hipError_t dispatch_stream_d64(const Plan& p, const FusedArgs& a, const Launch& l, int* occ) {
  SA_PLANS(SA_STREAM_PLAN)
  return hipErrorInvalidValue;
}

}  // namespace sa
