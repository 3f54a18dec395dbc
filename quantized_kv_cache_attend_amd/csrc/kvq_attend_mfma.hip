// Matrix-core fused attention for the 4-bit, group-32, D=128 packed cache.
#include "kvq_internal.h"

namespace kvq {

hipError_t launch_attend_mfma(const AttendProblem& p, hipStream_t stream) {
  (void)p;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace kvq
