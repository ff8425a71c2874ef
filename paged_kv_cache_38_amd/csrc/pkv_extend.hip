// Paged extend / prefill attention.  Placeholder until the MFMA kernel lands.
#include "pkv_launch.h"

namespace pkv {

bool extend_supported(const PoolInfo&, int32_t) { return false; }

hipError_t launch_extend(const PoolInfo&, int32_t, const void*, const int32_t*, int32_t, int32_t, const DevMap&,
                         int32_t, int32_t, int32_t, float, void*, float*, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace pkv
