// MLA (latent) paged decode.  Placeholder until the MFMA kernel lands:
// reports the configuration as unsupported.
#include "pkv_launch.h"

namespace pkv {

bool mla_decode_supported(const PoolInfo&, int32_t) { return false; }

DecodePlan plan_mla_decode(const PoolInfo&, int32_t, int32_t, int32_t) {
  DecodePlan p;
  p.chunk = 0;
  p.max_splits = 1;
  p.kind = 0;
  return p;
}

size_t mla_workspace_bytes(const PoolInfo&, const DecodePlan&, int32_t, int32_t) { return 0; }

hipError_t launch_mla_decode(const PoolInfo&, int32_t, const void*, int32_t, const DevMap&, int32_t,
                             const DecodePlan&, float, void*, float*, void*, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace pkv
