// Chunkwise gated-delta backward on gfx950 (state-gradient pass, per-chunk
// gradients, replay-gradient fixup).
#include "common.h"
#include "launch.h"

namespace harts {

hipError_t launch_kda_dstate(const KdaDims&, const BwdRoundArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_kda_grad(const KdaDims&, const BwdRoundArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_replay_fixup(const KdaDims&, const int32_t*, const int32_t*, const int32_t*, int32_t, const float*,
                               void*, void*, void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace harts
