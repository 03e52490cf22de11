// Stage 1 for an MXFP4 latent cache: not built yet. The launcher reports
// hipErrorNotSupported so that a run on an MXFP4 plan fails loudly.
#include "device_common.h"
#include "launch.h"

namespace mla {

hipError_t launch_stage1_mxfp4(const int4*, int, const uint8_t*, const float*, const uint8_t*,
                               const uint8_t*, float, float*, float*, uint16_t*, float*,
                               hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace mla
