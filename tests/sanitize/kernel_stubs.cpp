// Kernel launchers for the host-only sanitized build of the library
// (tests/test_sanitized_host.py): pool.cpp and capi.cpp are compiled with
// AddressSanitizer and UndefinedBehaviorSanitizer by the host compiler, and
// these stand in for the HIP kernels.  Host-only pools never launch a
// kernel; an attention call that passes validation gets hipErrorNoDevice.
#include "internal.h"

namespace hswa {

int pool_apply_blocks(int n_recs, int32_t) { return n_recs; }

hipError_t launch_pool_apply(const PoolDev&, const PoolRec*, int, const int32_t*, int32_t,
                             int32_t*, int32_t, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_append(const AttnParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_xfer(const XferParams&, bool, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_copy(const CopyParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill(const AttnParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode(const AttnParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t decode_scratch(float**) { return hipErrorNoDevice; }

}  // namespace hswa
