// Stand-ins for the kernel launchers, for the host-only build of the C ABI
// (api.cpp + plan.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.
// The argument checks run before any launch; a call that gets this far
// returns hipErrorNoDevice (the host build has no kernels).
#include "launch.h"

namespace gptoss {

hipError_t launch_fwd(const FwdArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_noalloc(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_rope_table(float2*, int, double, double, double, double, double, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_rope_rows(const uint16_t*, uint16_t*, const int*, const float2*, int, long long, int, int, bool,
                            hipStream_t) {
    return hipErrorNoDevice;
}

}  // namespace gptoss
