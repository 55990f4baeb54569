// launch_stubs.hip -- test infrastructure: stand-ins for the kernel
// launchers of libhq.so, so that the library's host-side argument
// validation (hq_api.hip) and the width split (hq_paley.hip) can be built
// host-only with AddressSanitizer and UndefinedBehaviorSanitizer and run
// without a GPU.  Every request that passes validation and would launch a
// kernel reaches one of these and is reported as a HIP error instead; the
// ABI tests run against this host-only library make no such request.
#include "hq_internal.h"

namespace hq {

bool paley_mfma_available(const Request &) { return false; }
bool generic_paley_fits(const Request &, const DeviceInfo &) { return false; }
bool fast_available(const Request &) { return false; }
bool mfma_available(const Request &) { return false; }
hipError_t launch_generic(const Request &, const DeviceInfo &) { return hipErrorNotSupported; }
hipError_t launch_paley_mfma(const Request &, const DeviceInfo &) { return hipErrorNotSupported; }
hipError_t launch_fast(const Request &, const DeviceInfo &) { return hipErrorNotSupported; }
hipError_t launch_mfma(const Request &, const DeviceInfo &) { return hipErrorNotSupported; }
hipError_t launch_attention(const AttnRequest &) { return hipErrorNotSupported; }
hipError_t attention_static_workspace(void **) { return hipErrorNotSupported; }

}  // namespace hq
