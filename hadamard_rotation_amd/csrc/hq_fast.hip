// hq_fast.hip -- register-resident kernels (placeholder: none yet).
#include "hq_internal.h"

namespace hq {

bool fast_available(const Request &r)
{
    (void)r;
    return false;
}

hipError_t launch_fast(const Request &r, const DeviceInfo &dev)
{
    (void)r;
    (void)dev;
    return hipErrorInvalidValue;
}

}  // namespace hq
