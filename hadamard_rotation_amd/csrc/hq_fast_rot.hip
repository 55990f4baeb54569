// hq_fast_rot.hip -- instantiations of the register-resident kernel for the
// rotation-only path (fp32 output; one per input dtype).
#include "hq_fast_impl.h"

namespace hq {
namespace fast {

hipError_t launch_rot(const Request &r, const DeviceInfo &dev)
{
    if (r.x_dtype == kF32) return dispatch_op<kRotate, kF32, false>(r, dev);
    if (r.x_dtype == kBF16) return dispatch_op<kRotate, kBF16, false>(r, dev);
    return dispatch_op<kRotate, kF16, false>(r, dev);
}

}  // namespace fast
}  // namespace hq
