// hq_fast_rq.hip -- instantiations of the register-resident kernel for the
// fused rotation + quantisation path (one per input dtype).
#include "hq_fast_impl.h"

namespace hq {
namespace fast {

hipError_t launch_rq(const Request &r, const DeviceInfo &dev)
{
    if (r.x_dtype == kF32) return dispatch_op<kRotateQuant, kF32, false>(r, dev);
    if (r.x_dtype == kBF16) return dispatch_op<kRotateQuant, kBF16, false>(r, dev);
    return dispatch_op<kRotateQuant, kF16, false>(r, dev);
}

}  // namespace fast
}  // namespace hq
