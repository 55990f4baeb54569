// hq_fast_rqg.hip -- instantiations of the register-resident kernel for the
// fused rotation + quantisation path with group-wise scales (one per input
// dtype).
#include "hq_fast_impl.h"

namespace hq {
namespace fast {

hipError_t launch_rq_grouped(const Request &r, const DeviceInfo &dev)
{
    if (r.x_dtype == kF32) return dispatch_op<kRotateQuant, kF32, true>(r, dev);
    if (r.x_dtype == kBF16) return dispatch_op<kRotateQuant, kBF16, true>(r, dev);
    return dispatch_op<kRotateQuant, kF16, true>(r, dev);
}

}  // namespace fast
}  // namespace hq
