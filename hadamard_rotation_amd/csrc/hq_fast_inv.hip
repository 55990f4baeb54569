// hq_fast_inv.hip -- instantiations of the register-resident kernel for the
// dequantisation + inverse rotation path (one per output dtype).
#include "hq_fast_impl.h"

namespace hq {
namespace fast {

hipError_t launch_inv(const Request &r, const DeviceInfo &dev)
{
    if (r.y_dtype == kF32) return dispatch_op<kDequantInv, kF32, false>(r, dev);
    return dispatch_op<kDequantInv, kBF16, false>(r, dev);
}

}  // namespace fast
}  // namespace hq
