// hq_fast_invg.hip -- instantiations of the register-resident kernel for the
// dequantisation + inverse rotation path with group-wise scales (one per
// output dtype).
#include "hq_fast_impl.h"

namespace hq {
namespace fast {

hipError_t launch_inv_grouped(const Request &r, const DeviceInfo &dev)
{
    if (r.y_dtype == kF32) return dispatch_op<kDequantInv, kF32, true>(r, dev);
    return dispatch_op<kDequantInv, kBF16, true>(r, dev);
}

}  // namespace fast
}  // namespace hq
