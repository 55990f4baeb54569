// hq_mfma_rot.hip -- instantiations of the matrix-core kernel for the
// rotation-only path (one per 16-bit input dtype).
#include "hq_mfma_impl.h"

namespace hq {
namespace mfma {

hipError_t launch_rot(const Request &r, const DeviceInfo &dev)
{
    if (r.x_dtype == kBF16) return dispatch_op<kRotate, kBF16, kPerRow>(r, dev);
    return dispatch_op<kRotate, kF16, kPerRow>(r, dev);
}

}  // namespace mfma
}  // namespace hq
