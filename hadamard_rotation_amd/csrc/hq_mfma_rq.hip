// hq_mfma_rq.hip -- instantiations of the matrix-core kernel for the fused
// rotation + quantisation path (one per 16-bit input dtype).
#include "hq_mfma_impl.h"

namespace hq {
namespace mfma {

hipError_t launch_rq(const Request &r, const DeviceInfo &dev)
{
    if (r.x_dtype == kBF16) return dispatch_op<kRotateQuant, kBF16, kPerRow>(r, dev);
    return dispatch_op<kRotateQuant, kF16, kPerRow>(r, dev);
}

}  // namespace mfma
}  // namespace hq
