// hq_mfma_rqg.hip -- instantiations of the matrix-core kernel for the fused
// rotation + quantisation path with group-wise scales (one per input dtype).
#include "hq_mfma_impl.h"

namespace hq {
namespace mfma {

hipError_t launch_rq_grouped(const Request &r, const DeviceInfo &dev)
{
    if (r.x_dtype == kBF16) return dispatch_op<kRotateQuant, kBF16, kGrouped>(r, dev);
    return dispatch_op<kRotateQuant, kF16, kGrouped>(r, dev);
}

}  // namespace mfma
}  // namespace hq
