// hq_mfma_rqa.hip -- instantiations of the matrix-core kernel for the fused
// rotation + quantisation path writing into a cache at given rows (one per
// 16-bit input dtype).
#include "hq_mfma_impl.h"

namespace hq {
namespace mfma {

hipError_t launch_rq_append(const Request &r, const DeviceInfo &dev)
{
    if (r.x_dtype == kBF16) return dispatch_op<kRotateQuant, kBF16, kAppend>(r, dev);
    return dispatch_op<kRotateQuant, kF16, kAppend>(r, dev);
}

}  // namespace mfma
}  // namespace hq
