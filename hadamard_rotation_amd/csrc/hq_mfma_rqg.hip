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

// Rows of several 128-blocks with one scale per block (see wide_fwd_ok) as
// rows of one block with one scale per row; groups of 2 or 4 tiles as for
// other 128-element rows.
hipError_t launch_rq_wide(const Request &r, const DeviceInfo &dev)
{
    const int blocks = r.n / 128;
    Request w = r;
    w.rows = r.rows * blocks;
    w.n = 128;
    w.group = 128;
    w.logg = 7;
    const int64_t groups4 = (w.rows * 128 + 4 * 512 - 1) / (4 * 512);
    const bool two = groups4 < (int64_t)dev.cu_count * 16 * 4;
    if (r.x_dtype == kBF16)
        return two ? launch_one<kRotateQuant, kBF16, 2, 7, 7, 7, false, true>(w, dev, blocks)
                   : launch_one<kRotateQuant, kBF16, 4, 7, 7, 7, false, true>(w, dev, blocks);
    return two ? launch_one<kRotateQuant, kF16, 2, 7, 7, 7, false, true>(w, dev, blocks)
               : launch_one<kRotateQuant, kF16, 4, 7, 7, 7, false, true>(w, dev, blocks);
}

}  // namespace mfma
}  // namespace hq
