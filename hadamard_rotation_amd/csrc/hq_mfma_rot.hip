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

// Rows of several 128-blocks (see wide_rot_ok) as rows of one block: the
// grid form, or groups of 2 or 4 tiles, as for other 128-element rows.
template <int IN>
hipError_t launch_rot_wide_in(const Request &w, const DeviceInfo &dev, int blocks)
{
    if (grid_launch(w, dev))
        return launch_one<kRotate, IN, 8, 7, 7, 7, false, true, true>(w, dev, blocks);
    const int64_t groups4 = (w.rows * 128 + 4 * 512 - 1) / (4 * 512);
    if (groups4 < (int64_t)dev.cu_count * 16 * 4)
        return launch_one<kRotate, IN, 2, 7, 7, 7, false, true>(w, dev, blocks);
    return launch_one<kRotate, IN, 4, 7, 7, 7, false, true>(w, dev, blocks);
}

hipError_t launch_rot_wide(const Request &r, const DeviceInfo &dev)
{
    const int blocks = r.n / 128;
    Request w = r;
    w.rows = r.rows * blocks;
    w.n = 128;
    w.group = 128;
    w.logg = 7;
    if (r.x_dtype == kBF16)
        return launch_rot_wide_in<kBF16>(w, dev, blocks);
    return launch_rot_wide_in<kF16>(w, dev, blocks);
}

}  // namespace mfma
}  // namespace hq
