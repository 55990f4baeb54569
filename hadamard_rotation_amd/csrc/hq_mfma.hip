// hq_mfma.hip -- host side of the matrix-core kernels: which requests they
// take, argument setup and dispatch to the per-path translation units
// (hq_mfma_rq.hip, hq_mfma_rot.hip).  The kernel template is in
// hq_mfma_impl.h.
#include <mutex>

#include "hq_mfma_impl.h"

namespace hq {
namespace mfma {

namespace {

int ilog2(int v)
{
    int r = 0;
    while ((1 << r) < v)
        ++r;
    return r;
}

struct OccEntry {
    const void *fn;
    size_t lds;
    int waves;
};
std::mutex g_occ_mu;
OccEntry g_occ[256];
int g_occ_used = 0;

}  // namespace

// Power-of-two rows of 32..4096 elements, rotated whole or in 128-element
// blocks: the forward paths on a 16-bit type, and the inverse path with one
// scale per row (its codes are exact in f16; group-wise scales make the
// dequantised values inexact there and stay on the butterfly kernel).
bool wide_inv_ok(const Request &r)
{
    // the inverse of 128-blocks as rows of one block: rows wider than the
    // per-row plans take (or not a power of two), or one scale per block
    if (r.op != kDequantInv || r.b != 128 || r.n <= 128 || r.n % 128 != 0)
        return false;
    const bool pow2 = (r.n & (r.n - 1)) == 0;
    const bool per_row_planned = pow2 && r.n <= 4096;
    if (!(r.group == 128 || (r.group == r.n && !per_row_planned)))
        return false;
    return r.rows * (int64_t)(r.n / 128) < ((int64_t)1 << 31);
}

bool wide_fwd_ok(const Request &r)
{
    // rotation + quantisation of 128-blocks with one scale per block, as rows
    // of one block, where the per-row plans do not take the row width
    if (r.op != kRotateQuant || r.dst_rows || r.b != 128 || r.group != 128 || r.n <= 128 ||
        r.n % 128 != 0)
        return false;
    if (r.x_dtype != kBF16 && r.x_dtype != kF16)
        return false;
    const bool pow2 = (r.n & (r.n - 1)) == 0;
    if (pow2 && r.n <= 4096)
        return false;
    return r.rows * (int64_t)(r.n / 128) < ((int64_t)1 << 31);
}

// The rotation alone of rows of several 128-blocks that the per-row tile
// plans do not take (wider than 4096, or not a power of two), 16-bit input:
// with no row scale the blocks are independent, so they run as rows of one
// block, each with the signs of its place in its real row.
bool wide_rot_ok(const Request &r)
{
    if (r.op != kRotate || r.b != 128 || r.n <= 128 || r.n % 128 != 0)
        return false;
    if (r.x_dtype != kBF16 && r.x_dtype != kF16)
        return false;
    const bool pow2 = (r.n & (r.n - 1)) == 0;
    if (pow2 && r.n <= 4096)
        return false;
    return r.rows * (int64_t)(r.n / 128) < ((int64_t)1 << 31);
}

bool plan_ok(const Request &r)
{
    if (wide_fwd_ok(r) || long_fwd_ok(r) || wide_rot_ok(r))
        return true;
    if (r.op == kDequantInv) {
        if (wide_inv_ok(r))
            return true;
        // group-wise scales: groups of at least one 32-element chunk
        if (r.group != r.n && r.logg < 5)
            return false;
    } else if (r.x_dtype != kBF16 && r.x_dtype != kF16) {
        return false;
    }
    if (r.n < 32 || r.n > 4096 || (r.n & (r.n - 1)) != 0)
        return false;
    // group-wise scales (forward quantisation, inverse): groups of 32 .. n/2
    if (r.group != r.n && (r.op == kRotate || r.logg < 5))
        return false;
    return r.b == r.n || (r.b == 128 && r.n >= 256);
}

void fill_args(MfmaArgs &ma, const Request &r, int tiles_per_group)
{
    ma.x = r.x;
    ma.s = r.s;
    ma.codes = r.codes;
    ma.scales = r.scales;
    ma.y = r.y;
    ma.rows = r.rows;
    ma.total = r.rows * (int64_t)r.n;
    ma.ngroups = r.rows * (int64_t)(r.n / r.group);
    ma.logg = r.logg;
    ma.dst_rows = r.dst_rows;
    ma.cache_rows = r.cache_rows;
    const int64_t per_group = (int64_t)tiles_per_group * 512;
    ma.groups = (ma.total + per_group - 1) / per_group;
    const int logb = ilog2(r.b);
    const int n_dpp = logb - 5 < 4 ? logb - 5 : 4;
    fast::dpp_tables(n_dpp, ma.pi, ma.neg);
    ma.n = r.n;
    ma.bits = r.bits;
    ma.scale_f16 = r.scale_dtype == kF16;
    const int qmax = r.bits == 8 ? 127 : 7;
    ma.kq = (float)(1.0 / (__builtin_sqrt((double)r.b) * qmax));
    ma.rb = (float)(1.0 / __builtin_sqrt((double)r.b));
}

int occupancy_waves(const void *fn, size_t lds)
{
    std::lock_guard<std::mutex> lk(g_occ_mu);
    for (int i = 0; i < g_occ_used; ++i)
        if (g_occ[i].fn == fn && g_occ[i].lds == lds)
            return g_occ[i].waves;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, 256, lds) != hipSuccess || nb < 1)
        nb = 1;
    const int waves = 4 * nb;
    if (g_occ_used < (int)(sizeof g_occ / sizeof g_occ[0]))
        g_occ[g_occ_used++] = OccEntry{fn, lds, waves};
    return waves;
}

hipError_t launch_rq(const Request &r, const DeviceInfo &dev);
hipError_t launch_rq_grouped(const Request &r, const DeviceInfo &dev);
hipError_t launch_rq_wide(const Request &r, const DeviceInfo &dev);
hipError_t launch_rq_long(const Request &r, const DeviceInfo &dev);
hipError_t launch_rq_append(const Request &r, const DeviceInfo &dev);
hipError_t launch_rot(const Request &r, const DeviceInfo &dev);
hipError_t launch_rot_wide(const Request &r, const DeviceInfo &dev);
hipError_t launch_inv(const Request &r, const DeviceInfo &dev);

}  // namespace mfma

bool mfma_available(const Request &r)
{
    return mfma::plan_ok(r);
}

hipError_t launch_mfma(const Request &r, const DeviceInfo &dev)
{
    if (r.op == kRotate)
        return mfma::wide_rot_ok(r) ? mfma::launch_rot_wide(r, dev) : mfma::launch_rot(r, dev);
    if (r.op == kDequantInv)
        return mfma::launch_inv(r, dev);
    if (r.dst_rows)
        return mfma::launch_rq_append(r, dev);
    if (mfma::long_fwd_ok(r))
        return mfma::launch_rq_long(r, dev);
    if (mfma::wide_fwd_ok(r))
        return mfma::launch_rq_wide(r, dev);
    return r.group == r.n ? mfma::launch_rq(r, dev) : mfma::launch_rq_grouped(r, dev);
}

}  // namespace hq
