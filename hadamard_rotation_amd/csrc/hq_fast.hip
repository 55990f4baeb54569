// hq_fast.hip -- host side of the register-resident kernels: the launch plan
// for a row width n and block size b, argument setup and dispatch to the
// per-path translation units (hq_fast_rq.hip, hq_fast_rot.hip,
// hq_fast_inv.hip).  The kernel template is in hq_fast_impl.h.
#include <mutex>

#include "hq_fast_impl.h"

namespace hq {
namespace fast {

namespace {

// Output chunk / sign of lane l & 15 after k DPP stages (k = 0..4), from
// composing the stage matrices (acc_l += sigma_l * x_src(l)) with sigma
// taken from the functionals b0^b2, b1^b2, b2, b3 of the lane bits; every
// resulting row is +- a row of the Hadamard matrix of its 2^k-lane block.
constexpr int kPi[5][16] = {
    {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15},
    {0, 1, 2, 3, 5, 4, 7, 6, 8, 9, 10, 11, 13, 12, 15, 14},
    {0, 1, 2, 3, 7, 6, 5, 4, 8, 9, 10, 11, 15, 14, 13, 12},
    {0, 5, 6, 3, 7, 2, 1, 4, 8, 13, 14, 11, 15, 10, 9, 12},
    {0, 5, 6, 3, 7, 2, 1, 4, 8, 13, 14, 11, 15, 10, 9, 12},
};
constexpr int kSign[5][16] = {
    {1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1},
    {1, -1, 1, -1, 1, 1, 1, 1, 1, -1, 1, -1, 1, 1, 1, 1},
    {1, -1, -1, 1, 1, 1, 1, 1, 1, -1, -1, 1, 1, 1, 1, 1},
    {1, -1, -1, 1, -1, 1, 1, -1, 1, -1, -1, 1, -1, 1, 1, -1},
    {1, -1, -1, 1, -1, 1, 1, -1, -1, 1, 1, -1, 1, -1, -1, 1},
};

int ilog2(int v)
{
    int r = 0;
    while ((1 << r) < v)
        ++r;
    return r;
}

// Largest block a 64-lane segment can rotate with `units` units per lane:
// lane bit 4 needs one unit register to swap with, lane bit 5 a second.
int max_block(int units)
{
    return units == 1 ? 128 : units == 2 ? 256 : 512 * units;
}

struct OccEntry {
    const void *fn;
    int threads;
    size_t lds;
    int blocks;
};
std::mutex g_occ_mu;
OccEntry g_occ[512];
int g_occ_used = 0;

}  // namespace

bool make_plan(int n, int b, Plan &p)
{
    const int units = n >> 3;
    p.logb = ilog2(b);
    const bool pow2 = (n & (n - 1)) == 0;
    if (pow2 && n <= 4096) {
        p.wpr = 1;
        p.is_long = false;
        if (units <= 16) {
            p.units = 1;
            p.log_lanes = ilog2(units);
            p.rpl = 4;
        } else if (units <= 128) {
            p.log_lanes = 4;
            p.units = units >> 4;
            p.rpl = units == 32 ? 2 : 1;
        } else if (units == 256) {
            p.log_lanes = 5;
            p.units = 8;
            p.rpl = 1;
        } else {
            p.log_lanes = 6;
            p.units = 8;
            p.rpl = 1;
        }
        return true;
    }
    // long rows: one row per workgroup, 64-lane segments
    int best_units = 0, best_wpr = 0, best_waste = 1 << 30;
    for (int uu : {8, 4, 2, 1}) {
        const int per_wave = 64 * uu;
        const int wpr = (units + per_wave - 1) / per_wave;
        const int max_wpr = uu >= 8 ? 4 : kMaxWpr;
        if (wpr > max_wpr || b > max_block(uu))
            continue;
        const int waste = wpr * per_wave - units;
        if (waste < best_waste || (waste == best_waste && uu > best_units)) {
            best_waste = waste;
            best_units = uu;
            best_wpr = wpr;
        }
    }
    if (!best_units)
        return false;
    p.units = best_units;
    p.log_lanes = 6;
    p.rpl = 1;
    p.wpr = best_wpr;
    p.is_long = true;
    return true;
}

void dpp_tables(int n_dpp, uint64_t &pi, uint32_t &neg)
{
    pi = 0;
    neg = 0;
    for (int i = 0; i < 16; ++i) {
        pi |= (uint64_t)kPi[n_dpp][i] << (4 * i);
        neg |= (kSign[n_dpp][i] < 0 ? 1u : 0u) << i;
    }
}

void fill_args(FastArgs &fa, const Request &r, const Plan &p)
{
    fa.x = r.x;
    fa.codes_in = r.codes_in;
    fa.scales_in = r.scales_in;
    fa.s = r.s;
    fa.codes = r.codes;
    fa.scales = r.scales;
    fa.y = r.y;
    fa.rows = r.rows;
    fa.n = r.n;
    fa.logb = p.logb;
    fa.log_lanes = p.log_lanes;
    fa.wpr = p.wpr;
    fa.bits = r.bits;
    fa.scale_f16 = r.scale_dtype == kF16;
    const bool grouped = r.group != r.n;
    fa.logg = grouped ? r.logg : 0;
    fa.ngroups_row = grouped ? r.n / r.group : 1;
    const int lane_bits = p.logb > 3 ? (p.logb - 3 < p.log_lanes ? p.logb - 3 : p.log_lanes) : 0;
    const int n_dpp = lane_bits < 4 ? lane_bits : 4;
    dpp_tables(n_dpp, fa.pi, fa.neg);
    const int qmax = r.bits == 8 ? 127 : 7;
    fa.kq = (float)(1.0 / (__builtin_sqrt((double)r.b) * qmax));
    fa.rb = (float)(1.0 / __builtin_sqrt((double)r.b));
}

int occupancy_blocks(const void *fn, int threads, size_t lds)
{
    std::lock_guard<std::mutex> lk(g_occ_mu);
    for (int i = 0; i < g_occ_used; ++i)
        if (g_occ[i].fn == fn && g_occ[i].threads == threads && g_occ[i].lds == lds)
            return g_occ[i].blocks;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, threads, lds) != hipSuccess || nb < 1)
        nb = 1;
    if (g_occ_used < (int)(sizeof g_occ / sizeof g_occ[0]))
        g_occ[g_occ_used++] = OccEntry{fn, threads, lds, nb};
    return nb;
}

hipError_t launch_rq(const Request &r, const DeviceInfo &dev);
hipError_t launch_rq_grouped(const Request &r, const DeviceInfo &dev);
hipError_t launch_rot(const Request &r, const DeviceInfo &dev);
hipError_t launch_inv(const Request &r, const DeviceInfo &dev);
hipError_t launch_inv_grouped(const Request &r, const DeviceInfo &dev);

}  // namespace fast

bool fast_available(const Request &r)
{
    fast::Plan p;
    if (r.dst_rows || !fast::make_plan(r.n, r.b, p))
        return false;
    if (r.group == r.n || (r.op != kRotateQuant && r.op != kDequantInv))
        return true;
    // group-wise scales: whole 8-element units per group, and (long rows)
    // no group across two waves' segments
    if (r.logg < 3)
        return false;
    return !p.is_long || (r.group >> 3) <= 64 * p.units;
}

hipError_t launch_fast(const Request &r, const DeviceInfo &dev)
{
    switch (r.op) {
    case kRotateQuant:
        return r.group == r.n ? fast::launch_rq(r, dev) : fast::launch_rq_grouped(r, dev);
    case kRotate: return fast::launch_rot(r, dev);
    case kDequantInv:
        return r.group == r.n ? fast::launch_inv(r, dev) : fast::launch_inv_grouped(r, dev);
    }
    return hipErrorInvalidValue;
}

}  // namespace hq
