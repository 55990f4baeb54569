// hq_fast_impl.h -- the register-resident kernel template of libhq.so for
// gfx950, included by the three translation units that instantiate it
// (forward quantisation, rotation only, inverse).
//
// Pages cited: [RQ] "旋转量化：大模型低比特量化中的离群值克星" section 2.1 (the
// Hadamard transform needs only additions and subtractions; rows whose width
// is not a power of two are rotated in independent b-element blocks, e.g.
// 4096 as 32 blocks of 128) and section 2.2 (per-row absmax scale, round and
// clip); [QT] "手把手教你用QuaRot实现LLM的4位量化：从原理到代码实践" section 2.1
// (sign flip, then Hadamard) and section 4.1 (the rotation belongs in the
// kernel that reads the activations, not in a separate pass).
//
// Layout.  A lane owns UNITS "units" of 8 consecutive elements of a row (one
// 16-byte load of bf16).  The lanes of one row segment hold consecutive
// units, so a wave instruction reads 1 KB of contiguous memory; unit u of
// lane l covers elements ((seg_base + u * LANES + l) * 8 + j), j = 0..7.
// Element index bits are [j: 3][lane: log2 LANES][unit: log2 UNITS], and a
// Hadamard block of b = 2^logb elements covers the low logb bits.  The fast
// Walsh-Hadamard transform is one butterfly stage per index bit:
//   j bits         between registers of one unit (bit 0 folded into the
//                  widening v_dot2 of the input pair, which also applies
//                  the sign vector)
//   unit bits      between registers of two units
//   lane bits 0..3 v_fmac_f32 with a DPP source (quad_perm, row_half_mirror,
//                  row_ror:8): exchange and butterfly in one instruction
//   lane bits 4, 5 v_permlane16_swap / v_permlane32_swap exchange the lane
//                  bit with a unit bit already finished, after which the
//                  butterfly is again between registers
// LDS holds only the per-workgroup copy of the sign vector and, for rows
// wider than one wave, the cross-wave absmax.
//
// The DPP stages compute acc_l += sigma_l * acc_partner(l): the difference
// half of every butterfly comes out negated, and the pairs follow the basis
// {1, 2, 7, 8} of the 16-lane index.  The result is still the Hadamard
// transform of the block, but lane l ends up holding the natural output
// chunk pi(l) times sign(l); the tables are in FastArgs (pi, neg) and the
// store addresses and the quantisation multiplier absorb both.
#pragma once

#include "hq_device.h"
#include "hq_internal.h"

namespace hq {
namespace fast {

constexpr int kMaxWpr = 16;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Loads of data that is read exactly once: the non-temporal hint keeps the
// streamed rows from displacing other lines in the caches.
template <class T>
__device__ __forceinline__ T stream_load(const T *p)
{
    return __builtin_nontemporal_load(p);
}

struct FastArgs {
    const void *x;
    const void *codes_in;
    const void *scales_in;
    const int8_t *s;
    void *codes;
    void *scales;
    void *y;
    int64_t rows;
    int64_t groups;       // row groups in total (see the work split)
    uint64_t pi;          // output chunk of lane l & 15 after the DPP stages
    uint32_t neg;         // bit l set: lane l holds the negated value
    int n;
    int logb;             // used when the template's LOGB is -1
    int log_lanes;        // used when the template's LOG_LANES is -1
    int wpr;              // waves per row (LONG kernels)
    int bits;             // 4 or 8
    int scale_f16;        // scales stored as fp16 (else fp32)
    int logg;             // log2 group size (group-wise kernels only; >= 3)
    int ngroups_row;      // n >> logg (group-wise kernels only)
    int gstride;          // floats of group scratch per wave (grouped forward)
    float kq;             // 1 / (sqrt(b) * qmax)
    float rb;             // 1 / sqrt(b)
};

// Orders the LDS accesses of one wave around an exchange between its lanes
// (LDS operations of a wave complete in order; this keeps the compiler
// from moving them across).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// ------------------------------------------------------------ primitives

// The DPP butterfly stages of one unit: for every stage t < NST and every
// register, v += sigma_t * v[partner lane of stage t].  One asm block per
// unit, opened by "s_nop 4": a DPP read needs two wait states after a VALU
// write of its source and five after an EXEC write.  Inside the block each
// register is read again only eight instructions after it was written.
#define HQ_DPP_ROW(C, S)                                                      \
    "v_fmac_f32_dpp %0, %0, %" S " " C " row_mask:0xf bank_mask:0xf\n\t"      \
    "v_fmac_f32_dpp %1, %1, %" S " " C " row_mask:0xf bank_mask:0xf\n\t"      \
    "v_fmac_f32_dpp %2, %2, %" S " " C " row_mask:0xf bank_mask:0xf\n\t"      \
    "v_fmac_f32_dpp %3, %3, %" S " " C " row_mask:0xf bank_mask:0xf\n\t"      \
    "v_fmac_f32_dpp %4, %4, %" S " " C " row_mask:0xf bank_mask:0xf\n\t"      \
    "v_fmac_f32_dpp %5, %5, %" S " " C " row_mask:0xf bank_mask:0xf\n\t"      \
    "v_fmac_f32_dpp %6, %6, %" S " " C " row_mask:0xf bank_mask:0xf\n\t"      \
    "v_fmac_f32_dpp %7, %7, %" S " " C " row_mask:0xf bank_mask:0xf\n\t"
#define HQ_DPP_C0 "quad_perm:[1,0,3,2]"
#define HQ_DPP_C1 "quad_perm:[2,3,0,1]"
#define HQ_DPP_C2 "row_half_mirror"
#define HQ_DPP_C3 "row_ror:8"
#define HQ_DPP_OPS                                                             \
    : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), \
      "+v"(v[6]), "+v"(v[7])                                                  \
    : "v"(s0), "v"(s1), "v"(s2), "v"(s3)

template <int NST>
__device__ __forceinline__ void dpp_stages(float (&v)[8], float s0, float s1, float s2, float s3)
{
    if constexpr (NST == 1)
        asm volatile("s_nop 4\n\t" HQ_DPP_ROW(HQ_DPP_C0, "8") HQ_DPP_OPS);
    else if constexpr (NST == 2)
        asm volatile("s_nop 4\n\t" HQ_DPP_ROW(HQ_DPP_C0, "8") HQ_DPP_ROW(HQ_DPP_C1, "9")
                     HQ_DPP_OPS);
    else if constexpr (NST == 3)
        asm volatile("s_nop 4\n\t" HQ_DPP_ROW(HQ_DPP_C0, "8") HQ_DPP_ROW(HQ_DPP_C1, "9")
                         HQ_DPP_ROW(HQ_DPP_C2, "10") HQ_DPP_OPS);
    else if constexpr (NST == 4)
        asm volatile("s_nop 4\n\t" HQ_DPP_ROW(HQ_DPP_C0, "8") HQ_DPP_ROW(HQ_DPP_C1, "9")
                         HQ_DPP_ROW(HQ_DPP_C2, "10") HQ_DPP_ROW(HQ_DPP_C3, "11") HQ_DPP_OPS);
}

// First butterfly of an input pair fused with widening and the sign flip:
// (s0*x0 + s1*x1, s0*x0 - s1*x1) from the packed pair w and the packed +-1
// pair sg; neg_hi negates the high half of sg for the difference.
template <int IN>
__device__ __forceinline__ void dot2_pair(uint32_t w, uint32_t sg, float &a, float &b)
{
    if constexpr (IN == kBF16) {
        asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(a) : "v"(w), "v"(sg));
        asm("v_dot2_f32_bf16 %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(b) : "v"(w), "v"(sg));
    } else {
        asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(a) : "v"(w), "v"(sg));
        asm("v_dot2_f32_f16 %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(b) : "v"(w), "v"(sg));
    }
}

// The first two butterfly stages of four inputs (pairs wl = (x0, x1) and
// wh = (x2, x3) with sign pairs sl, sh), widened and sign-flipped, in six
// dot products instead of four products and four add/subs: with
// B = s2x2 + s3x3 and B' = s2x2 - s3x3 (accumulator operand C, negated by
// neg_lo where needed)
//   y0 = s0x0 + s1x1 + B,  y1 = s0x0 - s1x1 + B',
//   y2 = s0x0 + s1x1 - B,  y3 = s0x0 - s1x1 - B'   (rows of H_4).
#define HQ_DOT2_QUAD(OPC)                                                                   \
    asm(OPC " %0, %1, %2, 0" : "=v"(B) : "v"(wh), "v"(sh));                                 \
    asm(OPC " %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(Bn) : "v"(wh), "v"(sh));                 \
    asm(OPC " %0, %1, %2, %3" : "=v"(y0) : "v"(wl), "v"(sl), "v"(B));                       \
    asm(OPC " %0, %1, %2, %3 neg_hi:[0,1,0]" : "=v"(y1) : "v"(wl), "v"(sl), "v"(Bn));       \
    asm(OPC " %0, %1, %2, %3 neg_lo:[0,0,1]" : "=v"(y2) : "v"(wl), "v"(sl), "v"(B));        \
    asm(OPC " %0, %1, %2, %3 neg_lo:[0,0,1] neg_hi:[0,1,0]" : "=v"(y3) : "v"(wl), "v"(sl), "v"(Bn))

template <int IN>
__device__ __forceinline__ void dot2_quad(uint32_t wl, uint32_t wh, uint32_t sl, uint32_t sh,
                                          float &y0, float &y1, float &y2, float &y3)
{
    float B, Bn;
    if constexpr (IN == kBF16) {
        HQ_DOT2_QUAD("v_dot2_f32_bf16");
    } else {
        HQ_DOT2_QUAD("v_dot2_f32_f16");
    }
}

__device__ __forceinline__ void bfly(float &a, float &b)
{
    float t = a + b;
    b = a - b;
    a = t;
}

__device__ __forceinline__ float flip(float v, uint32_t sbit)
{
    return __uint_as_float(__float_as_uint(v) ^ (sbit << 31));
}

// (a | b) ^ c in one v_bitop3_b32.  The constant sits in the middle operand,
// which makes the truth table the same whichever operand the hardware takes
// as the most significant index bit.
__device__ __forceinline__ uint32_t or_xor(uint32_t a, uint32_t b, uint32_t c)
{
    return __builtin_amdgcn_bitop3_b32(a, c, b, 0x36);
}

// Packs 8 INT4 codes: f[j] = 0x4B400008 + q_j with q_j in [-7, 7] (the +8
// offset keeps every nibble free of borrows, and byte 1 of every f is 0);
// element j lands in nibble j as 4-bit two's complement.
__device__ __forceinline__ uint32_t pack_int4(const uint32_t (&f)[8])
{
    const uint32_t t01 = (f[1] << 4) + f[0];  // byte 0 = (q1+8)<<4 | (q0+8)
    const uint32_t t23 = (f[3] << 4) + f[2];
    const uint32_t t45 = (f[5] << 4) + f[4];
    const uint32_t t67 = (f[7] << 4) + f[6];
    const uint32_t lo = __builtin_amdgcn_perm(t23, t01, 0x0c0c0400u);  // [t01.b0, t23.b0, 0, 0]
    const uint32_t hi = __builtin_amdgcn_perm(t67, t45, 0x04000c0cu);  // [0, 0, t45.b0, t67.b0]
    return or_xor(lo, hi, 0x88888888u);
}

// Packs 4 INT8 codes held as 0x4B400080 + q, q in [-127, 127].
__device__ __forceinline__ uint32_t pack_int8(uint32_t f0, uint32_t f1, uint32_t f2, uint32_t f3)
{
    const uint32_t lo = __builtin_amdgcn_perm(f1, f0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(f3, f2, 0x04000c0cu);
    return or_xor(lo, hi, 0x80808080u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v)
{
    // every source lane of these patterns exists, so bound_ctrl changes
    // nothing; it lets the compiler fuse the move into v_max_u32_dpp
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
    return v > o ? v : o;
}

// max over the 2^log_lanes aligned lanes of one row segment.  The values are
// |y| as bit patterns: for non-negative floats the integer order is the
// float order, and integer max needs no NaN canonicalisation.
__device__ __forceinline__ uint32_t segment_max(uint32_t v, int log_lanes)
{
    if (log_lanes > 0) v = dpp_max<0xB1>(v);   // quad_perm [1,0,3,2]
    if (log_lanes > 1) v = dpp_max<0x4E>(v);   // quad_perm [2,3,0,1]
    if (log_lanes > 2) v = dpp_max<0x141>(v);  // row_half_mirror
    if (log_lanes > 3) v = dpp_max<0x128>(v);  // row_ror:8
    if (log_lanes > 4) {
        // with both operands equal, the swap hands every lane the value of
        // its partner 16 lanes away in one of the two results
        auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = r[0] > r[1] ? r[0] : r[1];
    }
    if (log_lanes > 5) {
        auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = r[0] > r[1] ? r[0] : r[1];
    }
    return v;
}

// Raw input of one unit: 16 bytes of bf16/f16, 32 bytes of fp32, or 4/8
// bytes of codes plus the bits of the unit's group scale (inverse path).
template <int OP, int IN, bool GR>
struct RawUnit {
    uint32_t w[(OP != kDequantInv && IN == kF32) ? 8 : (OP == kDequantInv ? (GR ? 3 : 2) : 4)];
};

// ----------------------------------------------------------------- kernel
//
// OP         kRotateQuant, kRotate or kDequantInv
// IN         input dtype (forward) or output dtype (inverse: kF32 / kBF16)
// UNITS      8-element units per lane and row (registers)
// LOG_LANES  log2 lanes per row segment, or -1 for FastArgs::log_lanes
// LOGB       log2 b, or -1 for FastArgs::logb
// RPL        independent rows per lane per iteration (short rows)
// LONG       a row spans FastArgs::wpr waves (LOG_LANES == 6, RPL == 1);
//            units past the row end are loaded clamped and ignored
// GR         group-wise scales (FastArgs::logg) instead of one per row
template <int OP, int IN, int UNITS, int LOG_LANES, int LOGB, int RPL, bool LONG, bool GR>
__global__ __launch_bounds__(UNITS < 8 ? 1024 : (LONG ? 256 : 768))
void fast_kernel(FastArgs a)
{
    extern __shared__ __align__(16) uint32_t lds_sign[];  // sign material of one row width
    __shared__ uint32_t red[2][kMaxWpr];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int log_lanes = LOG_LANES >= 0 ? LOG_LANES : a.log_lanes;
    const int logb = LOGB >= 0 ? LOGB : a.logb;
    const int lanes = 1 << log_lanes;
    const int l = lane & (lanes - 1);  // lane within its row segment
    const int units_row = a.n >> 3;

    // ---- stage plan (compile-time when LOGB and LOG_LANES are)
    const int lane_bits = logb > 3 ? (logb - 3 < log_lanes ? logb - 3 : log_lanes) : 0;
    const int n_dpp = lane_bits < 4 ? lane_bits : 4;
    const bool swap16 = lane_bits > 4;
    const bool swap32 = lane_bits > 5;
    const int unit_bits = logb - 3 - log_lanes > 0 ? logb - 3 - log_lanes : 0;

    const int l16 = lane & 15;
    const float sig0 = ((l16 ^ (l16 >> 2)) & 1) ? -1.0f : 1.0f;
    const float sig1 = (((l16 >> 1) ^ (l16 >> 2)) & 1) ? -1.0f : 1.0f;
    const float sig2 = ((l16 >> 2) & 1) ? -1.0f : 1.0f;
    const float sig3 = ((l16 >> 3) & 1) ? -1.0f : 1.0f;
    const bool lane_neg = (a.neg >> l16) & 1;

    // row segment geometry
    const int seg = LONG ? wave : 0;
    const int seg_base = seg * UNITS * 64;
    const int rows_per_wave = LONG ? 0 : (64 >> log_lanes);
    // Work split.  Long rows: the waves of a workgroup share each row.
    // Short rows: a wave works alone on "wave groups" of
    // rows_per_wave * RPL consecutive rows, and each workgroup (one per CU,
    // holding all of that CU's waves) hands its share of the groups out
    // through an LDS counter:
    // the SIMD arbiter favours older waves, so a static split per wave
    // would leave the youngest waves with most of their rows at the end.
    __shared__ int pool_next;
    const int row_sub = LONG ? 0 : (lane >> log_lanes);
    const int rows_per_group = LONG ? 1 : rows_per_wave * RPL;
    // Workgroup b owns groups b, b + grid, b + 2*grid, ... (strided: speed
    // differences between CUs and address ranges average out).
    const int64_t pool_size = (a.groups - blockIdx.x + gridDim.x - 1) / gridDim.x;
    const int nwaves = blockDim.x >> 6;
    // the first group of every wave is fixed (no LDS round trip before the
    // first load); the counter starts after them
    const int64_t first = LONG ? 0 : wave;
    const bool has_work = first < pool_size;
    if (threadIdx.x == 0)
        pool_next = nwaves;
    auto grab = [&]() -> int64_t {
        int v = 0;
        if (lane == 0)
            v = atomicAdd(&pool_next, 1);
        return __builtin_amdgcn_readfirstlane(v);
    };

    // unit index (within the row) read by unit u, and written after the
    // DPP permutation and the permlane swaps
    auto in_unit = [&](int u) { return seg_base + u * lanes + l; };
    int pl = l;
    if (n_dpp > 0) {
        const int c = (int)((a.pi >> (4 * l16)) & 15);
        const int mask = (1 << n_dpp) - 1;
        pl = (l & ~mask) | (c & mask);
    }
    auto out_unit = [&](int u) {
        int lo = pl, uo = u;
        if (swap16) {  // lane bit 4 <-> unit bit 0
            const int lb = (lo >> 4) & 1, ub = uo & 1;
            lo = (lo & ~16) | (ub << 4);
            uo = (uo & ~1) | lb;
        }
        if (swap32) {  // lane bit 5 <-> unit bit 1
            const int lb = (lo >> 5) & 1, ub = (uo >> 1) & 1;
            lo = (lo & ~32) | (ub << 5);
            uo = (uo & ~2) | (lb << 1);
        }
        return seg_base + uo * lanes + lo;
    };

    // Rows of (pool-relative) group g: the group starts at the wave-uniform
    // row (b + g*grid)*rows_per_group, and this lane's k-th row is
    // lane_row(k) rows further.  Addresses are a wave-uniform 64-bit group
    // base plus 32-bit per-lane offsets.
    auto group_row0 = [&](int64_t g) {
        return ((int64_t)blockIdx.x + g * gridDim.x) * rows_per_group;
    };
    auto lane_row = [&](int k) { return row_sub + k * rows_per_wave; };

    // ---- loads (addresses clamped to valid memory; results of rows or
    // units past the end are never stored)
    auto load = [&](int64_t g, RawUnit<OP, IN, GR> (&raw)[RPL][UNITS]) {
        const int64_t r0 = group_row0(g);
        const int64_t left = a.rows - 1 - r0;  // rows after r0 in the tensor
        const int lim = left < rows_per_group ? (int)left : rows_per_group;
        const int64_t e0 = r0 * (int64_t)a.n;  // wave-uniform
#pragma unroll
        for (int k = 0; k < RPL; ++k) {
            int lr = lane_row(k);
            lr = lr < lim ? lr : lim;  // clamp into the tensor
#pragma unroll
            for (int u = 0; u < UNITS; ++u) {
                int un = in_unit(u);
                if (LONG)
                    un = un < units_row ? un : units_row - 1;
                const int eo = lr * a.n + un * 8;  // per-lane element offset
                if constexpr (OP == kDequantInv) {
                    if (a.bits == 4) {
                        const uint8_t *gp = (const uint8_t *)a.codes_in + (e0 >> 1);
                        raw[k][u].w[0] = stream_load((const uint32_t *)(gp + (eo >> 1)));
                        raw[k][u].w[1] = 0;
                    } else {
                        const int8_t *gp = (const int8_t *)a.codes_in + e0;
                        u32x2 t = stream_load((const u32x2 *)(gp + eo));
                        raw[k][u].w[0] = t[0];
                        raw[k][u].w[1] = t[1];
                    }
                    if constexpr (GR) {  // the scale of the unit's group
                        const int64_t gi = (r0 + lr) * a.ngroups_row + ((un * 8) >> a.logg);
                        raw[k][u].w[2] = a.scale_f16
                            ? (uint32_t)((const uint16_t *)a.scales_in)[gi]
                            : ((const uint32_t *)a.scales_in)[gi];
                    }
                } else if constexpr (IN == kF32) {
                    const float *gp = (const float *)a.x + e0;
                    const u32x4 *src = (const u32x4 *)(gp + eo);
                    u32x4 p = stream_load(src), q = stream_load(src + 1);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        raw[k][u].w[t] = p[t];
                        raw[k][u].w[4 + t] = q[t];
                    }
                } else {
                    const uint16_t *gp = (const uint16_t *)a.x + e0;
                    u32x4 p = stream_load((const u32x4 *)(gp + eo));
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        raw[k][u].w[t] = p[t];
                }
            }
        }
    };

    // ---- sign material -> LDS (row independent).  The sign vector is
    // requested before the first row group so that the table does not wait
    // behind the grid's initial burst of row loads; the LDS writes and the
    // barrier follow once the row loads are in flight.  Forward: +-1 pairs
    // in the input's 16-bit format, one word per element pair.  Inverse:
    // the raw sign bytes.  One pass of kSignChunks 16-sign chunks per
    // thread covers every row width the plans produce (n <= 1024 per wave
    // of the workgroup times kSignChunks * 16 / 16).
    constexpr int kSignChunks = 4;
    uint4 sraw[kSignChunks];
#pragma unroll
    for (int q = 0; q < kSignChunks; ++q) {
        const int c = threadIdx.x + q * blockDim.x;
        sraw[q] = c < (a.n >> 4) ? ((const uint4 *)a.s)[c] : make_uint4(0, 0, 0, 0);
    }

    // The first row group is loaded unconditionally (a wave without work
    // loads group 0 and ignores it), which keeps the count of loads in
    // flight static, so the sign table below waits only for its own loads.
    RawUnit<OP, IN, GR> cur[RPL][UNITS];
    load(has_work ? first : 0, cur);

#pragma unroll
    for (int q = 0; q < kSignChunks; ++q) {
        const int c = threadIdx.x + q * blockDim.x;
        if (c < (a.n >> 4)) {
            const uint4 w = sraw[q];
            if constexpr (OP == kDequantInv) {
                ((uint4 *)lds_sign)[c] = w;
            } else {
                const uint32_t one = (IN == kF16) ? 0x3C00u : 0x3F80u;
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
                uint32_t o[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const uint32_t two = ww[t >> 1] >> ((t & 1) * 16);
                    const uint32_t s0 = (two >> 7) & 1, s1 = (two >> 15) & 1;
                    o[t] = (one | (s0 << 15)) | ((one | (s1 << 15)) << 16);
                }
                ((uint4 *)lds_sign)[2 * c] = make_uint4(o[0], o[1], o[2], o[3]);
                ((uint4 *)lds_sign)[2 * c + 1] = make_uint4(o[4], o[5], o[6], o[7]);
            }
        }
    }
    // LDS-only release: the barrier must not wait for the row loads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    // Loads and stores share one completion counter, and with both kinds
    // in flight the compiler can only wait for all of them.  An empty asm
    // that reads and rewrites the loaded registers fixes where that wait
    // happens: the loop below never waits for the loads at its top (where
    // the previous group's stores were just issued).
    auto take_delivery = [&](RawUnit<OP, IN, GR> (&raw)[RPL][UNITS]) {
#pragma unroll
        for (int k = 0; k < RPL; ++k)
#pragma unroll
            for (int u = 0; u < UNITS; ++u)
#pragma unroll
                for (int t = 0; t < (int)(sizeof(raw[k][u].w) / 4); ++t)
                    asm volatile("" : "+v"(raw[k][u].w[t]));
    };
    take_delivery(cur);

    // ---- group-wise scales (forward).  Groups of 2^logg >= 8 elements
    // never cross a wave's row segment.  Every lane writes the maxima of its
    // 8-element chunks to this wave's scratch at their natural positions;
    // one lane per group reduces them, stores the scale and leaves
    // qmax/max in the group's first slot, which the lanes then read back.
    auto quant_groups = [&](int64_t g, float (&v)[RPL][UNITS][8]) {
        float *gm = (float *)((uint8_t *)lds_sign + (size_t)a.n * 2) + wave * a.gstride;
        const int64_t r0 = group_row0(g);
        const int64_t left = a.rows - 1 - r0;  // wave-uniform
        const int lim = left < rows_per_group ? (int)left : rows_per_group;
        const int lg = a.logg - 3;             // log2 units per group
        const int gu = 1 << lg;
#pragma unroll
        for (int k = 0; k < RPL; ++k)
#pragma unroll
            for (int u = 0; u < UNITS; ++u) {
                float mu = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; j += 2)
                    mu = fmaxf(fmaxf(mu, fabsf(v[k][u][j])), fabsf(v[k][u][j + 1]));
                const int ou = out_unit(u);
                if (!LONG || ou < units_row)
                    gm[LONG ? ou - seg_base : lane_row(k) * units_row + ou] = mu;
            }
        wave_lds_sync();
        const int used = LONG ? (units_row - seg_base < 64 * UNITS ? units_row - seg_base : 64 * UNITS)
                              : rows_per_group * units_row;
        const int ng = used >> lg;
        const int qmax = a.bits == 4 ? 7 : 127;
        for (int gi = lane; gi < ng; gi += 64) {
            float m = 0.0f;
            const float *p = gm + (gi << lg);
            if (gu >= 4) {
                for (int i = 0; i < gu; i += 4) {
                    const float4 q = *(const float4 *)(p + i);
                    m = fmaxf(fmaxf(m, q.x), fmaxf(q.y, fmaxf(q.z, q.w)));
                }
            } else {
                for (int i = 0; i < gu; ++i)
                    m = fmaxf(m, p[i]);
            }
            const RowQuant rq = row_quant(m, a.kq, qmax);
            int64_t sidx;
            bool ok;
            if (LONG) {
                sidx = r0 * a.ngroups_row + ((seg_base >> lg) + gi);
                ok = true;
            } else {
                const int lr = (gi << lg) / units_row;
                sidx = (r0 + lr) * a.ngroups_row + (gi - lr * a.ngroups_row);
                ok = lr <= lim;
            }
            if (ok) {
                if (a.scale_f16)
                    ((uint16_t *)a.scales)[sidx] = f32_to_f16(rq.scale);
                else
                    ((float *)a.scales)[sidx] = rq.scale;
            }
            // a magnified group is flagged by the sign (inv is otherwise >= 0)
            gm[gi << lg] = rq.boost != 1.0f ? -rq.inv : rq.inv;
        }
        wave_lds_sync();
        const int64_t e0 = r0 * (int64_t)a.n;  // wave-uniform
#pragma unroll
        for (int k = 0; k < RPL; ++k) {
            const int lr = lane_row(k);
            const bool row_ok = lr <= lim;
            const int ro = lr * a.n;
#pragma unroll
            for (int u = 0; u < UNITS; ++u) {
                const int ou = out_unit(u);
                if (LONG && ou >= units_row)
                    continue;
                const int idx = LONG ? ou - seg_base : lr * units_row + ou;
                float inv = gm[idx & ~(gu - 1)];
                const bool boosted = inv < 0.0f;
                inv = fabsf(inv);
                if (__builtin_amdgcn_ballot_w64(boosted) != 0) {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        v[k][u][j] *= boosted ? kBoost : 1.0f;
                }
                inv = lane_neg ? -inv : inv;
                if (!row_ok)
                    continue;
                if (a.bits == 4) {
                    uint32_t f[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)  // 1.5*2^23 + 8
                        f[j] = __float_as_uint(__builtin_fmaf(v[k][u][j], inv, 12582920.0f));
                    *(uint32_t *)((uint8_t *)a.codes + (e0 >> 1) + ((ro >> 1) + ou * 4)) =
                        pack_int4(f);
                } else {
                    uint32_t f[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)  // 1.5*2^23 + 128
                        f[j] = __float_as_uint(__builtin_fmaf(v[k][u][j], inv, 12583040.0f));
                    *(uint2 *)((int8_t *)a.codes + e0 + (ro + ou * 8)) =
                        make_uint2(pack_int8(f[0], f[1], f[2], f[3]), pack_int8(f[4], f[5], f[6], f[7]));
                }
            }
        }
        wave_lds_sync();  // the scratch is rewritten by the next row group
    };

    int parity = 0;
    int64_t g = first;
    while (g < pool_size) {
        float v[RPL][UNITS][8];
        // next group: the following one for long rows (every wave of the
        // workgroup walks the same rows), else a fresh one from the pool;
        // requested now, used at the prefetch below
        const int64_t g_next = LONG ? g + 1 : grab();
        // The lane's word offset in the sign table, passed through an empty
        // asm each row: the compiler cannot hoist the (row-independent)
        // table reads out of the loop, which would pin four registers per
        // unit, and the per-unit offsets stay immediate.
        int sofs = (seg_base + l) * 4;
        asm volatile("" : "+v"(sofs));
        int zofs = 0;  // the same for the inverse path's output-position signs
        asm volatile("" : "+v"(zofs));
        // -------------------------------------------- widen + sign + bit 0
#pragma unroll
        for (int u = 0; u < UNITS; ++u) {
            if constexpr (OP == kDequantInv) {
#pragma unroll
                for (int k = 0; k < RPL; ++k) {
                    if (a.bits == 4) {
                        uint32_t w = cur[k][u].w[0];
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            v[k][u][j] = (float)((int32_t)(w << (28 - 4 * j)) >> 28);
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            uint32_t word = cur[k][u].w[j >> 2];
                            v[k][u][j] = (float)((int32_t)(word << (24 - 8 * (j & 3))) >> 24);
                        }
                    }
                    if constexpr (GR) {
                        // group-wise scales: dequantise before the transform
                        const uint32_t sw = cur[k][u].w[2];
                        const float sc = a.scale_f16 ? f16_to_f32((uint16_t)sw) : __uint_as_float(sw);
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            v[k][u][j] *= sc;
                    }
                    if (logb > 0) {
                        bfly(v[k][u][0], v[k][u][1]);
                        bfly(v[k][u][2], v[k][u][3]);
                        bfly(v[k][u][4], v[k][u][5]);
                        bfly(v[k][u][6], v[k][u][7]);
                    }
                }
            } else {
                int sidx = sofs + u * lanes * 4;  // = in_unit(u) * 4
                if (LONG)
                    sidx = sidx < units_row * 4 ? sidx : (units_row - 1) * 4;
                const uint4 sg =
                    *(const uint4 *)__builtin_assume_aligned(&lds_sign[sidx], 16);
                const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
#pragma unroll
                for (int k = 0; k < RPL; ++k) {
                    if constexpr (IN == kF32) {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            v[k][u][j] = flip(__uint_as_float(cur[k][u].w[j]),
                                              (sw[j >> 1] >> ((j & 1) ? 31 : 15)) & 1);
                        if (logb > 0) {
                            bfly(v[k][u][0], v[k][u][1]);
                            bfly(v[k][u][2], v[k][u][3]);
                            bfly(v[k][u][4], v[k][u][5]);
                            bfly(v[k][u][6], v[k][u][7]);
                        }
                    } else if (logb > 1) {
                        dot2_quad<IN>(cur[k][u].w[0], cur[k][u].w[1], sw[0], sw[1], v[k][u][0],
                                      v[k][u][1], v[k][u][2], v[k][u][3]);
                        dot2_quad<IN>(cur[k][u].w[2], cur[k][u].w[3], sw[2], sw[3], v[k][u][4],
                                      v[k][u][5], v[k][u][6], v[k][u][7]);
                    } else if (logb > 0) {
#pragma unroll
                        for (int p = 0; p < 4; ++p)
                            dot2_pair<IN>(cur[k][u].w[p], sw[p], v[k][u][2 * p], v[k][u][2 * p + 1]);
                    } else {
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            uint32_t w = cur[k][u].w[p];
                            float lo, hi;
                            if constexpr (IN == kBF16) {
                                lo = bf16_lo(w);
                                hi = bf16_hi(w);
                            } else {
                                lo = f16_to_f32((uint16_t)(w & 0xffff));
                                hi = f16_to_f32((uint16_t)(w >> 16));
                            }
                            v[k][u][2 * p] = flip(lo, (sw[p] >> 15) & 1);
                            v[k][u][2 * p + 1] = flip(hi, (sw[p] >> 31) & 1);
                        }
                    }
                }
            }
        }

        // ------------------------------------ prefetch the next row group
        if (g_next < pool_size)  // wave-uniform
            load(g_next, cur);

        // ------------------------------------------ in-unit stages (bits 1, 2)
        // (bit 1 of 16-bit input is already folded into dot2_quad)
        constexpr bool kQuad = OP != kDequantInv && IN != kF32;
#pragma unroll
        for (int k = 0; k < RPL; ++k)
#pragma unroll
            for (int u = 0; u < UNITS; ++u) {
                if (!kQuad && logb > 1) {
                    bfly(v[k][u][0], v[k][u][2]);
                    bfly(v[k][u][1], v[k][u][3]);
                    bfly(v[k][u][4], v[k][u][6]);
                    bfly(v[k][u][5], v[k][u][7]);
                }
                if (logb > 2) {
                    bfly(v[k][u][0], v[k][u][4]);
                    bfly(v[k][u][1], v[k][u][5]);
                    bfly(v[k][u][2], v[k][u][6]);
                    bfly(v[k][u][3], v[k][u][7]);
                }
            }
        // --------------------------------------------------- unit-bit stages
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            if ((1 << t) < UNITS && t < unit_bits) {
#pragma unroll
                for (int k = 0; k < RPL; ++k)
#pragma unroll
                    for (int u = 0; u < UNITS; ++u) {
                        if ((u >> t) & 1)
                            continue;
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            bfly(v[k][u][j], v[k][u + (1 << t)][j]);
                    }
            }
        }
        // ----------------------------------------------- DPP lane stages 0..3
#pragma unroll
        for (int k = 0; k < RPL; ++k)
#pragma unroll
            for (int u = 0; u < UNITS; ++u) {
                switch (n_dpp) {
                case 1: dpp_stages<1>(v[k][u], sig0, sig1, sig2, sig3); break;
                case 2: dpp_stages<2>(v[k][u], sig0, sig1, sig2, sig3); break;
                case 3: dpp_stages<3>(v[k][u], sig0, sig1, sig2, sig3); break;
                case 4: dpp_stages<4>(v[k][u], sig0, sig1, sig2, sig3); break;
                default: break;
                }
            }
        // ---------------------------------------- lane bits 4, 5 via permlane
        if constexpr (UNITS >= 2) {
            if (swap16) {
#pragma unroll
                for (int k = 0; k < RPL; ++k)
#pragma unroll
                    for (int u = 0; u < UNITS; u += 2)
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            auto r = __builtin_amdgcn_permlane16_swap(
                                __float_as_uint(v[k][u][j]), __float_as_uint(v[k][u + 1][j]),
                                false, false);
                            v[k][u][j] = __uint_as_float(r[0]);
                            v[k][u + 1][j] = __uint_as_float(r[1]);
                            bfly(v[k][u][j], v[k][u + 1][j]);
                        }
            }
        }
        if constexpr (UNITS >= 4) {
            if (swap32) {
#pragma unroll
                for (int k = 0; k < RPL; ++k)
#pragma unroll
                    for (int u = 0; u < UNITS; ++u) {
                        if (u & 2)
                            continue;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            auto r = __builtin_amdgcn_permlane32_swap(
                                __float_as_uint(v[k][u][j]), __float_as_uint(v[k][u + 2][j]),
                                false, false);
                            v[k][u][j] = __uint_as_float(r[0]);
                            v[k][u + 2][j] = __uint_as_float(r[1]);
                            bfly(v[k][u][j], v[k][u + 2][j]);
                        }
                    }
            }
        }

        // Take delivery of the prefetched group here, before this group's
        // stores: the wait covers loads issued a group's compute ago and
        // the previous group's stores, not stores issued just before.
        take_delivery(cur);

        // ------------------------------------------------------------ outputs
        if constexpr (OP == kRotateQuant && GR) {
            quant_groups(g, v);
            g = g_next;
            continue;
        }
#pragma unroll
        for (int k = 0; k < RPL; ++k) {
            const int64_t r0 = group_row0(g);
            const int64_t left = a.rows - 1 - r0;  // wave-uniform
            const int lim = left < rows_per_group ? (int)left : rows_per_group;
            const int lr = lane_row(k);
            const bool row_ok = lr <= lim;
            const int64_t e0 = r0 * (int64_t)a.n;  // wave-uniform
            const int ro = lr * a.n;              // per-lane row offset

            if constexpr (OP == kRotate) {
                const float m = lane_neg ? -a.rb : a.rb;
                if (row_ok) {
#pragma unroll
                    for (int u = 0; u < UNITS; ++u) {
                        const int ou = out_unit(u);
                        if (LONG && ou >= units_row)
                            continue;
                        float4 *dst = (float4 *)((float *)a.y + e0 + (ro + ou * 8));
                        dst[0] = make_float4(v[k][u][0] * m, v[k][u][1] * m, v[k][u][2] * m,
                                             v[k][u][3] * m);
                        dst[1] = make_float4(v[k][u][4] * m, v[k][u][5] * m, v[k][u][6] * m,
                                             v[k][u][7] * m);
                    }
                }
            } else if constexpr (OP == kDequantInv) {
                float sc = 1.0f;  // group-wise scales were applied to the codes
                const int lc = lr < lim ? lr : lim;  // clamped into the tensor
                if constexpr (!GR) {
                    if (a.scale_f16)
                        sc = f16_to_f32(((const uint16_t *)a.scales_in + r0)[lc]);
                    else
                        sc = ((const float *)a.scales_in + r0)[lc];
                }
                float t = sc * a.rb;
                t = lane_neg ? -t : t;
                if (row_ok) {
#pragma unroll
                    for (int u = 0; u < UNITS; ++u) {
                        const int ou = out_unit(u);
                        if (LONG && ou >= units_row)
                            continue;
                        const uint2 sb = *(const uint2 *)&lds_sign[ou * 2 + zofs];
                        float o[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            uint32_t word = j < 4 ? sb.x : sb.y;
                            o[j] = flip(v[k][u][j] * t, (word >> (8 * (j & 3) + 7)) & 1);
                        }
                        if constexpr (IN == kF32) {
                            float4 *dst = (float4 *)((float *)a.y + e0 + (ro + ou * 8));
                            dst[0] = make_float4(o[0], o[1], o[2], o[3]);
                            dst[1] = make_float4(o[4], o[5], o[6], o[7]);
                        } else {
                            uint4 pk;
                            pk.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
                            pk.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
                            pk.z = (uint32_t)f32_to_bf16(o[4]) | ((uint32_t)f32_to_bf16(o[5]) << 16);
                            pk.w = (uint32_t)f32_to_bf16(o[6]) | ((uint32_t)f32_to_bf16(o[7]) << 16);
                            *(uint4 *)((uint16_t *)a.y + e0 + (ro + ou * 8)) = pk;
                        }
                    }
                }
            } else {
                // absmax of the row (units past the end of a long row
                // excluded); across lanes on the bit pattern of the
                // non-negative maximum
                float m = 0.0f;
#pragma unroll
                for (int u = 0; u < UNITS; ++u) {
                    float mu = 0.0f;
#pragma unroll
                    for (int j = 0; j < 8; j += 2)
                        mu = fmaxf(fmaxf(mu, fabsf(v[k][u][j])), fabsf(v[k][u][j + 1]));
                    // after the permlane swaps register u holds the data of
                    // output unit out_unit(u): that decides whether it lies
                    // past the end of the row
                    if (LONG)
                        mu = out_unit(u) < units_row ? mu : 0.0f;
                    m = fmaxf(m, mu);
                }
                uint32_t mb = segment_max(__float_as_uint(m), log_lanes);
                if constexpr (LONG) {
                    if (a.wpr > 1) {
                        if (lane == 0)
                            red[parity][wave] = mb;
                        // LDS-only: the barrier must not drain the prefetch
                        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
                        __builtin_amdgcn_s_barrier();
                        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
                        mb = red[parity][0];
                        for (int w2 = 1; w2 < a.wpr; ++w2)
                            mb = mb > red[parity][w2] ? mb : red[parity][w2];
                        parity ^= 1;
                    }
                }
                const int qmax = a.bits == 4 ? 7 : 127;
                RowQuant rq = row_quant(__uint_as_float(mb), a.kq, qmax);
                if (wave_any_boost(rq)) {  // rows too small for qmax / max
#pragma unroll
                    for (int u = 0; u < UNITS; ++u)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            v[k][u][j] *= rq.boost;
                }
                if (row_ok && l == 0 && seg == 0) {
                    if (a.scale_f16)
                        ((uint16_t *)a.scales + r0)[lr] = f32_to_f16(rq.scale);
                    else
                        ((float *)a.scales + r0)[lr] = rq.scale;
                }
                const float inv = lane_neg ? -rq.inv : rq.inv;
                if (a.bits == 4) {
                    if (row_ok) {
#pragma unroll
                        for (int u = 0; u < UNITS; ++u) {
                            uint32_t f[8];
#pragma unroll
                            for (int j = 0; j < 8; ++j)  // 1.5*2^23 + 8
                                f[j] = __float_as_uint(__builtin_fmaf(v[k][u][j], inv, 12582920.0f));
                            const int ou = out_unit(u);
                            if (LONG && ou >= units_row)
                                continue;
                            *(uint32_t *)((uint8_t *)a.codes + (e0 >> 1) + ((ro >> 1) + ou * 4)) =
                                pack_int4(f);
                        }
                    }
                } else {
                    if (row_ok) {
#pragma unroll
                        for (int u = 0; u < UNITS; ++u) {
                            uint32_t f[8];
#pragma unroll
                            for (int j = 0; j < 8; ++j)  // 1.5*2^23 + 128
                                f[j] = __float_as_uint(__builtin_fmaf(v[k][u][j], inv, 12583040.0f));
                            const int ou = out_unit(u);
                            if (LONG && ou >= units_row)
                                continue;
                            uint2 pk = make_uint2(pack_int8(f[0], f[1], f[2], f[3]),
                                                  pack_int8(f[4], f[5], f[6], f[7]));
                            *(uint2 *)((int8_t *)a.codes + e0 + (ro + ou * 8)) = pk;
                        }
                    }
                }
            }
        }
        g = g_next;
    }
}

// ------------------------------------------------------------- launching

struct Plan {
    int units;      // 1, 2, 4 or 8
    int log_lanes;  // 0..6
    int logb;       // log2 b
    int rpl;        // rows per lane per iteration
    int wpr;        // waves per row (> 1: long rows)
    bool is_long;
};

bool make_plan(int n, int b, Plan &p);
// Output chunk (4 bits per lane) and negation mask (1 bit per lane) of the
// 16 lanes of a DPP row after n_dpp = 0..4 DPP butterfly stages.
void dpp_tables(int n_dpp, uint64_t &pi, uint32_t &neg);
void fill_args(FastArgs &fa, const Request &r, const Plan &p);
int occupancy_blocks(const void *fn, int threads, size_t lds);

template <int OP, int IN, int UNITS, int LOG_LANES, int LOGB, int RPL, bool LONG, bool GR>
hipError_t launch_one(FastArgs fa, const Plan &p, const Request &r, const DeviceInfo &dev)
{
    // groups: rows of one workgroup iteration (LONG) or of one wave
    // iteration (short rows)
    const int rows_per_group = LONG ? 1 : (64 >> p.log_lanes) * RPL;
    fa.groups = (r.rows + rows_per_group - 1) / rows_per_group;
    const size_t lds_sign = OP == kDequantInv ? (size_t)r.n : (size_t)r.n * 2;
    // group-wise forward: per-wave scratch of one float per 8-element unit
    fa.gstride = 0;
    if (OP == kRotateQuant && GR)
        fa.gstride = LONG ? 64 * UNITS : rows_per_group * (r.n >> 3);
    const size_t per_wave = (size_t)fa.gstride * 4;
    auto fn = fast_kernel<OP, IN, UNITS, LOG_LANES, LOGB, RPL, LONG, GR>;
    int threads, grid_per_cu;
    if (LONG) {
        threads = 64 * p.wpr;
        grid_per_cu = occupancy_blocks((const void *)fn, threads, lds_sign + per_wave * p.wpr);
    } else {
        // every wave the CU can hold, in as few workgroups as the
        // 1024-thread (768 for the widest rows) limit allows
        const int max_threads = UNITS < 8 ? 1024 : 768;
        const int waves_cu = 4 * occupancy_blocks((const void *)fn, 256, lds_sign + per_wave * 4);
        grid_per_cu = (waves_cu * 64 + max_threads - 1) / max_threads;
        threads = 64 * (waves_cu / grid_per_cu);
    }
    const size_t lds = lds_sign + per_wave * (threads / 64);
    int64_t grid = (int64_t)dev.cu_count * grid_per_cu;
    if (grid > fa.groups)
        grid = fa.groups;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(threads), lds, r.stream, fa);
    return hipGetLastError();
}

// Specialised instantiations for one (OP, IN); anything else runs the
// variant with a run-time stage plan.  Group-wise scales (GR) have their own
// instantiations for the long 128-block rows, 4096-wide rows and 128-wide
// heads, and the run-time plan elsewhere.
template <int OP, int IN, bool GR>
hipError_t dispatch_op(const Request &r, const DeviceInfo &dev)
{
    Plan p;
    if (!make_plan(r.n, r.b, p))
        return hipErrorInvalidValue;
    FastArgs fa{};
    fill_args(fa, r, p);
    if (p.is_long) {
        if (p.logb == 7) {
            switch (p.units) {
            case 1: return launch_one<OP, IN, 1, 6, 7, 1, true, GR>(fa, p, r, dev);
            case 2: return launch_one<OP, IN, 2, 6, 7, 1, true, GR>(fa, p, r, dev);
            case 4: return launch_one<OP, IN, 4, 6, 7, 1, true, GR>(fa, p, r, dev);
            default: break;
            }
        }
        switch (p.units) {
        case 1: return launch_one<OP, IN, 1, 6, -1, 1, true, GR>(fa, p, r, dev);
        case 2: return launch_one<OP, IN, 2, 6, -1, 1, true, GR>(fa, p, r, dev);
        case 4: return launch_one<OP, IN, 4, 6, -1, 1, true, GR>(fa, p, r, dev);
        default: return launch_one<OP, IN, 8, 6, -1, 1, true, GR>(fa, p, r, dev);
        }
    }
    const int n = r.n;
    if (p.logb == 7 || (1 << p.logb) == n) {
        const bool full = (1 << p.logb) == n;
        if constexpr (GR) {
            if (n == 128)
                return launch_one<OP, IN, 1, 4, 7, 4, false, GR>(fa, p, r, dev);
            if (n == 4096)
                return full ? launch_one<OP, IN, 8, 6, 12, 1, false, GR>(fa, p, r, dev)
                            : launch_one<OP, IN, 8, 6, 7, 1, false, GR>(fa, p, r, dev);
        } else {
            switch (n) {
            case 16: return launch_one<OP, IN, 1, 1, 4, 4, false, GR>(fa, p, r, dev);
            case 32: return launch_one<OP, IN, 1, 2, 5, 4, false, GR>(fa, p, r, dev);
            case 64: return launch_one<OP, IN, 1, 3, 6, 4, false, GR>(fa, p, r, dev);
            case 128: return launch_one<OP, IN, 1, 4, 7, 4, false, GR>(fa, p, r, dev);
            case 256:
                return full ? launch_one<OP, IN, 2, 4, 8, 2, false, GR>(fa, p, r, dev)
                            : launch_one<OP, IN, 2, 4, 7, 2, false, GR>(fa, p, r, dev);
            case 512:
                return full ? launch_one<OP, IN, 4, 4, 9, 1, false, GR>(fa, p, r, dev)
                            : launch_one<OP, IN, 4, 4, 7, 1, false, GR>(fa, p, r, dev);
            case 1024:
                return full ? launch_one<OP, IN, 8, 4, 10, 1, false, GR>(fa, p, r, dev)
                            : launch_one<OP, IN, 8, 4, 7, 1, false, GR>(fa, p, r, dev);
            case 2048:
                return full ? launch_one<OP, IN, 8, 5, 11, 1, false, GR>(fa, p, r, dev)
                            : launch_one<OP, IN, 8, 5, 7, 1, false, GR>(fa, p, r, dev);
            case 4096:
                return full ? launch_one<OP, IN, 8, 6, 12, 1, false, GR>(fa, p, r, dev)
                            : launch_one<OP, IN, 8, 6, 7, 1, false, GR>(fa, p, r, dev);
            default: break;
            }
        }
    }
    switch (p.units) {
    case 1: return launch_one<OP, IN, 1, -1, -1, 1, false, GR>(fa, p, r, dev);
    case 2: return launch_one<OP, IN, 2, -1, -1, 1, false, GR>(fa, p, r, dev);
    case 4: return launch_one<OP, IN, 4, -1, -1, 1, false, GR>(fa, p, r, dev);
    default: return launch_one<OP, IN, 8, -1, -1, 1, false, GR>(fa, p, r, dev);
    }
}

}  // namespace fast
}  // namespace hq
