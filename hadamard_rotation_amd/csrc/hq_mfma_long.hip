// hq_mfma_long.hip -- matrix-core kernel for rotation + quantisation of
// long rows in 128-element blocks with one scale per row or one per block
// (group = 128): rows wider than
// the per-row tile plans (e.g. the FFN width 11008 = 86 blocks of 128,
// which is not a whole number of 512-element tiles), 16-bit input.
//
// Pages cited: [RQ] "旋转量化：大模型低比特量化中的离群值克星" section 2.1
// (a width that is not a power of two is rotated in independent 128-element
// blocks; H_128 as a Kronecker product, so its first five index bits can be
// one dense 32-point product), section 2.2 (per-token absmax scale over
// the whole row, round and clip) and section 6.2 (group size 128); [QT] "手把手教你用QuaRot实现LLM的4位量化：从原理到
// 代码实践" section 2.1 (signs, then Hadamard).
//
// One workgroup per row.  The row is cut into 512-element tiles (the last
// one may hold only 128, 256 or 384 elements); wave w takes tiles
// w*T .. w*T+T-1.  A tile is laid out exactly as in the matrix-core kernel
// of hq_mfma_impl.h (lane l loads the 8 elements at j + 8*(l >> 4) +
// 32*(l & 15)): its four 128-blocks are the lane bits 2, 3, the 32-point
// product covers P0..P4 and two DPP butterflies lane bits 0, 1.  Every load
// and store goes through a buffer resource bounded by the row (and the sign
// vector by its n bytes), with the whole offset in the bounds-checked vector
// operand (the scalar offset is not checked), so the lanes of a partial
// tile read zeros and their stores are dropped: each lane's 8 elements lie
// in one 128-block, and a 128-block is either inside the row or outside
// it.  Zeros rotate to
// zeros, so they never raise the row maximum.  With one scale per row the
// waves' maxima meet in LDS (one barrier), then every wave quantises and
// stores its own tiles; with one per block a wave's tiles need no other wave.
#include "hq_mfma_impl.h"

namespace hq {
namespace mfma {
namespace {

struct LongArgs {
    const void *x;
    const int8_t *s;
    void *codes;
    void *scales;
    int n;          // row width, a multiple of 128
    int bits;
    int scale_f16;
    uint64_t pi;    // output chunk of lane l & 15 after the two DPP stages
    uint32_t neg;   // bit l set: lane l holds the negated value
    float kq;       // 1 / (sqrt(128) * qmax)
};

// W waves per workgroup, T tiles per wave (W * T * 512 >= n).  GRP: one
// scale per 128-block (group = b = 128) instead of one per row: a block is
// 16 lanes of a tile (lane bits 2, 3 select it), so its maximum needs no
// other wave, and scales go to [rows, n / 128].
template <int IN, int W, int T, bool GRP = false>
__global__ __launch_bounds__(64 * W) void mfma_long_kernel(LongArgs a)
{
    constexpr int D = 2;  // DPP stages of a 128-point block: lane bits 0, 1
    __shared__ uint32_t red[W];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15;
    const int lane_off = 8 * (lane >> 4) + 32 * l16;  // element offset in a tile
    const int64_t row = blockIdx.x;
    const int t0 = wave * T;                           // the wave's first tile

    // ---- requests first: the sign bytes of the lane's 8 elements of each
    // tile (cache hits), then the row's tiles
    const auto rs_s = rsrc(a.s, a.n);
    u32x2 sb[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        sb[t] = __builtin_amdgcn_raw_buffer_load_b64(rs_s, lane_off + (t0 + t) * 512, 0, 0);
    const auto rs_x = rsrc((const uint16_t *)a.x + row * a.n, 2 * a.n);
    u32x4 cur[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        cur[t] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, 2 * lane_off + (t0 + t) * 1024, 0,
                                                       kNonTemporal);
    // every row load is issued before anything waits for the sign loads
    __builtin_amdgcn_sched_barrier(0);

    // ---- the two +-1 slices of H_32 (A operands), the DPP sign functionals
    // and the output permutation, as in the matrix-core kernel
    u32x4 amat[2];
    {
        const uint32_t one = IN == kF16 ? 0x3C00u : 0x3F80u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = (l16 & 3) | (h << 2) | ((l16 >> 2) << 3);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                uint32_t w = 0;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int k = 8 * (lane >> 4) + 2 * c + e;
                    w |= (one | ((uint32_t)(__builtin_popcount(q & k) & 1) << 15)) << (16 * e);
                }
                amat[h][c] = w;
            }
        }
    }
    const float sig0 = ((l16 ^ (l16 >> 2)) & 1) ? -1.0f : 1.0f;
    const float sig1 = (((l16 >> 1) ^ (l16 >> 2)) & 1) ? -1.0f : 1.0f;
    const bool lane_neg = (a.neg >> l16) & 1;
    const int c_pi = (int)((a.pi >> (4 * l16)) & 15);
    const int pl = (l16 & ~3) | (c_pi & 3);
    const int out_off = 8 * (lane >> 4) + 32 * pl;  // element offset of the lane's 8 outputs

    // ---- signs (XOR of the 16-bit sign bits) and the 32-point products
    float v[T][8];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        u32x4 b;
#pragma unroll
        for (int c = 0; c < 4; ++c)  // sign bits of bytes 2c, 2c+1 to bits 15, 31
            b[c] = cur[t][c] ^ (__builtin_amdgcn_perm(0u, sb[t][c >> 1], (c & 1) ? 0x030c020cu
                                                                                  : 0x010c000cu) &
                                0x80008000u);
        const f32x4 d0 = hmma<IN>(amat[0], b);
        const f32x4 d1 = hmma<IN>(amat[1], b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[t][i] = d0[i];
            v[t][4 + i] = d1[i];
        }
    }
    // ---- DPP stages.  The DPP blocks are inline asm, which the compiler does
    // not pad against the matrix unit's write latency: every product result
    // passes through an empty asm first (in program order), then 20 wait
    // states cover the longest MFMA-write -> VALU hazard.
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            asm volatile("" : "+v"(v[t][j]));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::);
#pragma unroll
    for (int t = 0; t < T; ++t)
        fast::dpp_stages<D>(v[t], sig0, sig1, 0.0f, 0.0f);

    const int qmax = a.bits == 4 ? 7 : 127;
    float inv[T];  // the lane's multiplier of each tile, sign included
    if constexpr (GRP) {
        // ---- one scale per 128-block, transposed: permlane16_swap of the
        // lane maxima of tiles (0, 1) and (2, 3) reduces lane bit 4 and
        // leaves rows [0, 1, 0, 1] and [2, 3, 2, 3]; permlane32_swap of the
        // two reduces lane bit 5 and leaves tile rho in 16-lane row rho.  Two
        // DPP steps over lane bits 0, 1 finish the blocks (lane bits 2, 3),
        // the reciprocal and the one scale store run once per wave, and the
        // same swaps in reverse hand every lane its block's multiplier.
        static_assert(T == 4, "the transposed reduction takes four tiles");
        uint32_t mt[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float m = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j += 2)
                m = fmaxf(fmaxf(m, fabsf(v[t][j])), fabsf(v[t][j + 1]));
            mt[t] = __float_as_uint(m);
        }
        uint32_t x[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const auto r = __builtin_amdgcn_permlane16_swap(mt[2 * p], mt[2 * p + 1], false, false);
            x[p] = r[0] > r[1] ? r[0] : r[1];
        }
        const auto r32 = __builtin_amdgcn_permlane32_swap(x[0], x[1], false, false);
        const uint32_t z = group_lane_max<D>(r32[0] > r32[1] ? r32[0] : r32[1], 7);
        const RowQuant rq = row_quant(__uint_as_float(z), a.kq, qmax);
        // lanes 4k of row rho store block 4 * (t0 + rho) + k; blocks past
        // the row end fall outside the row's scales and are dropped
        const int ss = a.scale_f16 ? 2 : 4;
        const int nb = a.n >> 7;
        const auto rs_sc = rsrc((uint8_t *)a.scales + row * nb * ss, nb * ss);
        const int so = (l16 & 3) == 0 ? (4 * (t0 + (lane >> 4)) + (l16 >> 2)) * ss : 0x7FFFFF00;
        if (a.scale_f16)
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_f16(rq.scale), rs_sc, so, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(rq.scale), rs_sc, so, 0, 0);
        auto untranspose = [](float zv, float (&out)[T]) {
            const uint32_t zi = __float_as_uint(zv);
            const auto w = __builtin_amdgcn_permlane32_swap(zi, zi, false, false);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const auto u = __builtin_amdgcn_permlane16_swap(w[h], w[h], false, false);
                out[2 * h] = __uint_as_float(u[0]);
                out[2 * h + 1] = __uint_as_float(u[1]);
            }
        };
        untranspose(lane_neg ? -rq.inv : rq.inv, inv);
        if (wave_any_boost(rq)) {  // blocks too small for qmax / max
            float boost[T];
            untranspose(rq.boost, boost);
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v[t][j] *= boost[t];
        }
    } else {
        // ---- row maximum: the lane's values, the wave, then the waves in LDS
        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int j = 0; j < 8; j += 2)
                m = fmaxf(fmaxf(m, fabsf(v[t][j])), fabsf(v[t][j + 1]));
        uint32_t mb = row_lane_max<4>(__float_as_uint(m));
        if (lane == 0)
            red[wave] = mb;
        lds_barrier();
#pragma unroll
        for (int w = 0; w < W; ++w)
            mb = mb > red[w] ? mb : red[w];
        const RowQuant rq = row_quant(__uint_as_float(mb), a.kq, qmax);
        if (wave_any_boost(rq)) {  // a row too small for qmax / max
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v[t][j] *= rq.boost;
        }
        if (wave == 0 && lane == 0) {
            if (a.scale_f16)
                ((uint16_t *)a.scales)[row] = f32_to_f16(rq.scale);
            else
                ((float *)a.scales)[row] = rq.scale;
        }
#pragma unroll
        for (int t = 0; t < T; ++t)
            inv[t] = lane_neg ? -rq.inv : rq.inv;
    }

    // ---- codes: 8 per lane and tile, stores past the row dropped;
    // non-temporal (16384 x 11008: 77.9 -> 72.7 us)
    if (a.bits == 4) {
        const auto rs_c = rsrc((uint8_t *)a.codes + row * (a.n >> 1), a.n >> 1);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            uint32_t f[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)  // 1.5*2^23 + 8
                f[j] = __float_as_uint(__builtin_fmaf(v[t][j], inv[t], 12582920.0f));
            __builtin_amdgcn_raw_buffer_store_b32(fast::pack_int4(f), rs_c,
                                                  (out_off >> 1) + (t0 + t) * 256, 0, kNonTemporal);
        }
    } else {
        const auto rs_c = rsrc((int8_t *)a.codes + row * a.n, a.n);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            uint32_t f[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)  // 1.5*2^23 + 128
                f[j] = __float_as_uint(__builtin_fmaf(v[t][j], inv[t], 12583040.0f));
            const u32x2 pk = {fast::pack_int8(f[0], f[1], f[2], f[3]),
                              fast::pack_int8(f[4], f[5], f[6], f[7])};
            __builtin_amdgcn_raw_buffer_store_b64(pk, rs_c, out_off + (t0 + t) * 512, 0, kNonTemporal);
        }
    }
}

template <int IN, int W, int T, bool GRP>
hipError_t launch_long_wt(const Request &r)
{
    LongArgs la;
    la.x = r.x;
    la.s = r.s;
    la.codes = r.codes;
    la.scales = r.scales;
    la.n = r.n;
    la.bits = r.bits;
    la.scale_f16 = r.scale_dtype == kF16;
    fast::dpp_tables(2, la.pi, la.neg);
    const int qmax = r.bits == 8 ? 127 : 7;
    la.kq = (float)(1.0 / (__builtin_sqrt(128.0) * qmax));
    hipLaunchKernelGGL((mfma_long_kernel<IN, W, T, GRP>), dim3((unsigned)r.rows), dim3(64 * W), 0,
                       r.stream, la);
    return hipGetLastError();
}

template <int IN, bool GRP>
hipError_t launch_long_in(const Request &r)
{
    // four tiles per wave, as many waves as the row needs
    switch ((r.n + 2047) / 2048) {
    case 1: return launch_long_wt<IN, 1, 4, GRP>(r);
    case 2: return launch_long_wt<IN, 2, 4, GRP>(r);
    case 3: return launch_long_wt<IN, 3, 4, GRP>(r);
    case 4: return launch_long_wt<IN, 4, 4, GRP>(r);
    case 5: return launch_long_wt<IN, 5, 4, GRP>(r);
    case 6: return launch_long_wt<IN, 6, 4, GRP>(r);
    case 7: return launch_long_wt<IN, 7, 4, GRP>(r);
    default: return launch_long_wt<IN, 8, 4, GRP>(r);
    }
}

}  // namespace

// Rows of several 128-blocks with one scale per row, or one per block, that
// the per-row tile plans do not take (wider than 4096, or not a power of
// two), 16-bit input, at most 32 tiles (16384 elements) per row.
bool long_fwd_ok(const Request &r)
{
    if (r.op != kRotateQuant || r.dst_rows || r.b != 128 || r.n % 128 != 0 || r.n <= 128 ||
        (r.group != r.n && r.group != 128))
        return false;
    if (r.x_dtype != kBF16 && r.x_dtype != kF16)
        return false;
    const bool pow2 = (r.n & (r.n - 1)) == 0;
    if (pow2 && r.n <= 4096)
        return false;
    return r.n <= 16384 && r.rows < ((int64_t)1 << 31);
}

hipError_t launch_rq_long(const Request &r, const DeviceInfo &)
{
    if (r.group == 128)
        return r.x_dtype == kBF16 ? launch_long_in<kBF16, true>(r) : launch_long_in<kF16, true>(r);
    return r.x_dtype == kBF16 ? launch_long_in<kBF16, false>(r) : launch_long_in<kF16, false>(r);
}

}  // namespace mfma
}  // namespace hq
