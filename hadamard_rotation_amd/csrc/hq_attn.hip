// hq_attn.hip -- decode attention over the rotated, quantised K/V cache that
// hq_rotate_quant / hq_rotate_quant_append write: the consumer of the codes.
//
// Pages cited: [QT] "手把手教你用QuaRot实现LLM的4位量化：从原理到代码实践"
// section 2.2 (K and V are rotated online, kept as 4-bit codes and
// dequantised when attention reads them); [HQA] "哈特曼旋转，轻量级QAT，流式注意力"
// section 1 (rotating Q and K with the same orthogonal matrix keeps Q.K^T);
// [MS] "QuaRot：基于旋转的离群值抑制算法说明" principle (the same transform
// rotates the result back).
//
// For one query token per head h and its kv head kh = h / G:
//   q'  = (q * s) . H_b / sqrt(b)                   (the cache's rotation)
//   c_t = q' . (code_k[t] * scale_k[t]) / sqrt(n)
//   o'  = sum_t softmax(c)_t * code_v[t] * scale_v[t]
//   o   = (o' . H_b / sqrt(b)) * s
//
// Kernel 1 (attn_part_kernel): one wave per (kv head, token range), two
// 16-token blocks per step.  The wave's G query rows (rotated and scaled by
// 1/sqrt(n) once per workgroup in LDS) are the B operand of 16x16x32 f16
// products: each row is scaled by a power of two that puts its largest entry
// in [512, 1024) and split into hi and lo f16 halves, and the two products
// accumulate into the same column, so the scores keep fp32 accuracy; the
// 4-bit key codes of 16 tokens are the A operand, exact in f16.  An online
// softmax (running maximum and sum per head) turns the scores into weights,
// which become the A operand of the value products: rows 0..G-1 hold their hi
// f16 halves, rows G..2G-1 the lo halves, the contraction runs over the 32
// tokens of the step, and the value codes (exact in f16) are the B operand,
// product ng covering dimensions 8*j + ng.  Each wave writes its partial
// (maximum, sum, 128 accumulators per head) to the workspace.
// Kernel 2 (attn_merge_kernel): per query head, merges the partials with the
// usual rescaling and rotates the result back.
#include <mutex>

#include "hq_device.h"
#include "hq_internal.h"

namespace hq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = kAttnHeadDim;
constexpr int kPartStride = kAttnPartStride;  // floats per (head, partial): o[128], max, sum, 2 unused
constexpr int kWaves = kAttnWaves;            // waves per workgroup of kernel 1

struct AttnArgs {
    const void *q;
    const int8_t *s;
    const uint8_t *k_codes;
    const void *k_scales;
    const uint8_t *v_codes;
    const void *v_scales;
    float *ws;
    float *out;
    int64_t tokens;
    int64_t blocks;     // ceil(tokens / 16)
    int q_dtype;
    int scale_f16;
    int q_heads;
    int kv_heads;
    int nparts;         // token ranges per kv head (= waves of kernel 1 per kv head)
    int nws;            // partials per query head in the workspace (= workgroups per kv head)
    int log_b;
    float rb;           // 1 / sqrt(b)
    float qscale;       // log2(e) / (sqrt(b) * sqrt(n)): rotation, softmax scale, base 2
};

// The query entries and sign bytes this thread rotates (element
// threadIdx.x + 256 r of the kv head's G rows) as raw dwords: one load each,
// whatever the query type, so that nothing waits for them before the key
// and value loads are issued; q_value() converts them afterwards.
template <int G, int R>
__device__ __forceinline__ void load_q_raw(const AttnArgs &a, int kh, uint32_t (&qw)[R], uint32_t (&sw)[R])
{
    const int esz = a.q_dtype == kF32 ? 4 : 2;
    const auto rq = rsrc(a.q, a.q_heads * kHeadDim * esz);
    const auto rs = rsrc(a.s, kHeadDim);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = threadIdx.x + 64 * kWaves * r;
        const int ic = i < G * kHeadDim ? i : G * kHeadDim - 1;
        const int e = kh * G * kHeadDim + ic;
        qw[r] = __builtin_amdgcn_raw_buffer_load_b32(rq, esz == 4 ? 4 * e : (2 * e) & ~3, 0, 0);
        sw[r] = __builtin_amdgcn_raw_buffer_load_b32(rs, (ic & (kHeadDim - 1)) & ~3, 0, 0);
    }
}

// entry r of load_q_raw as fp32, its sign applied
template <int G>
__device__ __forceinline__ float q_value(const AttnArgs &a, int kh, int r, uint32_t qw, uint32_t sw)
{
    const int i = threadIdx.x + 64 * kWaves * r;
    const int ic = i < G * kHeadDim ? i : G * kHeadDim - 1;
    const int e = kh * G * kHeadDim + ic;
    const uint16_t h = (uint16_t)((e & 1) ? qw >> 16 : qw);
    const float v = a.q_dtype == kF32 ? __uint_as_float(qw) : (a.q_dtype == kBF16 ? bf16_to_f32(h) : f16_to_f32(h));
    const int8_t sg = (int8_t)(sw >> (8 * (ic & 3)));
    return sg < 0 ? -v : v;
}

// Fast Walsh-Hadamard transform of `rows` rows of 128 floats in LDS, in
// blocks of 2^log_b (natural order), by the threads of the workgroup.
__device__ void fwht_rows(float *L, int rows, int log_b)
{
    for (int lh = 0; lh < log_b; ++lh) {
        lds_barrier();
        const int h = 1 << lh;
        for (int p = threadIdx.x; p < rows * (kHeadDim / 2); p += blockDim.x) {
            const int r = p / (kHeadDim / 2), pp = p % (kHeadDim / 2);
            const int i = ((pp >> lh) << (lh + 1)) | (pp & (h - 1));
            float *row = L + r * kHeadDim;
            const float x = row[i], y = row[i + h];
            row[i] = x + y;
            row[i + h] = x - y;
        }
    }
    lds_barrier();
}

__device__ __forceinline__ float xmax16_32(float v)
{
    auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

__device__ __forceinline__ float xsum16_32(float v)
{
    auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// x = hi + lo as f16 pairs, to about 2^-21 of |x| for |x| >= 2^-14 (and to
// 2^-25 absolute below): hi is x truncated to f16 by one conversion whose
// result both goes into the operand and forms the remainder, so the
// remainder x - hi is exact in fp32 and only its own rounding to f16 is lost.
// (Rounding hi to nearest instead lets the compiler round the same product
// twice, once through a mixed-precision multiply, and the two can differ by
// one f16 unit at a midpoint.)
__device__ __forceinline__ void split_f16x2(float x0, float x1, uint32_t &hi, uint32_t &lo)
{
    const auto h = __builtin_amdgcn_cvt_pkrtz(x0, x1);
    const f16x2 l = {(_Float16)(x0 - (float)h[0]), (_Float16)(x1 - (float)h[1])};
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}

// v(lane) + v(lane ^ 16)
__device__ __forceinline__ float xsum16(float v)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v(lane) + v(lane ^ 32)
__device__ __forceinline__ float xsum32(float v)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ks[j] = v of lane j, vs[j] = v of lane 8 + j, within each row of 16 lanes
template <int J>
__device__ __forceinline__ void bcast_row(float v, float (&ks)[8], float (&vs)[8])
{
    if constexpr (J < 8) {
        ks[J] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + J, 0xf, 0xf, false));
        vs[J] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x158 + J, 0xf, 0xf, false));
        bcast_row<J + 1>(v, ks, vs);
    }
}

constexpr float kGrowLog2 = 5.0f;  // scores are in base 2: a factor of 32

// 4-bit codes -> exact f16 pairs.  Of the 8 nibbles of a code word,
// (i, i + 4) share a 16-bit-lane pair: nibbles 0/4 and 2/6 (after >> 8) sit
// in bits 0-3 of each half, where 0x6400 | (nib ^ 8) is 1032 + q; nibbles 1/5
// and 3/7 sit in bits 4-7, where 0x6400 | ((nib ^ 8) << 4) is 1152 + 16 q.
// The offsets are subtracted in f16, exactly; the factor 16 of the odd
// nibbles is undone on the other operand or on the result.
__device__ __forceinline__ uint32_t codes_lo(uint32_t x)  // bits 0-3 of each half -> q
{
    const f16x2 h = __builtin_bit_cast(f16x2, (x & 0x000F000Fu) ^ 0x64086408u) +
                    (f16x2){(_Float16)-1032.0f, (_Float16)-1032.0f};
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint32_t codes_hi(uint32_t x)  // bits 4-7 of each half -> 16 q
{
    const f16x2 h = __builtin_bit_cast(f16x2, (x & 0x00F000F0u) ^ 0x64806480u) +
                    (f16x2){(_Float16)-1152.0f, (_Float16)-1152.0f};
    return __builtin_bit_cast(uint32_t, h);
}

// G: query heads per kv head (1, 2, 4 or 8)
template <int G>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(3))) void attn_part_kernel(AttnArgs a)
{
    __shared__ float qrot[G * kHeadDim];
    __shared__ float qpow[G];                  // power of two applied to each query row
    __shared__ float po[kWaves][G][kHeadDim];  // each wave's partial accumulators
    __shared__ float pm[kWaves][G], pl[kWaves][G];
    __shared__ u32x4 bq_lds[2][kWaves][64];    // query operands: [hi/lo][chunk][lane]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15;
    const int rg = lane >> 4;  // row group: tokens 4*rg .. 4*rg+3 of a block
    const int kh = blockIdx.y;
    const int part = blockIdx.x * kWaves + wave;

    // ---- token range of this wave
    const int64_t b0 = a.blocks * part / a.nparts;
    const int64_t b1 = a.blocks * (part + 1) / a.nparts;
    const int64_t lim = a.tokens < b1 * 16 ? a.tokens : b1 * 16;  // first token not ours

    // Raw data of two 16-token blocks.  Value element j is token
    // 4*rg + (j & 3) of block j >> 2: the tokens whose scores the lane holds,
    // and the tokens of contraction index 8*rg + j of the value products.
    // Each lane loads one scale: lane l16 = j < 8 the key scale of that token,
    // lane l16 = 8 + j its value scale; DPP broadcasts hand them out per row.
    struct Pair {
        u32x4 k[2];      // key codes: token l16 of each block, dimensions 32*rg .. +31
        uint32_t s;      // one scale, raw bits (f16 or f32)
        uint32_t v[8];   // value codes: dimensions 8*l16 .. +7
    };
    // The key and value loads are ordinary (cached) loads: a 128-byte line
    // holds the rows of two kv heads, and the workgroup of the other head
    // reads its second half at about the same time (same blockIdx.x; with
    // a grid row length that is a multiple of 8, as at long caches, the
    // round-robin placement puts it on the same XCD and its L2).
    // Loads go through buffer descriptors rebased to the step's first row
    // and cut off at the first row of a token >= lim: rows past the wave's
    // range read as 0 without touching memory.  Lane offsets (bytes from the
    // step's first row) are the same for every step.
    const int kv = a.kv_heads;
    const int ssz = a.scale_f16 ? 2 : 4;
    const int64_t lim_rows = lim * kv;
    auto span = [&](int64_t row0, int bytes_per_row) -> int {
        int64_t r = (lim_rows - row0) * bytes_per_row;
        r = r < 0 ? 0 : r;
        return (int)(r < 0x7FFFFFFF ? r : 0x7FFFFFFF);
    };
    // (the two blocks of a step have descriptors of their own, so they share
    // these offsets)
    const int ok_ = (l16 * kv + kh) * (kHeadDim / 2) + 16 * rg;
    int ov_[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        ov_[i] = ((4 * rg + i) * kv + kh) * (kHeadDim / 2) + 4 * l16;
    const int sj = l16 & 7;
    const int srow = (16 * (sj >> 2) + 4 * rg + (sj & 3)) * kv + kh;
    const int os_ = srow * ssz;
    // Loads are issued in the order a step uses them (key codes, scales,
    // value codes), and nothing combines their results here, so waits on the
    // in-order load counter cover only what a step is about to use.
    auto load_pair = [&](int64_t blk, Pair &r) {
        const int64_t row0 = blk * 16 * kv;
        const int64_t row1 = row0 + 16 * kv;
        const int cb0 = span(row0, kHeadDim / 2), cb1 = span(row1, kHeadDim / 2);
        const auto rk0 = rsrc(a.k_codes + row0 * (kHeadDim / 2), cb0);
        const auto rk1 = rsrc(a.k_codes + row1 * (kHeadDim / 2), cb1);
        const auto rv0 = rsrc(a.v_codes + row0 * (kHeadDim / 2), cb0);
        const auto rv1 = rsrc(a.v_codes + row1 * (kHeadDim / 2), cb1);
        r.k[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk0, ok_, 0, 0));
        r.k[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk1, ok_, 0, 0));
        const int sb = span(row0, ssz);
        const auto rks = rsrc((const uint8_t *)a.k_scales + row0 * ssz, sb);
        const auto rvs = rsrc((const uint8_t *)a.v_scales + row0 * ssz, sb);
        // lanes 0-7 of a row keep key scales, lanes 8-15 value scales, in
        // the same register (both are loaded: no branch around a load, which
        // would make the compiler's load-count waits wait for everything)
        const uint32_t sk = a.scale_f16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rks, os_, 0, 0)
                                        : __builtin_amdgcn_raw_buffer_load_b32(rks, os_, 0, 0);
        const uint32_t sv = a.scale_f16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rvs, os_, 0, 0)
                                        : __builtin_amdgcn_raw_buffer_load_b32(rvs, os_, 0, 0);
        r.s = l16 < 8 ? sk : sv;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.v[i] = __builtin_amdgcn_raw_buffer_load_b32(rv0, ov_[i], 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.v[4 + i] = __builtin_amdgcn_raw_buffer_load_b32(rv1, ov_[i], 0, 0);
    };

    // ---- the G query rows of this kv head, rotated and scaled, in LDS; the
    // scale includes log2(e), so scores come out in base 2 and exp2 serves.
    // Their loads are issued first and all at once; the first two steps'
    // codes follow and stay in flight while the rows are prepared.
    constexpr int kQPer = (G * kHeadDim + 64 * kWaves - 1) / (64 * kWaves);
    uint32_t qw[kQPer], sw[kQPer];
    load_q_raw<G, kQPer>(a, kh, qw, sw);
    // the first two steps' data, in flight during the set-up (an empty or
    // short range reads 0 without touching memory; no branch, see above)
    Pair pa, pb;
    load_pair(b0, pa);
    load_pair(b0 + 2, pb);
#pragma unroll
    for (int r = 0; r < kQPer; ++r) {
        const int i = threadIdx.x + 64 * kWaves * r;
        if (i < G * kHeadDim)
            qrot[i] = q_value<G>(a, kh, r, qw[r], sw[r]);
    }
    fwht_rows(qrot, G, a.log_b);
    for (int g = wave; g < G; g += kWaves) {  // row maxima, one wave per row
        float mx = fmaxf(fabsf(qrot[g * kHeadDim + lane]), fabsf(qrot[g * kHeadDim + 64 + lane]));
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        mx *= a.qscale;
        if (lane == 0) {
            int e = 0;
            (void)frexpf(mx, &e);  // mx = f * 2^e, f in [0.5, 1)
            qpow[g] = mx > 0.0f ? ldexpf(1.0f, 10 - e) : 1.0f;
        }
    }
    lds_barrier();

    // ---- B operands of the scores: column n < 2G holds query row n mod G
    // (hi halves in bqh, lo halves in bql; the copies in columns G..2G-1 give
    // the lanes that form the lo halves of the weights their own scores),
    // other columns zero.  For chunk c, lane l holds k = 8*(l >> 4) + 2p + e,
    // dimension 32*(l >> 4) + 8c + p + 4e: the order the key codes unpack in.
    // Odd p pairs with key codes carrying a factor 16, so those entries are
    // divided by 16 here.
    // Every wave of the workgroup needs the same operands: wave c builds
    // chunk c into LDS and all of them read the four chunks back.
    static_assert(kWaves == 4, "one chunk of the query operands per wave");
    const int gq = l16 & (G - 1);
    const bool qcol = l16 < 2 * G;
    {
        u32x4 h, l;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int d = 32 * rg + 8 * wave + p;
            float x0 = 0.0f, x1 = 0.0f;
            if (qcol) {
                const float sc = a.qscale * qpow[gq] * ((p & 1) ? 0.0625f : 1.0f);
                x0 = qrot[gq * kHeadDim + d] * sc;
                x1 = qrot[gq * kHeadDim + d + 4] * sc;
            }
            uint32_t wh, wl;
            split_f16x2(x0, x1, wh, wl);
            h[p] = wh;
            l[p] = wl;
        }
        bq_lds[0][wave][lane] = h;
        bq_lds[1][wave][lane] = l;
    }
    lds_barrier();
    u32x4 bqh[4], bql[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        bqh[c] = bq_lds[0][c][lane];
        bql[c] = bq_lds[1][c][lane];
    }
    const float unscale = qcol ? 1.0f / qpow[gq] : 1.0f;  // exact: a power of two

    // Running softmax state per head (score lanes l16 < 2G, the same in every
    // row group and in the two copies of a head).  The maximum only moves
    // when a step beats it by more than 5 (base 2), so exp2(s - m_run) stays
    // below 32 and the accumulators are rescaled rarely.  The weights also
    // carry the power of two 2^wexp that puts the largest value scale seen so
    // far in [512, 1024): with the bound on exp2 every weight stays below
    // 32768, inside f16.  l_run and the accumulators are kept in the same
    // units (times 2^wexp); the partial's maximum is stored as m_run - wexp,
    // which makes partials with different wexp merge correctly.
    float m_run = -INFINITY, l_run = 0.0f;
    int wexp = 0;
    bool wset = false;  // wave-uniform: a nonzero value scale has been seen
    // Weighted value sums: product ng covers dimensions 8*j + ng (column j),
    // odd ng times 16; row m < G holds the hi halves of head m's weights, row
    // G + m the lo halves.  Lane (l16, rg) holds rows 4*rg .. 4*rg+3 of
    // column l16.
    f32x4 acc[8];
#pragma unroll
    for (int ng = 0; ng < 8; ++ng)
        acc[ng] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    auto step = [&](const Pair &cur, int64_t blk) {
        // -------------------------------------------------------- scores
        f32x4 d[2];
        d[0] = d[1] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 bh = bqh[c], bl = bql[c];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const uint32_t w = cur.k[b][c];
                const uint32_t w8 = w >> 8;
                const u32x4 ak = {codes_lo(w), codes_hi(w), codes_lo(w8), codes_hi(w8)};
                d[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ak),
                                                              __builtin_bit_cast(f16x8, bh), d[b], 0, 0, 0);
                d[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ak),
                                                              __builtin_bit_cast(f16x8, bl), d[b], 0, 0, 0);
            }
        }
        const float sl = a.scale_f16 ? f16_to_f32((uint16_t)cur.s) : __uint_as_float(cur.s);
        float ks[8], vs[8];
        bcast_row<0>(sl, ks, vs);
        // lane l16 < 2G: scores of head l16 mod G for the lane's 8 tokens
        float sc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            sc[j] = d[j >> 2][j & 3] * unscale * ks[j];
        if (blk * 16 + 32 > lim) {  // the last step: tokens past the range
            const int left = (int)(lim - blk * 16) - 4 * rg;  // against the lane's token offsets
#pragma unroll
            for (int j = 0; j < 8; ++j)
                sc[j] = 16 * (j >> 2) + (j & 3) < left ? sc[j] : -INFINITY;
        }
        // ------------------------------------------------- online softmax
        float mb = sc[0], vm = vs[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) {
            mb = fmaxf(mb, sc[j]);
            vm = fmaxf(vm, vs[j]);
        }
        mb = xmax16_32(mb);
        vm = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, xmax16_32(vm))));
        const bool grow = qcol && mb > m_run + kGrowLog2;
        const bool need_e = wset ? vm * ldexpf(1.0f, wexp) >= 1024.0f : vm > 0.0f;
        if (__builtin_amdgcn_ballot_w64(grow) != 0 || need_e) {
            const float m_new = grow ? mb : m_run;
            float f = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // 0 on the first step
            m_run = m_new;
            if (need_e) {
                int e = 0;
                (void)frexpf(vm, &e);  // vm = f * 2^e, f in [0.5, 1)
                int enew = 10 - e;
                enew = enew < 90 ? enew : 90;  // keeps l_run * 2^wexp finite
                f *= ldexpf(1.0f, enew - wexp);
                wexp = enew;
                wset = true;
            }
            l_run *= f;
            float al[G];
#pragma unroll
            for (int g = 0; g < G; ++g)
                al[g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), g));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // row 4*rg + i belongs to head (4*rg + i) mod G
                float fr;
                if constexpr (G == 8)
                    fr = (rg & 1) ? al[4 + i] : al[i];
                else
                    fr = al[i % G];
#pragma unroll
                for (int ng = 0; ng < 8; ++ng)
                    acc[ng][i] *= fr;
            }
        }
        const float mw = m_run - (float)wexp;  // exp2(s - mw) = exp2(s - m_run) * 2^wexp
        float pw[8], ps = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pw[j] = __builtin_amdgcn_exp2f(sc[j] - mw);
            ps += pw[j];
        }
        ps = xsum16_32(ps);
        l_run += ps;
        // ------------------------------ A operand: weights as hi/lo f16 rows
        // (lanes l16 >= 2G feed rows that are never read)
        u32x4 aw;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t hw, lw;
            split_f16x2(pw[2 * p] * vs[2 * p], pw[2 * p + 1] * vs[2 * p + 1], hw, lw);
            aw[p] = l16 < G ? hw : lw;
        }
        // ------------------------------------------- weighted value codes
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // byte k of the codes of tokens (2p, 2p+1) -> 16-bit halves
            uint32_t x[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t sel = (uint32_t)k | (0x0Cu << 8) | ((uint32_t)(4 + k) << 16) | (0x0Cu << 24);
                x[p] = __builtin_amdgcn_perm(cur.v[2 * p + 1], cur.v[2 * p], sel);
            }
            // dimension 8*l16 + 2k (low nibbles) and 8*l16 + 2k + 1 (high, times 16)
            const u32x4 bv0 = {codes_lo(x[0]), codes_lo(x[1]), codes_lo(x[2]), codes_lo(x[3])};
            const u32x4 bv1 = {codes_hi(x[0]), codes_hi(x[1]), codes_hi(x[2]), codes_hi(x[3])};
            acc[2 * k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, aw),
                                                                __builtin_bit_cast(f16x8, bv0),
                                                                acc[2 * k], 0, 0, 0);
            acc[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, aw),
                                                                    __builtin_bit_cast(f16x8, bv1),
                                                                    acc[2 * k + 1], 0, 0, 0);
        }
    };

    // two register sets, alternating, so no step copies its data: a set is
    // refilled with the step after next as soon as its step is done (past
    // the range a load reads 0 without touching memory).  Steps run in
    // pairs with no exit between them, so the accumulators keep their
    // registers around the loop; an odd last step runs after it.
    const int64_t nsteps = (b1 - b0 + 1) / 2;
    int64_t blk = b0;
    for (int64_t i = 1; i < nsteps; i += 2) {
        step(pa, blk);
        load_pair(blk + 4, pa);
        step(pb, blk + 2);
        load_pair(blk + 6, pb);
        blk += 4;
    }
    if (nsteps & 1)
        step(pa, blk);

    // ---- partial of this wave: add the lo rows to the hi rows
    float o[4][8];  // [row i][product ng]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int ng = 0; ng < 8; ++ng) {
            float v;
            if constexpr (G == 1)
                v = acc[ng][0] + acc[ng][1];
            else if constexpr (G == 2)
                v = acc[ng][i & 1] + acc[ng][(i & 1) + 2];
            else if constexpr (G == 4)
                v = xsum16(acc[ng][i]);
            else
                v = xsum32(acc[ng][i]);
            o[i][ng] = v;
        }
    }
    // row 4*rg + i < G now holds head 4*rg + i: the wave's partials go to
    // LDS, and the workgroup merges its waves' partials (the largest maximum,
    // rescaled sums and accumulators) into one per head
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = 4 * rg + i;
        if (i < G && g < G) {
            *(float4 *)&po[wave][g][8 * l16] = make_float4(o[i][0], o[i][1], o[i][2], o[i][3]);
            *(float4 *)&po[wave][g][8 * l16 + 4] = make_float4(o[i][4], o[i][5], o[i][6], o[i][7]);
        }
    }
    if (lane < G) {
        pm[wave][lane] = m_run - (float)wexp;
        pl[wave][lane] = l_run;
    }
    lds_barrier();
    for (int t = threadIdx.x; t < G * kHeadDim; t += 64 * kWaves) {
        const int g = t / kHeadDim, dd = t % kHeadDim;
        float M = pm[0][g];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            M = fmaxf(M, pm[w][g]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            // waves with no tokens (sum 0) carry nothing
            const float e = pl[w][g] > 0.0f ? __builtin_amdgcn_exp2f(pm[w][g] - M) : 0.0f;
            L = __builtin_fmaf(e, pl[w][g], L);
            O = __builtin_fmaf(e, po[w][g][dd], O);
        }
        float *dst = a.ws + ((int64_t)(kh * G + g) * a.nws + blockIdx.x) * kPartStride;
        dst[dd] = (dd & 1) ? O * 0.0625f : O;  // odd dimensions were summed times 16
        if (dd == 0) {
            dst[kHeadDim] = M;
            dst[kHeadDim + 1] = L;
        }
    }
}

// v of lane l ^ m (m = 1, 2, ..., 32): DPP within rows of 16 lanes (lane
// bits 0-3; bit 2 from two shifts, each writing the banks of 4 lanes that
// read inside the row), permlane swaps across rows (bits 4, 5).
__device__ __forceinline__ float xor_lane(float v, int m, int lane)
{
    const int x = __float_as_int(v);
    switch (m) {
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xf, 0xf, false));  // quad_perm [1,0,3,2]
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xf, 0xf, false));  // quad_perm [2,3,0,1]
    case 4: {
        // banks 0, 2 (lane bit 2 clear) read lane + 4 (row_shl:4), banks 1, 3 lane - 4 (row_shr:4)
        const int t = __builtin_amdgcn_update_dpp(0, x, 0x104, 0xf, 0x5, false);
        return __int_as_float(__builtin_amdgcn_update_dpp(t, x, 0x114, 0xf, 0xA, false));
    }
    case 8: return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xf, 0xf, false));  // row_ror:8
    case 16: {
        const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
        return __uint_as_float((lane & 16) ? r[0] : r[1]);
    }
    default: {
        const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
        return __uint_as_float((lane & 32) ? r[0] : r[1]);
    }
    }
}

// One workgroup of 4 waves per query head.  Each wave merges every 4th
// partial online (the largest maximum so far, the rescaled sums and
// accumulators), lane l holding dimensions 2l and 2l + 1; the partials'
// loads go out 24 at a time.  The four waves meet once in LDS, and wave
// 0 divides by the sum, rotates back with butterflies between lanes and
// applies the signs.
constexpr int kMergeWaves = 4;
constexpr int kMergeBatch = 24;  // partials per wave whose loads go out together (96 per head: one round)

__global__ __launch_bounds__(64 * kMergeWaves) void attn_merge_kernel(AttnArgs a)
{
    __shared__ float wm[kMergeWaves], wl[kMergeWaves];
    __shared__ float2 wo[kMergeWaves][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int h = blockIdx.x;
    const float *base = a.ws + (int64_t)h * a.nws * kPartStride;
    // the signs of the lane's two dimensions, requested before the partials
    // so that their latency is not left for the end
    const uint32_t sgn = *(const uint16_t *)(a.s + 2 * lane);
    float M = -INFINITY, L = 0.0f;
    float2 O = make_float2(0.0f, 0.0f);
    for (int p0 = wave; p0 < a.nws; p0 += kMergeBatch * kMergeWaves) {
        float mp[kMergeBatch], lp[kMergeBatch];
        float2 op[kMergeBatch];
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            // (past the end: partial 0 is read and given no weight; no
            // branch around the loads)
            const int p = p0 + k * kMergeWaves;
            const bool ok = p < a.nws;
            const float *b = base + (int64_t)(ok ? p : 0) * kPartStride;
            const float m = b[kHeadDim], l = b[kHeadDim + 1];
            const float2 o = *(const float2 *)(b + 2 * lane);
            mp[k] = m;
            lp[k] = ok ? l : 0.0f;  // partials of empty token ranges (sum 0) carry nothing
            op[k] = o;
        }
        float cm = M;
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k)
            cm = lp[k] > 0.0f ? fmaxf(cm, mp[k]) : cm;
        const float f = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - cm);  // cm >= M
        L *= f;
        O.x *= f;
        O.y *= f;
        M = cm;
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            const float e = lp[k] > 0.0f ? __builtin_amdgcn_exp2f(mp[k] - M) : 0.0f;
            L = __builtin_fmaf(e, lp[k], L);
            O.x = __builtin_fmaf(e, op[k].x, O.x);
            O.y = __builtin_fmaf(e, op[k].y, O.y);
        }
    }
    if (lane == 0) {
        wm[wave] = M;
        wl[wave] = L;
    }
    wo[wave][lane] = O;
    lds_barrier();
    if (wave != 0)
        return;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w)
        Mt = wl[w] > 0.0f ? fmaxf(Mt, wm[w]) : Mt;
    float Lt = 0.0f, x0 = 0.0f, x1 = 0.0f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) {
        const float e = wl[w] > 0.0f ? __builtin_amdgcn_exp2f(wm[w] - Mt) : 0.0f;
        Lt = __builtin_fmaf(e, wl[w], Lt);
        x0 = __builtin_fmaf(e, wo[w][lane].x, x0);
        x1 = __builtin_fmaf(e, wo[w][lane].y, x1);
    }
    x0 /= Lt;
    x1 /= Lt;
    // inverse rotation in blocks of 2^log_b: dimension bit 0 in the lane,
    // bits 1..log_b-1 across lanes (lane bits 0..)
    if (a.log_b > 0) {
        const float t0 = x0 + x1, t1 = x0 - x1;
        x0 = t0;
        x1 = t1;
    }
    // (the partner lane l ^ m by DPP moves and permlane swaps, which stay in
    // the vector unit, instead of permutes through the LDS crossbar)
#pragma unroll
    for (int k = 1; k < 7; ++k) {
        if (k >= a.log_b)  // wave-uniform
            break;
        const int m = 1 << (k - 1);
        const float p0 = xor_lane(x0, m, lane), p1 = xor_lane(x1, m, lane);
        const float sg = (lane & m) ? -1.0f : 1.0f;
        x0 = __builtin_fmaf(x0, sg, p0);  // upper lane: partner - own
        x1 = __builtin_fmaf(x1, sg, p1);
    }
    const float v0 = x0 * a.rb, v1 = x1 * a.rb;
    *(float2 *)&a.out[(int64_t)h * kHeadDim + 2 * lane] =
        make_float2((sgn & 0x80u) ? -v0 : v0, (sgn & 0x8000u) ? -v1 : v1);
}

template <int G>
hipError_t launch_g(const AttnArgs &aa, hipStream_t st)
{
    hipLaunchKernelGGL(attn_part_kernel<G>, dim3(aa.nparts / kWaves, aa.kv_heads),
                       dim3(64 * kWaves), 0, st, aa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(aa.q_heads), dim3(64 * kMergeWaves), 0, st, aa);
    return hipGetLastError();
}

// The workspace of hq_decode_attention_noalloc (callers that cannot
// allocate): a file-scope device array, one copy per GPU, alive until the
// process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: kernels only ever get the address hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) unsigned char scratch[kAttnStaticWorkspaceBytes];

constexpr int kMaxScratchDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    hipError_t err = hipSuccess;
    void *ptr = nullptr;
};
ScratchSlot g_scratch[kMaxScratchDevices];

}  // namespace

hipError_t attention_static_workspace(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    ScratchSlot &slot = g_scratch[dev];
    // once per device, with that device current
    std::call_once(slot.once, [&]() {
        slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
    });
    if (slot.err != hipSuccess)
        return slot.err;
    *ptr = slot.ptr;
    return hipSuccess;
}

hipError_t launch_attention(const AttnRequest &r)
{
    AttnArgs aa{};
    aa.q = r.q;
    aa.s = r.s;
    aa.k_codes = (const uint8_t *)r.k_codes;
    aa.k_scales = r.k_scales;
    aa.v_codes = (const uint8_t *)r.v_codes;
    aa.v_scales = r.v_scales;
    aa.ws = (float *)r.workspace;
    aa.out = r.out;
    aa.tokens = r.tokens;
    aa.blocks = (r.tokens + 15) / 16;
    aa.q_dtype = r.q_dtype;
    aa.scale_f16 = r.scale_dtype == kF16;
    aa.q_heads = r.q_heads;
    aa.kv_heads = r.kv_heads;
    aa.nparts = attention_parts(r.kv_heads, r.tokens);
    aa.nws = aa.nparts / kWaves;
    int lb = 0;
    while ((1 << lb) < r.b)
        ++lb;
    aa.log_b = lb;
    aa.rb = (float)(1.0 / __builtin_sqrt((double)r.b));
    aa.qscale = (float)(1.4426950408889634 / (__builtin_sqrt((double)r.b) * __builtin_sqrt((double)kHeadDim)));
    switch (r.q_heads / r.kv_heads) {
    case 1: return launch_g<1>(aa, r.stream);
    case 2: return launch_g<2>(aa, r.stream);
    case 4: return launch_g<4>(aa, r.stream);
    default: return launch_g<8>(aa, r.stream);
    }
}

}  // namespace hq
