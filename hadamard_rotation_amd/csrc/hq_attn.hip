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
// Kernel 1 (attn_part_kernel): one wave per (kv head, token range).  The
// wave's G query rows (rotated and scaled by 1/sqrt(n) once per workgroup in
// LDS) are the B operand of 16x16x32 f16 products: each row is scaled by a
// power of two that puts its largest entry in [512, 1024) and split into hi
// and lo f16 halves, and the two products accumulate into the same column, so
// the scores keep fp32 accuracy; the 4-bit key
// codes of 16 tokens are the A operand, exact in f16.  Scores, an online
// softmax (running maximum and sum per head) and the weighted sum of the
// value codes follow; the value codes are summed on the VALU with lanes
// owning 8 dimensions, the weights passing through LDS.  Each wave writes its
// partial (maximum, sum, 128 accumulators per head) to the workspace.
// Kernel 2 (attn_merge_kernel): per query head, merges the partials with the
// usual rescaling and rotates the result back.
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;
constexpr int kPartStride = kHeadDim + 2;  // floats per (head, part): o[128], max, sum
constexpr int kWaves = 4;                  // waves per workgroup of kernel 1

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
    int nparts;         // partials per query head (= waves per kv head)
    int log_b;
    float rb;           // 1 / sqrt(b)
    float qscale;       // 1 / (sqrt(b) * sqrt(n)): rotation and softmax scale
};

__device__ __forceinline__ float load_scale(const void *p, int f16, int64_t i)
{
    return f16 ? f16_to_f32(((const uint16_t *)p)[i]) : ((const float *)p)[i];
}

__device__ __forceinline__ float load_q(const void *p, int dtype, int64_t i)
{
    if (dtype == kF32)
        return ((const float *)p)[i];
    if (dtype == kBF16)
        return bf16_to_f32(((const uint16_t *)p)[i]);
    return f16_to_f32(((const uint16_t *)p)[i]);
}

// Fast Walsh-Hadamard transform of `rows` rows of 128 floats in LDS, in
// blocks of 2^log_b (natural order), by the threads of the workgroup.
__device__ void fwht_rows(float *L, int rows, int log_b)
{
    for (int lh = 0; lh < log_b; ++lh) {
        __syncthreads();
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
    __syncthreads();
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

// G: query heads per kv head (1, 2, 4 or 8)
template <int G>
__global__ __launch_bounds__(64 * kWaves) void attn_part_kernel(AttnArgs a)
{
    __shared__ float qrot[G * kHeadDim];
    __shared__ float qpow[G];              // power of two applied to each query row
    __shared__ float wbuf[kWaves][16][G];  // per wave: weight of (token, head) for one block
    __shared__ float abuf[kWaves][G];      // per wave: rescale factor of each head

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15;
    const int rg = lane >> 4;  // row group: tokens 4*rg .. 4*rg+3 of a block
    const int kh = blockIdx.y;
    const int part = blockIdx.x * kWaves + wave;

    // ---- the G query rows of this kv head, rotated and scaled, in LDS
    for (int i = threadIdx.x; i < G * kHeadDim; i += blockDim.x) {
        const int g = i / kHeadDim, d = i % kHeadDim;
        const float v = load_q(a.q, a.q_dtype, (int64_t)(kh * G + g) * kHeadDim + d);
        qrot[i] = a.s[d] < 0 ? -v : v;
    }
    fwht_rows(qrot, G, a.log_b);
    if (threadIdx.x < G) {
        float mx = 0.0f;
        for (int d = 0; d < kHeadDim; ++d)
            mx = fmaxf(mx, fabsf(qrot[threadIdx.x * kHeadDim + d] * a.qscale));
        int e = 0;
        (void)frexpf(mx, &e);  // mx = f * 2^e, f in [0.5, 1)
        qpow[threadIdx.x] = mx > 0.0f ? ldexpf(1.0f, 10 - e) : 1.0f;
    }
    __syncthreads();

    // ---- B operands: column n < G holds query row n (hi halves in bqh, lo
    // halves in bql), other columns zero.  For chunk c lane l holds
    // k = 8*(l >> 4) + j, dimension 32*(l >> 4) + 8c + j (the same
    // permutation the key codes use).
    u32x4 bqh[4], bql[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t wh = 0, wl = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int d = 32 * rg + 8 * c + 2 * p + e;
                _Float16 hi = (_Float16)0.0f, lo = (_Float16)0.0f;
                if (l16 < G) {
                    const float x = qrot[l16 * kHeadDim + d] * a.qscale * qpow[l16];
                    hi = (_Float16)x;
                    lo = (_Float16)(x - (float)hi);
                }
                wh |= (uint32_t)__builtin_bit_cast(uint16_t, hi) << (16 * e);
                wl |= (uint32_t)__builtin_bit_cast(uint16_t, lo) << (16 * e);
            }
            bqh[c][p] = wh;
            bql[c][p] = wl;
        }
    }
    const float unscale = l16 < G ? 1.0f / qpow[l16] : 1.0f;  // exact: a power of two

    // ---- token range of this wave
    const int64_t b0 = a.blocks * part / a.nparts;
    const int64_t b1 = a.blocks * (part + 1) / a.nparts;
    const int64_t last_row = (a.tokens - 1) * a.kv_heads + kh;

    float m_run = -INFINITY, l_run = 0.0f;  // score lanes (l16 < G): head l16
    float acc[G][8];                        // value lanes: dims 8*l16 .. +7
    float wsum[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        wsum[g] = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[g][j] = 0.0f;
    }

    // raw data of one 16-token block
    struct Blk {
        u32x4 k;         // key codes: token l16, dimensions 32*rg .. +31
        uint32_t v[4];   // value codes: token 4*step + rg, dimensions 8*l16 .. +7
        float ks[4];     // key scales of tokens 4*rg + i
        float vs[4];     // value scales of the same tokens
    };
    auto load_blk = [&](int64_t blk, Blk &r) {
        const int64_t t0 = blk * 16;
        int64_t row = (t0 + l16) * a.kv_heads + kh;
        row = row < last_row ? row : last_row;  // rows past the end: read a valid one
        r.k = __builtin_nontemporal_load((const u32x4 *)(a.k_codes + row * (kHeadDim / 2)) + rg);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            int64_t vr = (t0 + 4 * st + rg) * a.kv_heads + kh;
            vr = vr < last_row ? vr : last_row;
            r.v[st] = __builtin_nontemporal_load((const uint32_t *)(a.v_codes + vr * (kHeadDim / 2)) + l16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int64_t sr = (t0 + 4 * rg + i) * a.kv_heads + kh;
            sr = sr < last_row ? sr : last_row;
            r.ks[i] = load_scale(a.k_scales, a.scale_f16, sr);
            r.vs[i] = load_scale(a.v_scales, a.scale_f16, sr);
        }
    };

    Blk cur;
    if (b0 < b1)
        load_blk(b0, cur);
    for (int64_t blk = b0; blk < b1; ++blk) {
        Blk nxt = cur;
        if (blk + 1 < b1)
            load_blk(blk + 1, nxt);
        // -------------------------------------------------------- scores
        f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // 8 key codes (dimension 32*rg + 8c + j) -> exact f16: 0x6400 |
            // (nib ^ 8) is 1032 + q, and 1032 is subtracted in f16
            const uint32_t w = cur.k[c];
            const uint32_t w4 = w >> 4;
            u32x4 ak;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t sel = (uint32_t)p | (0x0Cu << 8) | ((uint32_t)(4 + p) << 16) | (0x0Cu << 24);
                const uint32_t x = (__builtin_amdgcn_perm(w4, w, sel) & 0x000F000Fu) ^ 0x64086408u;
                const f16x2 h = __builtin_bit_cast(f16x2, x) + (f16x2){(_Float16)-1032.0f, (_Float16)-1032.0f};
                ak[p] = __builtin_bit_cast(uint32_t, h);
            }
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ak),
                                                       __builtin_bit_cast(f16x8, bqh[c]), d, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ak),
                                                       __builtin_bit_cast(f16x8, bql[c]), d, 0, 0, 0);
        }
        // lane l16 < G: scores of head l16 for tokens 4*rg + i
        float sc[4];
        const int64_t t0 = blk * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + 4 * rg + i;
            sc[i] = t < a.tokens ? d[i] * unscale * cur.ks[i] : -INFINITY;
        }
        // ------------------------------------------------- online softmax
        float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mb = xmax16_32(mb);
        const float m_new = fmaxf(m_run, mb);
        const float alpha = __expf(m_run - m_new);
        float p[4], ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = __expf(sc[i] - m_new);
            ps += p[i];
        }
        ps = xsum16_32(ps);
        l_run = l_run * alpha + ps;
        m_run = m_new;
        if (l16 < G) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wbuf[wave][4 * rg + i][l16] = p[i] * cur.vs[i];
            if (rg == 0)
                abuf[wave][l16] = alpha;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        // ------------------------------------------- weighted value codes
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float al = abuf[wave][g];
            wsum[g] *= al;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[g][j] *= al;
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            // codes + 8 as bytes, converted by v_cvt_f32_ubyte*
            const uint32_t xw = cur.v[st] ^ 0x88888888u;
            const uint32_t lo = xw & 0x0F0F0F0Fu, hi = (xw >> 4) & 0x0F0F0F0Fu;
            float cv[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                cv[2 * k] = (float)((lo >> (8 * k)) & 0xFFu);
                cv[2 * k + 1] = (float)((hi >> (8 * k)) & 0xFFu);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float wt = wbuf[wave][4 * st + rg][g];
                wsum[g] += wt;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[g][j] = __builtin_fmaf(wt, cv[j], acc[g][j]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
        cur = nxt;
    }

    // ---- partial of this wave: codes were summed as q + 8
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float v = __builtin_fmaf(-8.0f, wsum[g], acc[g][j]);
            v = xsum16_32(v);  // the four row groups hold different tokens
            acc[g][j] = v;
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float *dst = a.ws + ((int64_t)(kh * G + g) * a.nparts + part) * kPartStride;
        if (rg == 0) {
            *(float4 *)(dst + 8 * l16) = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
            *(float4 *)(dst + 8 * l16 + 4) = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
        }
        if (lane == g) {
            dst[kHeadDim] = m_run;
            dst[kHeadDim + 1] = l_run;
        }
    }
}

// One workgroup of 256 threads per query head: merge the partials (the
// largest maximum, the rescaled sums, the rescaled accumulators), rotate the
// result back, store.  exp(m_p - M) of every partial is kept in LDS.
constexpr int kMergeThreads = 256;

__device__ float block_reduce(float v, float *red, bool is_max)
{
    for (int off = 32; off > 0; off >>= 1) {
        const float o = __shfl_xor(v, off, 64);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < kMergeThreads / 64; ++w)
        r = is_max ? fmaxf(r, red[w]) : r + red[w];
    return r;
}

__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a)
{
    extern __shared__ float e_part[];  // [nparts]
    __shared__ float red[kMergeThreads / 64];
    __shared__ float osum[2][kHeadDim];
    __shared__ float o[kHeadDim];
    const int tid = threadIdx.x;
    const int h = blockIdx.x;
    const float *base = a.ws + (int64_t)h * a.nparts * kPartStride;
    float m = -INFINITY;
    for (int p = tid; p < a.nparts; p += kMergeThreads)
        m = fmaxf(m, base[(int64_t)p * kPartStride + kHeadDim]);
    const float M = block_reduce(m, red, true);
    float l = 0.0f;
    for (int p = tid; p < a.nparts; p += kMergeThreads) {
        const float *pp = base + (int64_t)p * kPartStride;
        const float pl = pp[kHeadDim + 1];
        // partials of empty token ranges (sum 0) carry nothing
        const float e = pl > 0.0f ? __expf(pp[kHeadDim] - M) : 0.0f;
        e_part[p] = e;
        l += e * pl;
    }
    const float L = block_reduce(l, red, false);  // also orders the e_part writes
    const int d = tid & (kHeadDim - 1), half = tid >> 7;
    float acc = 0.0f;
#pragma unroll 4
    for (int p = half; p < a.nparts; p += 2)
        acc = __builtin_fmaf(e_part[p], base[(int64_t)p * kPartStride + d], acc);
    osum[half][d] = acc;
    __syncthreads();
    if (tid < kHeadDim)
        o[tid] = (osum[0][tid] + osum[1][tid]) / L;
    fwht_rows(o, 1, a.log_b);
    if (tid < kHeadDim) {
        const float v = o[tid] * a.rb;
        a.out[(int64_t)h * kHeadDim + tid] = a.s[tid] < 0 ? -v : v;
    }
}

int parts_for(int kv_heads, int64_t tokens)
{
    // about 3072 waves in kernel 1 (12 per CU), whole workgroups, at most one
    // part per 16-token block
    const int64_t blocks = (tokens + 15) / 16;
    int64_t p = (3072 + kv_heads - 1) / kv_heads;
    p = (p + kWaves - 1) / kWaves * kWaves;
    const int64_t pmax = (blocks + kWaves - 1) / kWaves * kWaves;
    if (p > pmax)
        p = pmax;
    return (int)(p < kWaves ? kWaves : p);
}

template <int G>
hipError_t launch_g(const AttnArgs &aa, hipStream_t st)
{
    hipLaunchKernelGGL(attn_part_kernel<G>, dim3(aa.nparts / kWaves, aa.kv_heads),
                       dim3(64 * kWaves), 0, st, aa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(aa.q_heads), dim3(kMergeThreads),
                       (size_t)aa.nparts * sizeof(float), st, aa);
    return hipGetLastError();
}

}  // namespace

size_t attention_workspace(int q_heads, int kv_heads, int64_t tokens)
{
    return (size_t)q_heads * parts_for(kv_heads, tokens) * kPartStride * sizeof(float);
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
    aa.nparts = parts_for(r.kv_heads, r.tokens);
    int lb = 0;
    while ((1 << lb) < r.b)
        ++lb;
    aa.log_b = lb;
    aa.rb = (float)(1.0 / __builtin_sqrt((double)r.b));
    aa.qscale = (float)(1.0 / (__builtin_sqrt((double)r.b) * __builtin_sqrt((double)kHeadDim)));
    switch (r.q_heads / r.kv_heads) {
    case 1: return launch_g<1>(aa, r.stream);
    case 2: return launch_g<2>(aa, r.stream);
    case 4: return launch_g<4>(aa, r.stream);
    default: return launch_g<8>(aa, r.stream);
    }
}

}  // namespace hq
