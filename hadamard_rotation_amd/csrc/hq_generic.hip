// hq_generic.hip -- generic path of libhq.so: one workgroup per row, the row
// staged in LDS as fp32, the fast Walsh-Hadamard transform done stage by
// stage in LDS.  It serves every supported (n, b) that the register-resident
// kernels do not cover; it is simple rather than fast.
//
// Pages cited: [RQ] "旋转量化：大模型低比特量化中的离群值克星" section 2.1 (the
// transform needs only additions and subtractions; blockwise rotation of
// independent b-element blocks) and section 2.2 (absmax quantisation);
// [QT] "手把手教你用QuaRot实现LLM的4位量化：从原理到代码实践" section 2.1 (sign
// flip before the Hadamard matrix).
//
// Butterfly order: pairs (i, i+h) for h = 1, 2, 4, ..., b/2 with
// (a, c) -> (a+c, a-c).  This is the Sylvester factorisation
// H_b = H_2 (x) H_2 (x) ... (x) H_2, so the result comes out in natural order.
//
// Widths that are not a power of two rotate by H_n = H_k (x) H_m2 ([RQ] 2.1:
// larger Hadamard matrices as Kronecker products), H_k from Paley's first
// construction over GF(k - 1): the butterflies run on each run of m2
// elements, then a dense k-point stage mixes the runs (element i * m2 + j of
// the row is entry (i, j)).  The workgroup builds H_k as a +-1 bit matrix in
// LDS once: Q[a][b] = chi(a - b), chi the quadratic character of GF(q), from
// a table of the squares of GF(q) it computes itself.
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {
namespace {

constexpr int kThreads = 256;
constexpr int kStaticLds = 256;  // upper bound of the kernel's static LDS

struct GenericArgs {
    const void *x;
    const void *codes_in;
    const void *scales_in;
    const int8_t *s;
    void *codes;
    void *scales;
    void *y;
    int64_t rows;
    int n;
    int log_b;
    int group;  // elements per scale (n: one scale per row)
    const int64_t *dst_rows;  // output row of each input row, or null
    int64_t cache_rows;
    float kq;   // 1 / (sqrt(b) * qmax)
    float rb;   // 1 / sqrt(b)
    // b == n not a power of two: H_pk (x) H_(n/pk) over GF(pp^pe) (see
    // PaleySpec); pk == 1 otherwise
    int pk, pm2, pp, pe, pmod0, pmod1, pmod2;
    int pwords;  // 32-bit words per row of the bit matrix: ceil(pk / 32)
    int pjb;     // columns of the dense stage per pass
};

// GF(p^e) arithmetic on element indices c0 + p c1 + p^2 c2 (e <= 3)
__device__ int gf_sub_dev(int a, int b, int p, int e)
{
    int r = 0, w = 1;
    for (int i = 0; i < e; ++i) {
        int d = a % p - b % p;
        d += d < 0 ? p : 0;
        r += d * w;
        w *= p;
        a /= p;
        b /= p;
    }
    return r;
}

__device__ int gf_mul_dev(int a, int b, const GenericArgs &g)
{
    const int p = g.pp, e = g.pe;
    if (e == 1)
        return (int)((int64_t)a * b % p);
    int ca[3] = {0, 0, 0}, cb[3] = {0, 0, 0}, pr[5] = {0, 0, 0, 0, 0};
    const int md[3] = {g.pmod0, g.pmod1, g.pmod2};
    for (int i = 0; i < e; ++i) {
        ca[i] = a % p;
        cb[i] = b % p;
        a /= p;
        b /= p;
    }
    for (int i = 0; i < e; ++i)
        for (int j = 0; j < e; ++j)
            pr[i + j] += ca[i] * cb[j];
    // x^e = -(md[e-1] x^(e-1) + ... + md[0]), highest power first
    for (int d = 2 * e - 2; d >= e; --d) {
        const int c = pr[d] % p;
        pr[d] = 0;
        for (int i = 0; i < e; ++i)
            pr[d - e + i] -= c * md[i];
    }
    int r = 0;
    for (int i = e - 1; i >= 0; --i)
        r = r * p + ((pr[i] % p) + p) % p;
    return r;
}

// Entry (r, c) of Paley's H_k: row/column 0 is the extra point
__device__ int paley_entry(int r, int c, const unsigned char *sq, const GenericArgs &g)
{
    if (r == 0)
        return 1;
    if (c == 0)
        return -1;
    if (r == c)
        return 1;  // chi(0) + 1
    return sq[gf_sub_dev(r - 1, c - 1, g.pp, g.pe)] ? 1 : -1;
}

// Builds, for every output index c of the k-point stage, the bits of the k
// coefficients it sums (bit set: -1): column c of H_k for the forward
// rotation u.H, row c for the inverse v.H^T.
__device__ void paley_setup(uint32_t *Pb, unsigned char *sq, const GenericArgs &g, bool transpose)
{
    const int k = g.pk, q = k - 1;
    for (int i = threadIdx.x; i < q; i += kThreads)
        sq[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x + 1; i < q; i += kThreads)
        sq[gf_mul_dev(i, i, g)] = 1;  // concurrent writes store the same 1
    __syncthreads();
    for (int idx = threadIdx.x; idx < k * g.pwords; idx += kThreads) {
        const int c = idx / g.pwords, w = idx % g.pwords;
        uint32_t bits = 0;
        for (int t = 0; t < 32 && 32 * w + t < k; ++t) {
            const int i = 32 * w + t;
            const int v = transpose ? paley_entry(c, i, sq, g) : paley_entry(i, c, sq, g);
            bits |= (v < 0 ? 1u : 0u) << t;
        }
        Pb[idx] = bits;
    }
    __syncthreads();
}

// L[c * m2 + j] = sum_i (+-1) L[i * m2 + j] with the signs of output c's
// bit row; pjb columns j at a time through the scratch C.
__device__ void paley_stage(float *L, float *C, const uint32_t *Pb, const GenericArgs &g)
{
    const int k = g.pk, m2 = g.pm2, jb = g.pjb;
    for (int j0 = 0; j0 < m2; j0 += jb) {
        __syncthreads();
        for (int t = threadIdx.x; t < jb * k; t += kThreads) {
            const int jj = t / k, i = t % k;
            C[t] = L[i * m2 + j0 + jj];
        }
        __syncthreads();
        for (int t = threadIdx.x; t < jb * k; t += kThreads) {
            const int jj = t / k, c = t % k;
            const float *col = C + jj * k;
            const uint32_t *bits = Pb + c * g.pwords;
            float acc = 0.0f;
            for (int w = 0; w < g.pwords; ++w) {  // one partial sum per word
                const uint32_t bw = bits[w];
                const int i0 = 32 * w, lim = k - i0 < 32 ? k - i0 : 32;
                float part = 0.0f;
                for (int t2 = 0; t2 < lim; ++t2) {
                    const float v = col[i0 + t2];
                    part += ((bw >> t2) & 1u) ? -v : v;
                }
                acc += part;
            }
            L[c * m2 + j0 + jj] = acc;
        }
    }
    __syncthreads();
}

template <int IN>
__device__ __forceinline__ float load_in(const void *x, int64_t idx)
{
    if constexpr (IN == kF32)
        return ((const float *)x)[idx];
    else if constexpr (IN == kBF16)
        return bf16_to_f32(((const uint16_t *)x)[idx]);
    else
        return f16_to_f32(((const uint16_t *)x)[idx]);
}

__device__ float block_max(float v, float *red)
{
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        red[wave] = v;
    __syncthreads();
    float m = red[0];
    for (int w = 1; w < kThreads / 64; ++w)
        m = fmaxf(m, red[w]);
    __syncthreads();
    return m;
}

__device__ void fwht_lds(float *L, int n, int log_b)
{
    for (int lh = 0; lh < log_b; ++lh) {
        __syncthreads();
        int h = 1 << lh;
        for (int p = threadIdx.x; p < (n >> 1); p += kThreads) {
            int i = ((p >> lh) << (lh + 1)) | (p & (h - 1));
            float a = L[i], c = L[i + h];
            L[i] = a + c;
            L[i + h] = a - c;
        }
    }
    __syncthreads();
}

// OP = kRotateQuant / kRotate: IN is the input dtype, OUT_SC the scale dtype
// (kRotateQuant only).  OP = kDequantInv: OUT_SC is the stored scale dtype,
// IN the output dtype (kF32 or kBF16).
template <int OP, int IN, int BITS, int SC>
__global__ __launch_bounds__(kThreads) void generic_kernel(GenericArgs a)
{
    extern __shared__ float L[];
    __shared__ float red[kThreads / 64];
    const int n = a.n;
    constexpr int qmax = (1 << (BITS - 1)) - 1;
    // dynamic LDS: the row, then (k > 1) the dense stage's scratch, the bit
    // matrix and the table of squares
    float *C = L + n;
    uint32_t *Pb = (uint32_t *)(C + a.pjb * a.pk);
    unsigned char *sq = (unsigned char *)(Pb + a.pk * a.pwords);
    if (a.pk > 1)
        paley_setup(Pb, sq, a, OP == kDequantInv);

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t base = row * (int64_t)n;
        if constexpr (OP == kDequantInv) {
            // one scale per row: applied after the (exact, integer) transform;
            // group-wise scales: applied to every code before it
            const bool grouped = a.group != n;
            const int ngroups = n / a.group;
            auto scale_at = [&](int64_t idx) -> float {
                if constexpr (SC == kF32)
                    return ((const float *)a.scales_in)[idx];
                else
                    return f16_to_f32(((const uint16_t *)a.scales_in)[idx]);
            };
            const float sc = grouped ? 1.0f : scale_at(row);
            for (int i = threadIdx.x; i < n; i += kThreads) {
                int q;
                if constexpr (BITS == 8) {
                    q = ((const int8_t *)a.codes_in)[base + i];
                } else {
                    uint8_t byte = ((const uint8_t *)a.codes_in)[(base >> 1) + (i >> 1)];
                    int nib = (i & 1) ? (byte >> 4) : (byte & 15);
                    q = nib >= 8 ? nib - 16 : nib;
                }
                L[i] = grouped ? (float)q * scale_at(row * ngroups + i / a.group)
                               : (float)q;  // exact; the FWHT of integer codes stays exact
            }
            fwht_lds(L, n, a.log_b);
            if (a.pk > 1)
                paley_stage(L, C, Pb, a);
            const float t = sc * a.rb;
            for (int i = threadIdx.x; i < n; i += kThreads) {
                float v = L[i] * t;
                v = a.s[i] < 0 ? -v : v;
                if constexpr (IN == kF32)
                    ((float *)a.y)[base + i] = v;
                else
                    ((uint16_t *)a.y)[base + i] = f32_to_bf16(v);
            }
            __syncthreads();
            continue;
        } else {
            for (int i = threadIdx.x; i < n; i += kThreads) {
                float v = load_in<IN>(a.x, base + i);
                L[i] = a.s[i] < 0 ? -v : v;
            }
            fwht_lds(L, n, a.log_b);
            if (a.pk > 1)
                paley_stage(L, C, Pb, a);
            if constexpr (OP == kRotate) {
                for (int i = threadIdx.x; i < n; i += kThreads)
                    ((float *)a.y)[base + i] = L[i] * a.rb;
                __syncthreads();
            } else if (a.group != n) {
                // group-wise scales: each wave takes whole groups; lanes
                // stride over the group's elements
                const int g = a.group;
                const int ngroups = n / g;
                const int lane = threadIdx.x & 63;
                for (int k = threadIdx.x >> 6; k < ngroups; k += kThreads / 64) {
                    const int i0 = k * g;
                    float m = 0.0f;
                    for (int i = lane; i < g; i += 64)
                        m = fmaxf(m, fabsf(L[i0 + i]));
                    for (int off = 32; off > 0; off >>= 1)
                        m = fmaxf(m, __shfl_xor(m, off, 64));
                    RowQuant rq = row_quant(m, a.kq, qmax);
                    if (lane == 0) {
                        if constexpr (SC == kF32)
                            ((float *)a.scales)[row * ngroups + k] = rq.scale;
                        else
                            ((uint16_t *)a.scales)[row * ngroups + k] = f32_to_f16(rq.scale);
                    }
                    if constexpr (BITS == 8) {
                        for (int i = lane; i < g; i += 64)
                            ((int8_t *)a.codes)[base + i0 + i] =
                                (int8_t)quant_code(L[i0 + i] * rq.boost, rq.inv, qmax);
                    } else {
                        for (int j = lane; j < (g >> 1); j += 64) {
                            int q0 = quant_code(L[i0 + 2 * j] * rq.boost, rq.inv, qmax);
                            int q1 = quant_code(L[i0 + 2 * j + 1] * rq.boost, rq.inv, qmax);
                            ((uint8_t *)a.codes)[((base + i0) >> 1) + j] =
                                (uint8_t)((q0 & 15) | ((q1 & 15) << 4));
                        }
                    }
                }
                __syncthreads();
            } else {
                float m = 0.0f;
                for (int i = threadIdx.x; i < n; i += kThreads)
                    m = fmaxf(m, fabsf(L[i]));
                m = block_max(m, red);
                RowQuant rq = row_quant(m, a.kq, qmax);
                // output row: the row itself, or its cache row (append);
                // a cache row outside the cache writes nothing
                const int64_t orow = a.dst_rows ? a.dst_rows[row] : row;
                const bool live = !a.dst_rows || (orow >= 0 && orow < a.cache_rows);
                const int64_t obase = orow * (int64_t)n;
                if (live && threadIdx.x == 0) {
                    if constexpr (SC == kF32)
                        ((float *)a.scales)[orow] = rq.scale;
                    else
                        ((uint16_t *)a.scales)[orow] = f32_to_f16(rq.scale);
                }
                if constexpr (BITS == 8) {
                    for (int i = threadIdx.x; live && i < n; i += kThreads)
                        ((int8_t *)a.codes)[obase + i] = (int8_t)quant_code(L[i] * rq.boost, rq.inv, qmax);
                } else {
                    for (int j = threadIdx.x; live && j < (n >> 1); j += kThreads) {
                        int q0 = quant_code(L[2 * j] * rq.boost, rq.inv, qmax);
                        int q1 = quant_code(L[2 * j + 1] * rq.boost, rq.inv, qmax);
                        ((uint8_t *)a.codes)[(obase >> 1) + j] =
                            (uint8_t)((q0 & 15) | ((q1 & 15) << 4));
                    }
                }
                __syncthreads();
            }
        }
    }
}

// dynamic LDS of a launch (see the kernel's layout)
size_t generic_lds(const GenericArgs &ga)
{
    size_t lds = (size_t)ga.n * sizeof(float);
    if (ga.pk > 1)
        lds += (size_t)ga.pjb * ga.pk * sizeof(float) + (size_t)ga.pk * ga.pwords * sizeof(uint32_t) +
               (size_t)((ga.pk + 3) & ~3);
    return lds;
}

template <int OP, int IN, int BITS, int SC>
hipError_t go(const GenericArgs &ga, const Request &r, const DeviceInfo &dev)
{
    // persistent workgroups when each builds a Paley matrix first
    const int64_t cap = ga.pk > 1 ? (int64_t)dev.cu_count * 2 : (1 << 20);
    int64_t grid = r.rows < cap ? r.rows : cap;
    size_t lds = generic_lds(ga);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void *)generic_kernel<OP, IN, BITS, SC>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((generic_kernel<OP, IN, BITS, SC>), dim3((unsigned)grid),
                       dim3(kThreads), lds, r.stream, ga);
    return hipGetLastError();
}

template <int OP, int IN>
hipError_t pick_bits(const GenericArgs &ga, const Request &r, const DeviceInfo &dev)
{
    if (r.bits == 4)
        return r.scale_dtype == kF32 ? go<OP, IN, 4, kF32>(ga, r, dev)
                                     : go<OP, IN, 4, kF16>(ga, r, dev);
    return r.scale_dtype == kF32 ? go<OP, IN, 8, kF32>(ga, r, dev)
                                 : go<OP, IN, 8, kF16>(ga, r, dev);
}

}  // namespace

bool generic_paley_fits(const Request &r, const DeviceInfo &dev)
{
    const int k = r.paley.k, m2 = r.paley.m2;
    const size_t lds = (size_t)r.n * sizeof(float) + (size_t)(m2 < 8 ? m2 : 8) * k * sizeof(float) +
                       (size_t)k * ((k + 31) / 32) * sizeof(uint32_t) + (size_t)((k + 3) & ~3);
    return (int64_t)(lds + kStaticLds) <= dev.lds_per_block;
}

hipError_t launch_generic(const Request &r, const DeviceInfo &dev)
{
    GenericArgs ga{};
    ga.x = r.x;
    ga.codes_in = r.codes_in;
    ga.scales_in = r.scales_in;
    ga.s = r.s;
    ga.codes = r.codes;
    ga.scales = r.scales;
    ga.y = r.y;
    ga.rows = r.rows;
    ga.n = r.n;
    // butterflies over runs of b elements, or of m2 for H_k (x) H_m2
    const int fw = r.paley.k > 1 ? r.paley.m2 : r.b;
    int lb = 0;
    while ((1 << lb) < fw)
        ++lb;
    ga.log_b = lb;
    ga.pk = r.paley.k;
    ga.pm2 = r.paley.m2;
    ga.pp = r.paley.p;
    ga.pe = r.paley.e;
    ga.pmod0 = r.paley.mod[0];
    ga.pmod1 = r.paley.mod[1];
    ga.pmod2 = r.paley.mod[2];
    ga.pwords = (r.paley.k + 31) / 32;
    ga.pjb = r.paley.m2 < 8 ? r.paley.m2 : 8;
    ga.group = r.group;
    ga.dst_rows = r.dst_rows;
    ga.cache_rows = r.cache_rows;
    int qmax = r.bits == 8 ? 127 : 7;
    ga.kq = (float)(1.0 / (__builtin_sqrt((double)r.b) * qmax));
    ga.rb = (float)(1.0 / __builtin_sqrt((double)r.b));

    if ((int64_t)(generic_lds(ga) + kStaticLds) > dev.lds_per_block)
        return hipErrorInvalidValue;

    switch (r.op) {
    case kRotateQuant:
        if (r.x_dtype == kF32) return pick_bits<kRotateQuant, kF32>(ga, r, dev);
        if (r.x_dtype == kBF16) return pick_bits<kRotateQuant, kBF16>(ga, r, dev);
        return pick_bits<kRotateQuant, kF16>(ga, r, dev);
    case kRotate:
        if (r.x_dtype == kF32) return go<kRotate, kF32, 4, kF32>(ga, r, dev);
        if (r.x_dtype == kBF16) return go<kRotate, kBF16, 4, kF32>(ga, r, dev);
        return go<kRotate, kF16, 4, kF32>(ga, r, dev);
    case kDequantInv:
        if (r.y_dtype == kF32) return pick_bits<kDequantInv, kF32>(ga, r, dev);
        return pick_bits<kDequantInv, kBF16>(ga, r, dev);
    }
    return hipErrorInvalidValue;
}

}  // namespace hq
