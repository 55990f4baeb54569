// hq_paley_mfma.hip -- matrix-core kernels for the full-width rotation of
// rows whose width is not a power of two: n = k * 32, H_n = H_k (x) H_32 with
// H_k from Paley's first construction, fused with the per-row quantiser.
// For k = 344 (the FFN width 11008, GF(7^3)) paley343h_kernel quantises
// (three product waves and a helper wave, see its own comment),
// paley343_kernel rotates only and paley343_inv_kernel inverts, both from the
// block structure of H_344; paley_mfma_kernel takes the other orders in
// (320, 352] as one dense product.
//
// Pages cited: [RQ] "旋转量化：大模型低比特量化中的离群值克星" section 2.1 (larger
// Hadamard matrices as Kronecker products; the transform is additions and
// subtractions) and section 2.2 (absmax quantisation); [QT]
// "手把手教你用QuaRot实现LLM的4位量化：从原理到代码实践" section 2.1 (sign flip, then the
// Hadamard matrix); [MS] "QuaRot：基于旋转的离群值抑制算法说明" YAML table (full-width
// block size).
//
// Element i * 32 + j of a row is entry (i, j).  y = (x * s) . H_n splits into
//   Z[i'][j] = sum_i H_k[i][i'] u[i][j]      a dense k-point product
//   y[i'][j'] = sum_j H_32[j][j'] Z[i'][j]   32-point butterflies
// The dense product runs on the matrix core: u is bf16 or f16 and H_k is
// +-1, so every product is exact and the sums are fp32.  As a 16x16x32
// product D[m][n] = sum_k A[m][k] B[k][n] it has m = j (two tiles of 16),
// k = i (chunks of 32) and n = i' (tiles of 16): A is the row, staged in LDS
// transposed to [j][i]; B is H_k, which each wave builds once for its share
// of the i' tiles and keeps in registers.  The butterflies then run on the
// result in registers: j = 16 mt + 4 rg + r is the tile, the lane's row
// group and the register, so two of the five stages cross lanes.
#include <mutex>

#include "hq_device.h"
#include "hq_internal.h"
#include "hq_fast_impl.h"  // the INT4 / INT8 code packers

namespace hq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;               // waves per workgroup (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kM2 = 32;                 // the power-of-two factor this kernel takes

struct PaleyArgs {
    const void *x;
    const int8_t *s;
    void *codes;
    void *scales;
    int64_t rows;
    int n;          // k * 32
    int k;          // Paley order
    int p, e, mod0, mod1, mod2;  // GF(k - 1) = GF(p^e) (see PaleySpec)
    float kq;       // 1 / (sqrt(n) * qmax)
    // inverse: codes and scales above are its inputs
    void *y;
    int y_bf16;
    int scale_f16;
    float rb;       // 1 / sqrt(n)
    // k = 344 forward: the product waves' and the helper's operands (see
    // paley343h_kernel), [operand][lane], for the input's 16-bit type
    const void *hop;
};

// GF(p^e) on element indices c0 + p c1 + p^2 c2 (e <= 3): the square of a
__device__ int gfp_square(int a, const PaleyArgs &g)
{
    const int p = g.p, e = g.e;
    if (e == 1)
        return (int)((int64_t)a * a % p);
    int c[3] = {0, 0, 0}, pr[5] = {0, 0, 0, 0, 0};
    const int md[3] = {g.mod0, g.mod1, g.mod2};
    for (int i = 0; i < e; ++i) {
        c[i] = a % p;
        a /= p;
    }
    for (int i = 0; i < e; ++i)
        for (int j = 0; j < e; ++j)
            pr[i + j] += c[i] * c[j];
    for (int d = 2 * e - 2; d >= e; --d) {  // x^e = -(md[e-1] x^(e-1) + ... + md[0])
        const int t = pr[d] % p;
        pr[d] = 0;
        for (int i = 0; i < e; ++i)
            pr[d - e + i] -= t * md[i];
    }
    int r = 0;
    for (int i = e - 1; i >= 0; --i)
        r = r * p + ((pr[i] % p) + p) % p;
    return r;
}

// Field elements as packed digits, one byte each (a prime order keeps its
// index): a - b digit by digit mod p without any division, then back to an
// element index.  Every byte of t stays in [1, 2p - 1] and of t + 128 - p
// below 256, so no carry crosses a byte.
__device__ __forceinline__ int diff_index(int pa, int pb, int p, int e)
{
    if (e == 1) {
        const int d = pa - pb;
        return d < 0 ? d + p : d;
    }
    constexpr int kOnes = 0x10101;
    int t = pa + p * kOnes - pb;
    t -= (((t + (128 - p) * kOnes) >> 7) & kOnes) * p;  // digits >= p
    return (t & 0xFF) + p * ((t >> 8) & 0xFF) + p * p * ((t >> 16) & 0xFF);
}

// LDS tables of the set-up: the packed digits of every element, the squares
// by packed code, and H_k as bits (bit i of word [i'][i / 32] set: -1)
struct PaleyLds {
    int digits[352];
    unsigned char square[352];
    uint32_t hbits[352 * 11];
};

// Builds the LDS tables (all threads of the workgroup; ends with a barrier)
__device__ void paley_build(PaleyLds &L, const PaleyArgs &g, int words)
{
    const int q = g.k - 1, p = g.p, e = g.e;
    for (int a = threadIdx.x; a < q; a += kThreads) {
        L.square[a] = 0;
        int code = a;
        if (e > 1) {
            int r = a;
            code = 0;
            for (int i = 0; i < e; ++i) {
                code |= (r % p) << (8 * i);
                r /= p;
            }
        }
        L.digits[a] = code;
    }
    lds_barrier();
    for (int a = threadIdx.x + 1; a < q; a += kThreads)
        L.square[gfp_square(a, g)] = 1;  // concurrent writes store the same 1
    lds_barrier();
    // H_k[i][i']: row 0 all +1; column 0 -1 below row 0; 1 on the diagonal;
    // chi(a - b) for a = i - 1, b = i' - 1 elsewhere
    for (int idx = threadIdx.x; idx < g.k * words; idx += kThreads) {
        const int ip = idx / words, w = idx % words;
        uint32_t bits = 0;
        const int pb = ip > 0 ? L.digits[ip - 1] : 0;
        for (int t = 0; t < 32; ++t) {
            const int i = 32 * w + t;
            bool neg = false;
            if (i > 0 && i < g.k) {
                if (ip == 0)
                    neg = true;
                else if (i != ip)
                    neg = !L.square[diff_index(L.digits[i - 1], pb, p, e)];
            }
            bits |= (neg ? 1u : 0u) << t;
        }
        L.hbits[idx] = bits;
    }
    lds_barrier();
}

// One B operand from the bit matrix: H_k[i][i'] for i = 32c + 8rg + e
// (e = 0..7) and i' = 16t + l16, as +-1 in the 16-bit type
template <int IN>
__device__ __forceinline__ u32x4 paley_operand(const PaleyLds &L, int t, int c, int l16, int rg, int words,
                                               int k)
{
    constexpr uint32_t kOnes = IN == kBF16 ? 0x3F803F80u : 0x3C003C00u;
    const int ip = 16 * t + l16;
    const uint32_t b = ip < k ? (L.hbits[ip * words + c] >> (8 * rg)) & 0xFFu : 0u;
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p)
        r[p] = kOnes | (((b >> (2 * p)) & 1u) << 15) | (((b >> (2 * p + 1)) & 1u) << 31);
    return r;
}

template <int IN>
__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (IN == kBF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// butterfly across lanes l and l ^ 16 (X = 16) or l ^ 32 (X = 32): the lower
// lane gets own + partner, the upper partner - own
template <int X>
__device__ __forceinline__ float xbutterfly(float v, float sgn)
{
    const uint32_t u = __float_as_uint(v);
    auto r = X == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                     : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // lower lane: r[0] own, r[1] partner; upper lane: r[0] partner, r[1] own
    return __builtin_fmaf(sgn, __uint_as_float(r[1]), __uint_as_float(r[0]));
}

// KC: chunks of 32 of the contraction index i (k <= 32 KC); the i' tiles
// number 2 KC, and wave w takes tiles w, w + 8, ...
template <int KC, int IN, int BITS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void paley_mfma_kernel(PaleyArgs a)
{
    constexpr int kNT = 2 * KC;                 // i' tiles of 16
    constexpr int kTPW = (kNT + kWaves - 1) / kWaves;
    constexpr int kChunks = KC * 32 * kM2 / 8;  // 16-byte chunks of a padded row
    constexpr int kCPT = (kChunks + kThreads - 1) / kThreads;
    // LDS row stride of the staged row (elements): every chunk index a thread
    // takes lands inside a row (those past the data write zeros into the
    // padding), and 16 rows apart by a multiple of 4 banks plus 4
    constexpr int kRS = ((kCPT * kThreads / 4 + 31) / 32) * 32 + 8;
    constexpr int qmax = (1 << (BITS - 1)) - 1;
    __shared__ __align__(16) uint16_t xt[2][kM2 * kRS];  // two rows, [j][i]
    __shared__ __align__(16) uint32_t cst[KC * 32 * kM2 * BITS / 32];  // its codes
    __shared__ PaleyLds pl;
    __shared__ float red[kWaves];
    static_assert(KC <= 11, "the set-up tables hold k <= 352");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, rg = lane >> 4;
    const int n = a.n, k = a.k;
    const int nchunks = n / 8;  // 16-byte chunks of a row

    // ---- once: H_k as bits in LDS, the zero padding of the staged row, and
    // this wave's B operands in registers
    for (int t = tid; t < 2 * kM2 * kRS; t += kThreads)
        (&xt[0][0])[t] = 0;
    paley_build(pl, a, KC);
    u32x4 hb[kTPW][KC];
    // (a wave without a tile in the last slot computes a copy of the last
    // tile there and drops it: no branch around any product)
#pragma unroll
    for (int tt = 0; tt < kTPW; ++tt) {
        const int t = wave + kWaves * tt;
#pragma unroll
        for (int c = 0; c < KC; ++c)
            hb[tt][c] = paley_operand<IN>(pl, t < kNT ? t : kNT - 1, c, l16, rg, KC, k);
    }

    // ---- the chunks this thread stages: chunk q holds elements 8q .. 8q+7,
    // i.e. i = q / 4, j = 8 (q % 4) .. +7.  The 64 lanes of a wave take 64
    // consecutive i of one j block, so their LDS writes fall in consecutive
    // words.  Their signs are the same every row.
    auto chunk_of = [&](int cc) {
        const int c = tid + kThreads * cc;
        const int i = (c >> 8) * 64 + (c & 63), jq = (c >> 6) & 3;
        return 4 * i + jq;
    };
    uint32_t neg[kCPT];
#pragma unroll
    for (int cc = 0; cc < kCPT; ++cc) {
        const int q = chunk_of(cc);
        uint32_t m = 0;
        if (q < nchunks)
            for (int e = 0; e < 8; ++e)
                m |= (a.s[8 * q + e] < 0 ? 1u : 0u) << e;
        neg[cc] = m;
    }
    auto load_row = [&](int64_t row, u32x4 (&r)[kCPT]) {
        const auto rs = rsrc((const uint16_t *)a.x + row * n, 2 * n);
#pragma unroll
        for (int cc = 0; cc < kCPT; ++cc) {
            const int q = chunk_of(cc);
            r[cc] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rs, q < nchunks ? 16 * q : 0x7FFFFFF0, 0, kNonTemporal));
        }
    };

    const float sgn16 = (lane & 16) ? -1.0f : 1.0f;
    const float sgn32 = (lane & 32) ? -1.0f : 1.0f;

    u32x4 cur[kCPT];
    // stages the row held in cur into LDS buffer `buf`, transposed, signs
    // applied (chunks past the row were read as 0 and write 0 into the
    // padding)
    auto stage = [&](int buf) {
#pragma unroll
        for (int cc = 0; cc < kCPT; ++cc) {
            const int q = chunk_of(cc);
            const int i = q >> 2, j0 = 8 * (q & 3);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t wv = cur[cc][e >> 1];
                uint32_t h = (e & 1) ? (wv >> 16) : (wv & 0xFFFFu);
                h ^= ((neg[cc] >> e) & 1u) << 15;
                xt[buf][(j0 + e) * kRS + i] = (uint16_t)h;
            }
        }
    };
    // Rows go through two LDS buffers: while one row is multiplied, the next
    // is staged and the one after it is loaded.
    int64_t row = blockIdx.x;
    if (row < a.rows) {
        load_row(row, cur);
        stage(0);
        if (row + gridDim.x < a.rows)
            load_row(row + gridDim.x, cur);
    }
    lds_barrier();
    int buf = 0;
    for (; row < a.rows; row += gridDim.x, buf ^= 1) {
        if (row + gridDim.x < a.rows) {
            stage(buf ^ 1);
            if (row + 2 * gridDim.x < a.rows)
                load_row(row + 2 * gridDim.x, cur);
        }

        // ---- Z[i'][j] on the matrix core
        f32x4 acc[kTPW][2];
#pragma unroll
        for (int tt = 0; tt < kTPW; ++tt)
            acc[tt][0] = acc[tt][1] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const u32x4 av = *(const u32x4 *)&xt[buf][(16 * mt + l16) * kRS + 32 * c + 8 * rg];
#pragma unroll
                for (int tt = 0; tt < kTPW; ++tt)
                    acc[tt][mt] = mma<IN>(av, hb[tt][c], acc[tt][mt]);
            }
        }

        // ---- 32-point butterflies over j = 16 mt + 4 rg + r, natural order
        float mx = 0.0f;
        // (a duplicated last tile repeats values of the row: harmless to the
        // maximum)
#pragma unroll
        for (int tt = 0; tt < kTPW; ++tt) {
            float v[2][4];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[mt][r] = acc[tt][mt][r];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                // j bit 0, then bit 1
                float a0 = v[mt][0] + v[mt][1], a1 = v[mt][0] - v[mt][1];
                float a2 = v[mt][2] + v[mt][3], a3 = v[mt][2] - v[mt][3];
                v[mt][0] = a0 + a2;
                v[mt][2] = a0 - a2;
                v[mt][1] = a1 + a3;
                v[mt][3] = a1 - a3;
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[mt][r] = xbutterfly<32>(xbutterfly<16>(v[mt][r], sgn16), sgn32);  // bits 2, 3
#pragma unroll
            for (int r = 0; r < 4; ++r) {  // bit 4
                const float lo = v[0][r], hi = v[1][r];
                v[0][r] = lo + hi;
                v[1][r] = lo - hi;
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[tt][mt][r] = v[mt][r];
                    mx = fmaxf(mx, fabsf(v[mt][r]));
                }
        }
        // ---- row maximum (columns i' >= k are 0)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        if (lane == 0)
            red[wave] = mx;
        lds_barrier();
        float m = red[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            m = fmaxf(m, red[w]);
        const RowQuant rq = row_quant(m, a.kq, qmax);
        if (rq.boost != 1.0f) {  // workgroup-uniform: a row too small for qmax / max
#pragma unroll
            for (int tt = 0; tt < kTPW; ++tt)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    acc[tt][mt] *= rq.boost;
        }

        // ---- codes of y[i'][16 mt + 4 rg .. +3] into LDS
#pragma unroll
        for (int tt = 0; tt < kTPW; ++tt) {
            const int ip = 16 * (wave + kWaves * tt) + l16;
            if (wave + kWaves * tt >= kNT || ip >= k)
                continue;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int e0 = ip * kM2 + 16 * mt + 4 * rg;  // first element
                uint32_t w = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qc = quant_code(acc[tt][mt][r], rq.inv, qmax);
                    w |= BITS == 4 ? ((uint32_t)qc & 15u) << (4 * r) : ((uint32_t)qc & 255u) << (8 * r);
                }
                if constexpr (BITS == 4)
                    ((uint16_t *)cst)[e0 >> 2] = (uint16_t)w;
                else
                    cst[e0 >> 2] = w;
            }
        }
        lds_barrier();
        // ---- coalesced stores
        const int cbytes = n * BITS / 8;
        uint8_t *crow = (uint8_t *)a.codes + row * (int64_t)cbytes;
        for (int t = tid; t < cbytes / 16; t += kThreads)
            ((u32x4 *)crow)[t] = ((const u32x4 *)cst)[t];
        if (tid == 0)
            ((float *)a.scales)[row] = rq.scale;
    }
}

// ---------------------------------------------------------------------------
// k = 344 (q = 343 = 7^3): H_k from its block structure.
//
// The additive group of GF(7^3) is Z_7^3 (digits c0, c1, c2 of a = c0 + 7 c1
// + 49 c2), so chi(a - b) depends on the top digits only through
// d = (a2 - b2) mod 7: the 343 x 343 core of H_k is 7 x 7 blocks of 49 x 49,
// and block (a2, b2) is the same matrix K_d for every pair with the same d.
// Each block is padded to 64 x 64 and the border of H_k goes into the
// padding: input slot 49 of block 0 holds u[0] (the extra point), and
//   K_d[sa][sb]  = chi(49 d + (sa - sb digit-wise)), sa, sb < 49,
//                  with 1 on the diagonal of K_0 (the identity of H_k)
//   K_d[49][sb]  = +1        (H_k[0][i'] = +1 for every i')
//   K_d[sa][49]  = -1        (H_k[i][0] = -1 for i >= 1)
//   K_d[49][49]  = +1        (H_k[0][0])
// so that output (b2, sb < 49) is Z[1 + 49 b2 + sb] and output (b2, 49) is
// Z[0] for every b2 (the copies with b2 > 0 are dropped; columns 50..63
// are zero).  The product is 7 x 7 x 2 x 2 matrix-core steps per 16-column
// tile and 32 rows j, 1.62 times the dense count, but a wave's share of H
// (its 16 columns of every K_d) is 56 registers instead of 132, which
// leaves room for a row of prefetch and for two workgroups per compute unit
// that overlap their rows' phases.
constexpr int kBW = 4;                   // waves per workgroup: one 16-column tile each
constexpr int kBThreads = 64 * kBW;
constexpr int kBTop = 7;                 // values of the top digit
constexpr int kBBlk = 49;                // block size 7^2
constexpr int kBPad = 64;                // padded block
constexpr int kBK = 344;                 // Paley order
constexpr int kBRS = kBTop * kBPad + 8;  // LDS row stride of the staged row (elements)
constexpr int kBCPT = 6;                 // 16-byte chunks per thread (6 x 256 >= 1376)
constexpr int kBOcc = 2;                 // workgroups per compute unit
// Staged row of the forward kernel: row j starts at element frow(j).  One
// staging store of a wave covers 16 consecutive slots of four rows 8 apart;
// the shift of 16 elements per group of 8 rows puts those four rows in
// different LDS banks (at the stride kBRS all four share the same 8 banks).
// The stride 504 (252 dwords, 28 mod 32) keeps the matrix-core operand
// reads of 8 consecutive rows in distinct banks.
constexpr int kBRSF = 504;
constexpr int kDropOffset = 0x7FFFFF00;  // buffer offset past every buffer: the store is dropped
__device__ __forceinline__ int frow(int j) { return j * kBRSF + 16 * (j >> 3); }
static_assert(31 * kBRSF + 16 * 3 + kBTop * kBPad <= 32 * kBRSF, "staged row fits");

// entry (sa, sb) of the padded block K_d (see above); sq: the squares of
// GF(343) by element index.  TR: the blocks of H_k^T instead, for the
// inverse: chi(-x) = -chi(x) (q = 3 mod 4), so the core changes sign and the
// border rows and columns trade theirs:
//   K_d[sa][sb] = -chi(49 d + (sa - sb)), 1 on the diagonal of K_0;
//   K_d[49][sb] = -1; K_d[sa][49] = +1; K_d[49][49] = +1.
template <bool TR = false>
__device__ int block_entry(const unsigned char *sq, int d, int sa, int sb)
{
    if (sa < kBBlk && sb < kBBlk) {
        if (d == 0 && sa == sb)
            return 1;
        const int d0 = (sa % 7 - sb % 7 + 7) % 7;
        const int d1 = (sa / 7 - sb / 7 + 7) % 7;
        const bool sqr = sq[d0 + 7 * d1 + 49 * d];
        return (sqr != TR) ? 1 : -1;
    }
    if (sa < kBBlk && sb == kBBlk)
        return TR ? 1 : -1;
    if (sa == kBBlk && sb < kBBlk)
        return TR ? -1 : 1;
    if (sa == kBBlk && sb == kBBlk)
        return 1;
    return 0;
}

// Rotation only (hq_rotate): the rotated row y / sqrt(n) in fp32 to a.y
template <int IN>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(kBOcc))) void paley343_kernel(PaleyArgs a)
{
    constexpr int n = kBK * kM2;
    __shared__ __align__(16) uint16_t xt[kM2 * kBRSF];            // [j][a2][slot] from frow(j)
    __shared__ unsigned char sq[kBK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, rg = lane >> 4;

    // ---- once: zero padding, the squares, this wave's 16 columns of every K_d
    for (int t = tid; t < kM2 * kBRSF / 8; t += kBThreads)
        ((u32x4 *)xt)[t] = (u32x4){0u, 0u, 0u, 0u};
    for (int t = tid; t < kBK; t += kBThreads)
        sq[t] = 0;
    lds_barrier();
    for (int t = tid + 1; t < kBK - 1; t += kBThreads)
        sq[gfp_square(t, a)] = 1;  // concurrent writes store the same 1
    lds_barrier();
    constexpr uint32_t kOne = IN == kBF16 ? 0x3F80u : 0x3C00u;
    u32x4 bd[kBTop][2];
#pragma unroll
    for (int d = 0; d < kBTop; ++d)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint32_t w = 0;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int v = block_entry(sq, d, 32 * c + 8 * rg + 2 * p + h, 16 * wave + l16);
                    const uint32_t bits = v == 0 ? 0u : (v > 0 ? kOne : (kOne | 0x8000u));
                    w |= bits << (16 * h);
                }
                bd[d][c][p] = w;
            }

    // ---- the chunks this thread stages: chunk q = 256 cc + tid holds the
    // elements 8q .. 8q + 7 of a row, i.e. i = q / 4 and j = 8 (q % 4) .. +7,
    // so a wave's load is 1 KB of contiguous memory; the chunk's slot in the
    // staged row and its signs are the same every row
    // Signs of a chunk as one word: element 2p's at bit 15 - 4p and element
    // 2p + 1's at bit 31 - 4p, so (w << 4p) & 0x80008000 is the sign mask of
    // dword p.
    uint32_t neg[kBCPT];
#pragma unroll
    for (int cc = 0; cc < kBCPT; ++cc) {
        const int q = kBThreads * cc + tid;
        uint32_t m = 0;
        if (q < kBK * kM2 / 8)
            for (int e = 0; e < 8; ++e)
                m |= (a.s[8 * q + e] < 0 ? 1u : 0u) << ((e & 1) ? 31 - 2 * (e - 1) : 15 - 2 * e);
        neg[cc] = m;
    }
    // (no branch around the loads: past the last row the buffer has size 0
    // and every load reads 0, so the waits before the row is staged count
    // only these loads, not the stores issued after them)
    u32x4 cur[kBCPT];
    auto load_row = [&](int64_t row) {
        const bool ok = row < a.rows;
        const auto rs = rsrc((const uint16_t *)a.x + (ok ? row : 0) * n, ok ? 2 * n : 0);
#pragma unroll
        for (int cc = 0; cc < kBCPT; ++cc) {
            const int q = kBThreads * cc + tid;
            cur[cc] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rs, q < kBK * kM2 / 8 ? 16 * q : 0x7FFFFFF0, 0, 0));
        }
    };
    // the row held in cur into the staged layout, signs applied
    auto stage = [&]() {
#pragma unroll
        for (int cc = 0; cc < kBCPT; ++cc) {
            const int q = kBThreads * cc + tid;
            const int i = q >> 2;
            if (i >= kBK)
                continue;
            const int slot = i == 0 ? kBBlk : kBPad * ((i - 1) / kBBlk) + (i - 1) % kBBlk;
            uint16_t *dst = xt + frow(8 * (q & 3)) + slot;  // rows 8 (q & 3) + e at dst + e kBRSF
            // (opaque to the compiler: otherwise it keeps all 48 masks of
            // the loop in registers)
            uint32_t ng = neg[cc];
            asm volatile("" : "+v"(ng));
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                // ((ng << 4p) & 0x80008000) ^ data in one v_bitop3_b32 (the
                // data in the middle operand: the truth table is then the
                // same whichever outer operand indexes its high bit)
                const uint32_t wv = __builtin_amdgcn_bitop3_b32(ng << (4 * p), cur[cc][p], 0x80008000u, 0x6C);
                dst[2 * p * kBRSF] = (uint16_t)wv;
                dst[(2 * p + 1) * kBRSF] = (uint16_t)(wv >> 16);
            }
        }
    };

    const float sgn32 = (lane & 32) ? -1.0f : 1.0f;
    const int sb = 16 * wave + l16;  // this lane's column in every block
    // One row at a time per workgroup, the next one in flight: its loads go
    // out as soon as the row before it is staged and are staged once this
    // row's codes are in LDS.  Two workgroups per compute unit cover each
    // other's barriers.
    int64_t row = blockIdx.x;
    if (row < a.rows) {
        load_row(row);
        stage();
        load_row(row + gridDim.x);
    }
    lds_barrier();
    for (; row < a.rows; row += gridDim.x) {
        // ---- Z on the matrix core: acc[b2][mt] = block row b2, j tile mt
        f32x4 acc[kBTop][2];
#pragma unroll
        for (int b2 = 0; b2 < kBTop; ++b2)
            acc[b2][0] = acc[b2][1] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int a2 = 0; a2 < kBTop; ++a2) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const u32x4 av = *(const u32x4 *)&xt[frow(16 * mt + l16) + kBPad * a2 + 32 * c + 8 * rg];
#pragma unroll
                    for (int b2 = 0; b2 < kBTop; ++b2)
                        acc[b2][mt] = mma<IN>(av, bd[(a2 - b2 + kBTop) % kBTop][c], acc[b2][mt]);
                }
            // (keeps the scheduler from hoisting every block's operand
            // reads to the top, which would need 112 registers at once)
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- 32-point butterflies over j = 16 mt + 4 rg + r.  Bits 0, 1
        // (r) and 4 (mt) are in registers.  Bits 2 and 3 cross lanes; each
        // swap exchanges two registers at once, which hands the register
        // index to the lanes and takes the j bit into the registers:
        //  - bit 2 pairs mt = 0, 1: afterwards lane bit 4 is output bit 4 and
        //    register slot s is output bit 2;
        //  - bit 3 pairs b2 = 2k, 2k + 1: afterwards lane bit 5 is the low bit
        //    of b2 and register 2k + t is output bit 3.  Block 6 has no
        //    partner and keeps bit 3 on lane bit 5.
        // So for k < 3 a lane ends with the 16 outputs j = 16 (lane bit 4) +
        // r + 4 s + 8 t of row 1 + 49 (2k + lane bit 5) + sb, and with the 8
        // outputs j = 16 (lane bit 4) + 8 (lane bit 5) + r + 4 s of block 6.
#pragma unroll
        for (int b2 = 0; b2 < kBTop; ++b2)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const float a0 = acc[b2][mt][0] + acc[b2][mt][1], a1 = acc[b2][mt][0] - acc[b2][mt][1];
                const float a2_ = acc[b2][mt][2] + acc[b2][mt][3], a3 = acc[b2][mt][2] - acc[b2][mt][3];
                acc[b2][mt][0] = a0 + a2_;
                acc[b2][mt][2] = a0 - a2_;
                acc[b2][mt][1] = a1 + a3;
                acc[b2][mt][3] = a1 - a3;
            }
#pragma unroll
        for (int b2 = 0; b2 < kBTop; ++b2)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float lo = acc[b2][0][r], hi = acc[b2][1][r];  // bit 4
                const auto w = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo + hi), __float_as_uint(lo - hi),
                                                                false, false);  // bit 2
                const float x0 = __uint_as_float(w[0]), x1 = __uint_as_float(w[1]);
                acc[b2][0][r] = x0 + x1;
                acc[b2][1][r] = x0 - x1;
            }
#pragma unroll
        for (int k = 0; k < kBTop / 2; ++k)
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[2 * k][sl][r]),
                                                                    __float_as_uint(acc[2 * k + 1][sl][r]), false,
                                                                    false);  // bit 3
                    const float x0 = __uint_as_float(w[0]), x1 = __uint_as_float(w[1]);
                    acc[2 * k][sl][r] = x0 + x1;
                    acc[2 * k + 1][sl][r] = x0 - x1;
                }
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[kBTop - 1][sl][r] = xbutterfly<32>(acc[kBTop - 1][sl][r], sgn32);
        lds_barrier();  // every wave is done with the staged row
        if (row + gridDim.x < a.rows)  // the next row (loaded one row ago) into the staged layout
            stage();
        load_row(row + 2 * gridDim.x);
        // y / sqrt(n): 16 (block 6: 8) consecutive outputs per lane
        const auto ry = rsrc((uint8_t *)a.y + row * (int64_t)(n * 4), n * 4);
        const int lb4r = (lane >> 4) & 1, lb5r = lane >> 5;
        // (every lane issues every store, those with nothing to store at
        // an offset past the buffer, which drops them: no branch, so the
        // next row's loads wait for loads only)
        auto st8 = [&](bool ok, int e0, const float (&o)[8]) {
            const int off = ok ? 4 * e0 : kDropOffset;
            __builtin_amdgcn_raw_buffer_store_b128(
                (u32x4){__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])},
                ry, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(
                (u32x4){__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]), __float_as_uint(o[7])},
                ry, off + 16, 0, 0);
        };
#pragma unroll
        for (int k = 0; k < kBTop / 2; ++k) {
            const int b2 = 2 * k + lb5r;
            const bool ok = sb < kBBlk || (sb == kBBlk && b2 == 0);
            const int ip = sb >= kBBlk ? 0 : 1 + kBBlk * b2 + sb;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                float o[8];
#pragma unroll
                for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        o[4 * sl + r] = acc[2 * k + t][sl][r] * a.rb;
                st8(ok, ip * kM2 + 16 * lb4r + 8 * t, o);
            }
        }
        {
            const int ip = 1 + kBBlk * (kBTop - 1) + (sb < kBBlk ? sb : 0);
            float o[8];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[4 * sl + r] = acc[kBTop - 1][sl][r] * a.rb;
            st8(sb < kBBlk, ip * kM2 + 16 * lb4r + 8 * lb5r, o);
        }
        lds_barrier();  // the next row is staged
    }
}

// ---------------------------------------------------------------------------
// k = 344 forward with a helper wave (paley343h_kernel): the dense count of
// products and no padded outputs.
//
// Input slots.  Slot 48 (the last) of each block and the extra point are
// taken out of the blocks, so that a block keeps 48 slots: the contraction
// index ("K-index") of Paley index i is
//   48 a2 + sa           for i = 1 + 49 a2 + sa, sa < 48     (0 .. 335)
//   336 + a2             for i = 1 + 49 a2 + 48              (336 .. 342)
//   343                  for i = 0                            (the extra point)
// and 344 .. 351 are zero: 11 chunks of 32, the dense count.  Blocks 2p and
// 2p + 1 fill chunks 3p .. 3p + 2: chunk 3p is block 2p's slots 0..31, chunk
// 3p + 1 its slots 32..47 and block 2p + 1's slots 0..15, chunk 3p + 2 block
// 2p + 1's slots 16..47; chunk 9 is block 6's slots 0..31, and chunk 10 holds
// block 6's slots 32..47, the seven slots 48 and the extra point.  Against
// the output column (b2, sb), sb < 48, a chunk's 32 x 16 operand therefore
// depends only on its kind (3p, 3p + 1, 3p + 2) and on (2p - b2) mod 7
// (H_k's blocks are circulant in the top digit), and chunk 10's on b2: 28
// operands per 16-column tile of every block, 112 registers.
//
// Waves 0..2 each own the 16 columns 16 w .. 16 w + 15 of every block: 154
// products per row, then the 32-point butterflies of the forward kernel, the
// maximum of their values and the values themselves (fp32) into an LDS row
// buffer in natural order.  The fourth wave (the helper) computes the
// columns that the blocks no longer hold (column 48 of every block and
// column 0, the extra point's: 8 of a 16-column tile, 22 products), stages
// the rows (loads, signs, the transposed layout) and quantises the row
// before from the LDS buffer: the maximum, the codes of 32 consecutive
// outputs per lane and 1 KB code stores per wave instruction.  Per row the
// product waves run 154 products and the butterflies, and the work they no
// longer do (staging, quantiser, stores, the padded columns) goes to the
// helper, whose products and vector work fit beside theirs.
constexpr int kHW = 4;                       // waves: three product waves and the helper
constexpr int kHThreads = 64 * kHW;
constexpr int kHK = 352;                     // K-indices: 11 chunks of 32
constexpr int kHRS = 376;                    // staged row stride (188 dwords, 28 mod 32)
constexpr int kHOS = 36;                     // LDS row buffer: floats per output column
// Staged row j starts at element hrow(j).  As in the forward kernel, the
// stride keeps the operand reads of 8 consecutive rows in distinct banks and
// the shift of 16 elements per group of 8 rows separates the four rows one
// staging store covers.
__device__ __forceinline__ constexpr int hrow(int j) { return j * kHRS + 16 * (j >> 3); }
static_assert(kHRS >= kHK, "staged rows do not overlap");

// K-index of Paley index i, and back (a K-index past 343 has no index: -1)
__device__ __forceinline__ int hkappa(int i)
{
    if (i == 0)
        return kBK - 1;
    const int a2 = (i - 1) / kBBlk, sa = (i - 1) % kBBlk;
    return sa < kBBlk - 1 ? (kBBlk - 1) * a2 + sa : (kBBlk - 1) * kBTop + a2;
}
__device__ __forceinline__ int hindex(int kk)
{
    constexpr int kMain = (kBBlk - 1) * kBTop;  // 336
    if (kk < kMain)
        return 1 + kBBlk * (kk / (kBBlk - 1)) + kk % (kBBlk - 1);
    if (kk < kMain + kBTop)
        return 1 + kBBlk * (kk - kMain) + kBBlk - 1;
    return kk == kBK - 1 ? 0 : -1;
}
// H_k[i][ip] (Paley's first construction, I + [[0, 1^T], [-1, Q]]); 0 for i < 0
__device__ int hentry(const unsigned char *sq, int i, int ip)
{
    if (i < 0 || ip < 0)
        return 0;
    if (i == 0)
        return 1;
    if (ip == 0)
        return -1;
    if (i == ip)
        return 1;
    const int x = i - 1, y = ip - 1;
    const int d0 = (x % 7 - y % 7 + 7) % 7;
    const int d1 = ((x / 7) % 7 - (y / 7) % 7 + 7) % 7;
    const int d2 = (x / 49 - y / 49 + 7) % 7;
    return sq[d0 + 7 * d1 + 49 * d2] ? 1 : -1;
}
// the operand slot of chunk c against block b2 (see above), and a chunk and
// block that use slot ix
__device__ __forceinline__ constexpr int hslot(int c, int b2)
{
    return c == 10 ? 21 + b2
                   : (c % 3 == 0 ? (2 * (c / 3) - b2 + 7) % 7
                                 : (c % 3 == 1 ? 7 + (2 * (c / 3) - b2 + 7) % 7 : 14 + (2 * (c / 3) + 1 - b2 + 7) % 7));
}
__device__ __forceinline__ constexpr int hrep_c(int ix) { return ix >= 21 ? 10 : ix / 7; }
__device__ __forceinline__ constexpr int hrep_b2(int ix)
{
    return ix >= 21 ? ix - 21 : (ix / 7 == 2 ? (1 - ix % 7 + 7) % 7 : (7 - ix % 7) % 7);
}
// output column of lane l16 in the helper's tile: column 48 of block l16
// (l16 < 7), the extra point's column (l16 = 7), none (l16 > 7)
__device__ __forceinline__ int hxcol(int l16)
{
    return l16 < kBTop ? kBBlk * l16 + kBBlk : (l16 == kBTop ? 0 : -1);
}

// maximum of a non-negative value over the wave, in every lane (DPP within
// rows of 16 lanes, then the two permlane swaps)
__device__ __forceinline__ float wave_max_nonneg(float m)
{
    uint32_t v = __float_as_uint(m);
    v = fast::dpp_max<0xB1>(v);   // quad_perm [1,0,3,2]
    v = fast::dpp_max<0x4E>(v);   // quad_perm [2,3,0,1]
    v = fast::dpp_max<0x141>(v);  // row_half_mirror
    v = fast::dpp_max<0x140>(v);  // row_mirror
    const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = r16[0] > r16[1] ? r16[0] : r16[1];
    const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(r32[0] > r32[1] ? r32[0] : r32[1]);
}

__device__ u32x4 hoperand(const unsigned char *sq, int c, int rg, int ip, uint32_t kOne)
{
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t w = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int v = hentry(sq, hindex(32 * c + 8 * rg + 2 * p + h), ip);
            const uint32_t bits = v == 0 ? 0u : (v > 0 ? kOne : (kOne | 0x8000u));
            w |= bits << (16 * h);
        }
        r[p] = w;
    }
    return r;
}

// The operands every launch of paley343h_kernel uses, built once per GPU:
// operand 28 w + ix (w < 3) is slot ix of product wave w, operand 84 + c the
// helper's chunk c; [type][operand][lane], type 0 bf16, 1 f16.
constexpr int kHOps = 3 * 28 + kHK / 32;
__global__ __launch_bounds__(64) void paley343h_build(PaleyArgs a, u32x4 *tab)
{
    __shared__ unsigned char sq[kBK];
    const int lane = threadIdx.x, l16 = lane & 15, rg = lane >> 4;
    for (int t = lane; t < kBK; t += 64)
        sq[t] = 0;
    lds_barrier();
    for (int t = lane + 1; t < kBK - 1; t += 64)
        sq[gfp_square(t, a)] = 1;  // concurrent writes store the same 1
    lds_barrier();
    const int t = blockIdx.x;
    const uint32_t one = blockIdx.y == 0 ? 0x3F80u : 0x3C00u;
    u32x4 v;
    if (t < 84) {
        const int w = t / 28, ix = t % 28;
        v = hoperand(sq, hrep_c(ix), rg, 1 + kBBlk * hrep_b2(ix) + 16 * w + l16, one);
    } else {
        v = hoperand(sq, t - 84, rg, hxcol(l16), one);
    }
    tab[((int)blockIdx.y * kHOps + t) * 64 + lane] = v;
}

template <int IN, int BITS>
__global__ __launch_bounds__(kHThreads) __attribute__((amdgpu_waves_per_eu(kBOcc))) void paley343h_kernel(PaleyArgs a)
{
    constexpr int qmax = (1 << (BITS - 1)) - 1;
    constexpr int n = kBK * kM2;
    constexpr int kRowBytes = n * BITS / 8;
    constexpr float kMagic = BITS == 4 ? 12582920.0f : 12583040.0f;
    __shared__ __align__(16) uint16_t xt[hrow(31) + kHK];  // staged row [j][K-index]
    __shared__ __align__(16) float ob[kBK * kHOS];        // rotated row [i'][j], fp32
    __shared__ float red[kHW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, rg = lane >> 4;
    const int lb4 = (lane >> 4) & 1, lb5 = lane >> 5;
    const int64_t G = gridDim.x;
    int64_t row = blockIdx.x;

    const u32x4 *hop = (const u32x4 *)a.hop;
    // ---- once: zero the staged row (K-indices 344 .. 351 stay 0)
    for (int t = tid; t < (hrow(31) + kHK) / 8; t += kHThreads)
        ((u32x4 *)xt)[t] = (u32x4){0u, 0u, 0u, 0u};
    lds_barrier();

    if (wave < kHW - 1) {
        // ================= product waves: columns sb = 16 wave + l16 of every block
        const int sb = 16 * wave + l16;
        u32x4 op[28];
#pragma unroll
        for (int ix = 0; ix < 28; ++ix)
            op[ix] = hop[(28 * wave + ix) * 64 + lane];
        lds_barrier();  // the first row is staged
        for (; row - G < a.rows; row += G) {
            const bool valid = row < a.rows;
            f32x4 acc[kBTop][2];
            // ---- the codes of output columns 64 wave .. 64 wave + 63 of the
            // row before (none in the first pass: its buffers have size 0),
            // eight values at a time between the products of this row
            const bool have = row != (int64_t)blockIdx.x;
            const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
            const RowQuant rq = row_quant(m, a.kq, qmax);
            const auto rc = rsrc((uint8_t *)a.codes + (have ? row - G : 0) * (int64_t)kRowBytes, have ? kRowBytes : 0);
            const int qip = 64 * wave + lane;
            uint32_t qw[BITS == 4 ? 4 : 8];
            // (the magnification of tiny rows is a product by 1 for the others:
            // no branch among the products)
            auto qgroup = [&](int g) {
                const f32x4 w0 = *(const f32x4 *)&ob[qip * kHOS + 8 * g];
                const f32x4 w1 = *(const f32x4 *)&ob[qip * kHOS + 8 * g + 4];
                float v[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] *= rq.boost;
                uint32_t f[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    f[e] = __float_as_uint(__builtin_fmaf(v[e], rq.inv, kMagic));
                if constexpr (BITS == 4) {
                    qw[g] = fast::pack_int4(f);
                } else {
                    qw[2 * g] = fast::pack_int8(f[0], f[1], f[2], f[3]);
                    qw[2 * g + 1] = fast::pack_int8(f[4], f[5], f[6], f[7]);
                }
            };
            auto qstore = [&]() {
                if constexpr (BITS == 4) {
                    __builtin_amdgcn_raw_buffer_store_b128((u32x4){qw[0], qw[1], qw[2], qw[3]}, rc, 16 * qip, 0,
                                                           kNonTemporal);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b128((u32x4){qw[0], qw[1], qw[2], qw[3]}, rc, 32 * qip, 0,
                                                           kNonTemporal);
                    __builtin_amdgcn_raw_buffer_store_b128((u32x4){qw[4], qw[5], qw[6], qw[7]}, rc, 32 * qip + 16,
                                                           0, kNonTemporal);
                }
            };
            if (valid) {
#pragma unroll
                for (int b2 = 0; b2 < kBTop; ++b2)
                    acc[b2][0] = acc[b2][1] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
                // the operands of chunk c + 1 are read while chunk c multiplies
                u32x4 av[2][2];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    av[0][mt] = *(const u32x4 *)&xt[hrow(16 * mt + l16) + 8 * rg];
#pragma unroll
                for (int c = 0; c < kHK / 32; ++c) {
                    if (c + 1 < kHK / 32) {
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt)
                            av[(c + 1) & 1][mt] = *(const u32x4 *)&xt[hrow(16 * mt + l16) + 32 * (c + 1) + 8 * rg];
                    }
                    __builtin_amdgcn_sched_barrier(0);  // (the reads go out before the products)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int b2 = 0; b2 < kBTop; ++b2)
                            acc[b2][mt] = mma<IN>(av[c & 1][mt], op[hslot(c, b2)], acc[b2][mt]);
                    if (c < 4)
                        qgroup(c);
                    if (c == 3)
                        qstore();
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    qgroup(g);
                qstore();
            }
            lds_barrier();  // (1) the staged row is free; the row buffer has been read
            if (valid) {
                // 32-point butterflies over j = 16 mt + 4 rg + r, as in the
                // forward kernel: a lane ends with the 16 outputs j = 16 lb4 +
                // r + 4 s + 8 t of column 1 + 49 (2k + lb5) + sb (k < 3) and
                // the 8 outputs j = 16 lb4 + 8 lb5 + r + 4 s of block 6
#pragma unroll
                for (int b2 = 0; b2 < kBTop; ++b2)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const float a0 = acc[b2][mt][0] + acc[b2][mt][1], a1 = acc[b2][mt][0] - acc[b2][mt][1];
                        const float a2_ = acc[b2][mt][2] + acc[b2][mt][3], a3 = acc[b2][mt][2] - acc[b2][mt][3];
                        acc[b2][mt][0] = a0 + a2_;
                        acc[b2][mt][2] = a0 - a2_;
                        acc[b2][mt][1] = a1 + a3;
                        acc[b2][mt][3] = a1 - a3;
                    }
                // (each stage over all blocks before the next: the swaps then
                // find their inputs computed long before)
                uint32_t sw[kBTop][4][2];
#pragma unroll
                for (int b2 = 0; b2 < kBTop; ++b2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float lo = acc[b2][0][r], hi = acc[b2][1][r];  // bit 4
                        sw[b2][r][0] = __float_as_uint(lo + hi);
                        sw[b2][r][1] = __float_as_uint(lo - hi);
                    }
#pragma unroll
                for (int b2 = 0; b2 < kBTop; ++b2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const auto w = __builtin_amdgcn_permlane16_swap(sw[b2][r][0], sw[b2][r][1], false, false);
                        sw[b2][r][0] = w[0];
                        sw[b2][r][1] = w[1];
                    }
#pragma unroll
                for (int b2 = 0; b2 < kBTop; ++b2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {  // bit 2
                        const float x0 = __uint_as_float(sw[b2][r][0]), x1 = __uint_as_float(sw[b2][r][1]);
                        acc[b2][0][r] = x0 + x1;
                        acc[b2][1][r] = x0 - x1;
                    }
                uint32_t tw[kBTop / 2][2][4][2];
#pragma unroll
                for (int k = 0; k < kBTop / 2; ++k)
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[2 * k][sl][r]),
                                                                            __float_as_uint(acc[2 * k + 1][sl][r]),
                                                                            false, false);
                            tw[k][sl][r][0] = w[0];
                            tw[k][sl][r][1] = w[1];
                        }
                const float sgn32 = (lane & 32) ? -1.0f : 1.0f;
#pragma unroll
                for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[kBTop - 1][sl][r] = xbutterfly<32>(acc[kBTop - 1][sl][r], sgn32);
#pragma unroll
                for (int k = 0; k < kBTop / 2; ++k)
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {  // bit 3
                            const float x0 = __uint_as_float(tw[k][sl][r][0]), x1 = __uint_as_float(tw[k][sl][r][1]);
                            acc[2 * k][sl][r] = x0 + x1;
                            acc[2 * k + 1][sl][r] = x0 - x1;
                        }
                float mx = 0.0f;
#pragma unroll
                for (int b2 = 0; b2 < kBTop; ++b2)
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                        for (int r = 0; r < 4; r += 2)
                            mx = fmaxf(fmaxf(mx, fabsf(acc[b2][sl][r])), fabsf(acc[b2][sl][r + 1]));
                mx = wave_max_nonneg(mx);
                if (lane == 0)
                    red[wave] = mx;
#pragma unroll
                for (int k = 0; k < kBTop / 2; ++k) {
                    const int ip = 1 + kBBlk * (2 * k + lb5) + sb;
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int sl = 0; sl < 2; ++sl)
                            *(f32x4 *)&ob[ip * kHOS + 16 * lb4 + 8 * t + 4 * sl] = acc[2 * k + t][sl];
                }
                {
                    const int ip = 1 + kBBlk * (kBTop - 1) + sb;
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl)
                        *(f32x4 *)&ob[ip * kHOS + 16 * lb4 + 8 * lb5 + 4 * sl] = acc[kBTop - 1][sl];
                }
            }
            lds_barrier();  // (2) the row buffer holds this row; the next row is staged
        }
        return;
    }

    // ================= the helper wave
    const int xcol = hxcol(l16);
    u32x4 xo[kHK / 32];
#pragma unroll
    for (int c = 0; c < kHK / 32; ++c)
        xo[c] = hop[(84 + c) * 64 + lane];
    // Staging.  Unit U = 64 u + lane is the K-indices 4 G .. 4 G + 3 (G = U /
    // 4) against j = 8 h .. 8 h + 7 (h = U % 4): four 16-byte loads (the
    // rows i of the four K-indices), the signs, and a transpose in registers
    // into eight 8-byte LDS stores (four consecutive K-indices of one row j).
    // Within a block consecutive K-indices are consecutive rows i, so units
    // 0 .. 319 read rows i(4G) + t; the last lane group also holds G = 84,
    // 85 (the slots 48 and the extra point) and the 24 units past 343.
    constexpr int kHU = kBK;                // units: 86 groups of 4 K-indices x 4 groups of 8 j
    constexpr int kHUPL = (kHU + 63) / 64;  // 6 per lane
    int ubase[kHUPL - 1], ulast[4];
    uint32_t usg[kHUPL];  // signs: bits 15 - k and 31 - k for dword k = 4 t + q
    {
        // the unit's 8 signs of each row as one 8-byte load (all issued
        // before any is used); sign e of a row is bit 7 of its byte
        const auto rsg = rsrc(a.s, n);
        u32x2 sw[kHUPL][4];
#pragma unroll
        for (int u = 0; u < kHUPL; ++u) {
            const int U = 64 * u + lane, Gq = U >> 2, h = U & 3;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int i = U < kHU ? hindex(4 * Gq + t) : -1;
                const int off = i < 0 ? 0x7FFFFFF0 : 64 * i + 16 * h;
                if (u < kHUPL - 1) {
                    if (t == 0)
                        ubase[u] = off;
                } else {
                    ulast[t] = off;
                }
                sw[u][t] = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsg, i < 0 ? 0x7FFFFFF0 : i * kM2 + 8 * h, 0, 0));
            }
        }
#pragma unroll
        for (int u = 0; u < kHUPL; ++u) {
            uint32_t m = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    const int k = 4 * t + (b >> 1);
                    const uint32_t bit = (sw[u][t][b >> 2] >> (8 * (b & 3) + 7)) & 1u;
                    m |= bit << ((b & 1) ? 31 - k : 15 - k);
                }
            usg[u] = m;
        }
    }
    const int uwr = hrow(8 * (lane & 3)) + 4 * (lane >> 2);  // unit 0's first store (elements)
    // (no branch around the loads: past the last row the buffer has size 0)
    u32x4 cur[kHUPL][4];
    auto load_row = [&](int64_t r) {
        const bool ok = r < a.rows;
        const auto rs = rsrc((const uint16_t *)a.x + (ok ? r : 0) * n, ok ? 2 * n : 0);
#pragma unroll
        for (int u = 0; u < kHUPL; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                cur[u][t] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, u < kHUPL - 1 ? ubase[u] : ulast[t],
                                                                 u < kHUPL - 1 ? 64 * t : 0, 0));
    };
    // signs and transpose, in place: afterwards dwords 2v, 2v + 1 of a unit
    // (cur[u][v / 2][2 (v % 2)] ..) are row j = 8h + v at K-indices 4G .. 4G + 3
    auto prep = [&]() {
#pragma unroll
        for (int u = 0; u < kHUPL; ++u) {
            uint32_t d[16], o[16];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                d[k] = __builtin_amdgcn_bitop3_b32(usg[u] << k, cur[u][k >> 2][k & 3], 0x80008000u, 0x6C);
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const uint32_t sel = (v & 1) ? 0x07060302u : 0x05040100u;
                o[2 * v] = __builtin_amdgcn_perm(d[4 + (v >> 1)], d[v >> 1], sel);
                o[2 * v + 1] = __builtin_amdgcn_perm(d[12 + (v >> 1)], d[8 + (v >> 1)], sel);
            }
#pragma unroll
            for (int k = 0; k < 16; ++k)
                cur[u][k >> 2][k & 3] = o[k];
        }
    };
    auto put = [&]() {
#pragma unroll
        for (int u = 0; u < kHUPL; ++u) {
            if (u == kHUPL - 1 && 64 * u + lane >= kHU)
                continue;
#pragma unroll
            for (int v = 0; v < 8; ++v)
                *(u32x2 *)&xt[uwr + 64 * u + v * kHRS] =
                    (u32x2){cur[u][v >> 1][2 * (v & 1)], cur[u][v >> 1][2 * (v & 1) + 1]};
        }
    };
    const float sgn16 = (lane & 16) ? -1.0f : 1.0f, sgn32 = (lane & 32) ? -1.0f : 1.0f;
    if (row < a.rows) {
        load_row(row);
        prep();
        put();
        load_row(row + G);
    }
    lds_barrier();  // the first row is staged
    for (; row - G < a.rows; row += G) {
        const bool valid = row < a.rows;
        // ---- the helper's columns: two chains per j tile
        f32x4 xa[2][2];
        if (valid) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                xa[mt][0] = xa[mt][1] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int c = 0; c < kHK / 32; ++c)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const u32x4 av = *(const u32x4 *)&xt[hrow(16 * mt + l16) + 32 * c + 8 * rg];
                    xa[mt][c & 1] = mma<IN>(av, xo[c], xa[mt][c & 1]);
                }
        }
        // ---- codes of the row before (none in the first pass: its buffers have size 0)
        {
            const bool have = row != (int64_t)blockIdx.x;
            const int64_t pr = have ? row - G : 0;
            const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
            const RowQuant rq = row_quant(m, a.kq, qmax);
            const auto rc = rsrc((uint8_t *)a.codes + pr * (int64_t)kRowBytes, have ? kRowBytes : 0);
#pragma unroll
            for (int it = kHW - 1; it < (kBK + 63) / 64; ++it) {  // (the product waves take 0 .. 2)
                const int ip = 64 * it + lane;
                const int ipc = ip < kBK ? ip : kBK - 1;
                float v[32];
#pragma unroll
                for (int qd = 0; qd < 8; ++qd) {
                    const f32x4 w = *(const f32x4 *)&ob[ipc * kHOS + 4 * qd];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[4 * qd + r] = w[r];
                }
                if (wave_any_boost(rq)) {  // a row too small for qmax / max
#pragma unroll
                    for (int e = 0; e < 32; ++e)
                        v[e] *= rq.boost;
                }
                uint32_t f[32];
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    f[e] = __float_as_uint(__builtin_fmaf(v[e], rq.inv, kMagic));
                if constexpr (BITS == 4) {
                    u32x4 w;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        uint32_t f8[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            f8[e] = f[8 * g + e];
                        w[g] = fast::pack_int4(f8);
                    }
                    __builtin_amdgcn_raw_buffer_store_b128(w, rc, ip < kBK ? 16 * ip : kDropOffset, 0, kNonTemporal);
                } else {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        u32x4 w;
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            w[g] = fast::pack_int8(f[16 * hh + 4 * g], f[16 * hh + 4 * g + 1], f[16 * hh + 4 * g + 2],
                                                   f[16 * hh + 4 * g + 3]);
                        __builtin_amdgcn_raw_buffer_store_b128(w, rc, ip < kBK ? 32 * ip + 16 * hh : kDropOffset, 0,
                                                               kNonTemporal);
                    }
                }
            }
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(rq.scale), rsrc((float *)a.scales + pr, have ? 4 : 0),
                                                  lane == 0 ? 0 : kDropOffset, 0, 0);
        }
        if (row + G < a.rows)  // the next row (loaded one row ago): signs and transpose
            prep();
        lds_barrier();  // (1)
        if (valid) {
            // butterflies of the helper's columns (positions kept: lane (l16,
            // rg), register (mt, r) holds output j = 16 mt + 4 rg + r)
            f32x4 v[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                v[mt] = xa[mt][0] + xa[mt][1];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const float a0 = v[mt][0] + v[mt][1], a1 = v[mt][0] - v[mt][1];
                const float a2_ = v[mt][2] + v[mt][3], a3 = v[mt][2] - v[mt][3];
                v[mt][0] = a0 + a2_;
                v[mt][2] = a0 - a2_;
                v[mt][1] = a1 + a3;
                v[mt][3] = a1 - a3;
            }
            float mx = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float lo = v[0][r], hi = v[1][r];
                v[0][r] = xbutterfly<32>(xbutterfly<16>(lo + hi, sgn16), sgn32);
                v[1][r] = xbutterfly<32>(xbutterfly<16>(lo - hi, sgn16), sgn32);
                mx = fmaxf(mx, fmaxf(fabsf(v[0][r]), fabsf(v[1][r])));
            }
            mx = wave_max_nonneg(mx);
            if (lane == 0)
                red[kHW - 1] = mx;
            if (xcol >= 0) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    *(f32x4 *)&ob[xcol * kHOS + 16 * mt + 4 * rg] = v[mt];
            }
        }
        if (row + G < a.rows)  // the next row into the staged layout
            put();
        load_row(row + 2 * G);
        lds_barrier();  // (2)
    }
}

// Inverse for k = 344: y = scale * (q . H_n^T) / sqrt(n), then the signs.
// The codes are integers, exact in f16, and one scale per row commutes with
// the transform, so the codes go onto the matrix core as they are, with the
// blocks of H_k^T (block_entry<true>); the butterflies are those of the
// forward kernel (H_32 is symmetric).  No row maximum: one barrier per row,
// two staging buffers, and each lane stores its 16 (block 6: 8) consecutive
// outputs directly.
template <int BITS, int OUT>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(kBOcc))) void paley343_inv_kernel(PaleyArgs a)
{
    constexpr int n = kBK * kM2;
    constexpr int kChunks = n * BITS / 8 / 16;  // 16-byte chunks of a row's codes
    constexpr int kCPTi = (kChunks + kBThreads - 1) / kBThreads;
    constexpr int OB = OUT == kF32 ? 4 : 2;      // output bytes per element
    __shared__ __align__(16) uint16_t xt[2][kM2 * kBRS];  // [buffer][j][a2][slot]
    __shared__ unsigned char sq[kBK];
    // fp32 out: each wave's outputs pass through LDS on their way out, 64
    // bytes per lane at a stride of 80 (the 16-byte accesses of 8
    // consecutive lanes then fall in distinct banks)
    constexpr int kOst = OUT == kF32 ? kBW * 64 * 5 : 1;
    __shared__ __align__(16) u32x4 ost[kOst];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, rg = lane >> 4;
    const int lb4 = (lane >> 4) & 1, lb5 = lane >> 5;
    const int sb = 16 * wave + l16;  // this lane's column in every block

    // ---- once: zero padding, the squares, this wave's columns of H_k^T
    for (int t = tid; t < 2 * kM2 * kBRS / 8; t += kBThreads)
        ((u32x4 *)&xt[0][0])[t] = (u32x4){0u, 0u, 0u, 0u};
    for (int t = tid; t < kBK; t += kBThreads)
        sq[t] = 0;
    lds_barrier();
    for (int t = tid + 1; t < kBK - 1; t += kBThreads)
        sq[gfp_square(t, a)] = 1;  // concurrent writes store the same 1
    lds_barrier();
    u32x4 bd[kBTop][2];
#pragma unroll
    for (int d = 0; d < kBTop; ++d)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint32_t w = 0;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int v = block_entry<true>(sq, d, 32 * c + 8 * rg + 2 * p + h, sb);
                    const uint32_t bits = v == 0 ? 0u : (v > 0 ? 0x3C00u : 0xBC00u);
                    w |= bits << (16 * h);
                }
                bd[d][c][p] = w;
            }
    // the output signs of this lane, one bit per value: bits 16k .. 16k+15
    // for rows 1 + 49 (2k + lane bit 5) + sb (k < 3), bits 48 .. 55 for block
    // 6 (see the butterflies for which outputs a lane holds)
    uint32_t sgw[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < kBTop / 2; ++k) {
        const int b2 = 2 * k + lb5;
        if (sb < kBBlk || (sb == kBBlk && b2 == 0)) {
            const int ip = sb == kBBlk ? 0 : 1 + kBBlk * b2 + sb;
            for (int jj = 0; jj < 16; ++jj)
                if (a.s[ip * kM2 + 16 * lb4 + jj] < 0)
                    sgw[k >> 1] |= 1u << ((16 * k + jj) & 31);
        }
    }
    if (sb < kBBlk) {
        const int ip = 1 + kBBlk * (kBTop - 1) + sb;
        for (int jj = 0; jj < 8; ++jj)
            if (a.s[ip * kM2 + 16 * lb4 + 8 * lb5 + jj] < 0)
                sgw[1] |= 1u << (16 + jj);
    }

    // ---- codes -> f16 in the staged layout [j][block][slot] (no signs: they
    // apply to the outputs).  INT4: chunk c is row i = c (32 codes); INT8:
    // chunk c holds i = c / 2, j = 16 (c % 2) .. +15.
    // The codes of one row and its scale, loaded together and with no branch
    // around the loads (past the last row the buffers have size 0 and every
    // load reads 0), so that the waits before they are used count only these
    // loads and not the stores of the row before.  The scale comes as two
    // 16-bit halves: f16 scales are the low half alone (the high one lies
    // outside their 2-byte buffer and reads 0).
    u32x4 cur[kCPTi];
    uint32_t sc_lo = 0, sc_hi = 0;
    auto load_row = [&](int64_t row) {
        const bool ok = row < a.rows;
        const int64_t rr = ok ? row : 0;
        const auto rs = rsrc((const uint8_t *)a.codes + rr * (int64_t)(n * BITS / 8), ok ? n * BITS / 8 : 0);
#pragma unroll
        for (int cc = 0; cc < kCPTi; ++cc) {
            const int c = kBThreads * cc + tid;
            cur[cc] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rs, c < kChunks ? 16 * c : 0x7FFFFFF0, 0, kNonTemporal));
        }
        const int ssz = a.scale_f16 ? 2 : 4;
        const auto ss = rsrc((const uint8_t *)a.scales + rr * ssz, ok ? ssz : 0);
        sc_lo = __builtin_amdgcn_raw_buffer_load_b16(ss, 0, 0, 0);
        sc_hi = __builtin_amdgcn_raw_buffer_load_b16(ss, 2, 0, 0);
    };
    auto loaded_scale = [&]() {
        return a.scale_f16 ? f16_to_f32((uint16_t)sc_lo) : __uint_as_float(sc_lo | (sc_hi << 16));
    };
    auto put2 = [&](uint16_t *dst, int ja, int jb, uint32_t h2) {
        dst[ja * kBRS] = (uint16_t)h2;
        dst[jb * kBRS] = (uint16_t)(h2 >> 16);
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int cc = 0; cc < kCPTi; ++cc) {
            const int c = kBThreads * cc + tid;
            const int i = BITS == 4 ? c : c >> 1;
            const int j0 = BITS == 4 ? 0 : 16 * (c & 1);
            // (rows past the codes go to slot 448 + , which no product reads)
            const int slot = c >= kChunks ? kBTop * kBPad : (i == 0 ? kBBlk : kBPad * ((i - 1) / kBBlk) + (i - 1) % kBBlk);
            uint16_t *dst = &xt[buf][j0 * kBRS + slot];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t w = cur[cc][p];
                if constexpr (BITS == 4) {
                    // element 8p + e sits in nibble e: even e in the low
                    // nibbles of the bytes, odd e in the high ones
                    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
                    const f16x2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
                    auto cv = [&](uint32_t x) {
                        return __builtin_bit_cast(uint32_t,
                                                  __builtin_bit_cast(f16x2, (x & 0x000F000Fu) ^ 0x64086408u) + bias);
                    };
                    put2(dst, 8 * p + 0, 8 * p + 4, cv(lo));
                    put2(dst, 8 * p + 2, 8 * p + 6, cv(lo >> 8));
                    put2(dst, 8 * p + 1, 8 * p + 5, cv(hi));
                    put2(dst, 8 * p + 3, 8 * p + 7, cv(hi >> 8));
                } else {
                    const f16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
                    auto cv = [&](uint32_t x) {
                        return __builtin_bit_cast(uint32_t,
                                                  __builtin_bit_cast(f16x2, (x & 0x00FF00FFu) ^ 0x64806480u) + bias);
                    };
                    put2(dst, 4 * p + 0, 4 * p + 2, cv(w));
                    put2(dst, 4 * p + 1, 4 * p + 3, cv(w >> 8));
                }
            }
        }
    };

    const float sgn32 = (lane & 32) ? -1.0f : 1.0f;
    int64_t row = blockIdx.x;
    const int64_t G = gridDim.x;
    float sc = 0.0f;  // scale of the staged row
    if (row < a.rows) {
        load_row(row);
        stage(0);
        sc = loaded_scale();
        load_row(row + G);
    }
    lds_barrier();
    int buf = 0;
    for (; row < a.rows; row += G, buf ^= 1) {
        // ---- Z on the matrix core
        f32x4 acc[kBTop][2];
#pragma unroll
        for (int b2 = 0; b2 < kBTop; ++b2)
            acc[b2][0] = acc[b2][1] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int a2 = 0; a2 < kBTop; ++a2) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const u32x4 av = *(const u32x4 *)&xt[buf][(16 * mt + l16) * kBRS + kBPad * a2 + 32 * c + 8 * rg];
#pragma unroll
                    for (int b2 = 0; b2 < kBTop; ++b2)
                        acc[b2][mt] = mma<kF16>(av, bd[(a2 - b2 + kBTop) % kBTop][c], acc[b2][mt]);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- 32-point butterflies (as in the forward kernel)
#pragma unroll
        for (int b2 = 0; b2 < kBTop; ++b2)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const float a0 = acc[b2][mt][0] + acc[b2][mt][1], a1 = acc[b2][mt][0] - acc[b2][mt][1];
                const float a2_ = acc[b2][mt][2] + acc[b2][mt][3], a3 = acc[b2][mt][2] - acc[b2][mt][3];
                acc[b2][mt][0] = a0 + a2_;
                acc[b2][mt][2] = a0 - a2_;
                acc[b2][mt][1] = a1 + a3;
                acc[b2][mt][3] = a1 - a3;
            }
#pragma unroll
        for (int b2 = 0; b2 < kBTop; ++b2)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float lo = acc[b2][0][r], hi = acc[b2][1][r];  // bit 4
                const auto w = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo + hi), __float_as_uint(lo - hi),
                                                                false, false);  // bit 2
                const float x0 = __uint_as_float(w[0]), x1 = __uint_as_float(w[1]);
                acc[b2][0][r] = x0 + x1;
                acc[b2][1][r] = x0 - x1;
            }
#pragma unroll
        for (int k = 0; k < kBTop / 2; ++k)
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[2 * k][sl][r]),
                                                                    __float_as_uint(acc[2 * k + 1][sl][r]), false,
                                                                    false);  // bit 3
                    const float x0 = __uint_as_float(w[0]), x1 = __uint_as_float(w[1]);
                    acc[2 * k][sl][r] = x0 + x1;
                    acc[2 * k + 1][sl][r] = x0 - x1;
                }
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[kBTop - 1][sl][r] = xbutterfly<32>(acc[kBTop - 1][sl][r], sgn32);

        // ---- outputs: times scale / sqrt(n), signs, stores
        const float mul = sc * a.rb;
        const auto ry = rsrc((uint8_t *)a.y + row * (int64_t)(n * OB), n * OB);
        // value of output bit `bit` of the lane's sign words
        auto outv = [&](float v, int bit) {
            const uint32_t sw = sgw[bit >> 5];
            // ((sw << (31 - bit)) & 0x80000000) ^ v (the value in the middle
            // operand keeps the truth table independent of operand order)
            return __uint_as_float(__builtin_amdgcn_bitop3_b32(sw << (31 - (bit & 31)), __float_as_uint(v * mul),
                                                               0x80000000u, 0x6C));
        };
        // 8 consecutive outputs from element e0.  Every lane issues every
        // store, those with nothing to store (ok false) at an offset past the
        // buffer, which drops them: no branch, so the next row's loads wait
        // for loads only.
        auto store8 = [&](bool ok, int e0, const float (&o)[8]) {
            if constexpr (OUT == kF32) {
                const int off = ok ? 4 * e0 : kDropOffset;
                __builtin_amdgcn_raw_buffer_store_b128(
                    (u32x4){__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])},
                    ry, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(
                    (u32x4){__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]), __float_as_uint(o[7])},
                    ry, off + 16, 0, 0);
            } else {
                u32x4 p;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x2 f = {o[2 * q], o[2 * q + 1]};
                    p[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
                }
                __builtin_amdgcn_raw_buffer_store_b128(p, ry, ok ? 2 * e0 : kDropOffset, 0, 0);
            }
        };
        if constexpr (OUT == kF32) {
            // Whole 128-byte lines per store instruction.  Output row ip (32
            // fp32, one line) sits in two lanes (its halves, lane bit 4), so
            // a direct store writes a quarter of each of 32 lines; through
            // LDS, lane c of each group of 8 stores 16-byte chunk c of one
            // line instead (16384 x 11008: 272.0 -> 206.0 us; without any
            // stores the kernel took 167.5, so the quarter-line stores had
            // not overlapped the products at all).  Non-temporal, which
            // gains about 1 % on whole lines (on quarter lines it had taken
            // 272 to 831 us).  Stores of the padding columns' rows go past
            // the end and are dropped, as before.
            u32x4 *mine = &ost[(wave * 64) * 5];
            auto line_of = [&](int l16x, int b2) -> int {  // -1: nothing to store
                const int sbx = 16 * wave + l16x;
                if (sbx < kBBlk)
                    return 1 + kBBlk * b2 + sbx;
                return sbx == kBBlk && b2 == 0 ? 0 : -1;
            };
#pragma unroll
            for (int k = 0; k < kBTop / 2; ++k) {
                // lane (l16, lb4, lb5): half lb4 of the row of column l16
                // in block 2k + lb5, 4 chunks of 16 bytes
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl) {
                        u32x4 w;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            w[r] = __float_as_uint(outv(acc[2 * k + t][sl][r], 16 * k + 8 * t + 4 * sl + r));
                        mine[lane * 5 + 2 * t + sl] = w;
                    }
                fast::wave_lds_sync();
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // row (lb5', l16') = 8i + (lane >> 3), chunk c = lane & 7
                    const int rowx = 8 * i + (lane >> 3), c = lane & 7;
                    const int l16x = rowx & 15, lb5x = rowx >> 4;
                    const u32x4 w = mine[(l16x + 16 * (c >> 2) + 32 * lb5x) * 5 + (c & 3)];
                    const int ipx = line_of(l16x, 2 * k + lb5x);
                    __builtin_amdgcn_raw_buffer_store_b128(w, ry, ipx < 0 ? kDropOffset : 128 * ipx + 16 * c, 0,
                                                           kNonTemporal);
                }
                fast::wave_lds_sync();
            }
            {
                // block 6: lane (l16, lb4, lb5) holds quarter 2 lb4 + lb5 of
                // the row of column l16 (2 chunks)
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) {
                    u32x4 w;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        w[r] = __float_as_uint(outv(acc[kBTop - 1][sl][r], 48 + 4 * sl + r));
                    mine[lane * 5 + sl] = w;
                }
                fast::wave_lds_sync();
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int l16x = 8 * i + (lane >> 3), c = lane & 7;
                    const int qd = c >> 1;  // quarter: lb4 = qd >> 1, lb5 = qd & 1
                    const u32x4 w = mine[(l16x + 16 * (qd >> 1) + 32 * (qd & 1)) * 5 + (c & 1)];
                    const int sbx = 16 * wave + l16x;
                    const int ipx = 1 + kBBlk * (kBTop - 1) + sbx;
                    __builtin_amdgcn_raw_buffer_store_b128(w, ry, sbx < kBBlk ? 128 * ipx + 16 * c : kDropOffset,
                                                           0, kNonTemporal);
                }
                fast::wave_lds_sync();
            }
        } else {
#pragma unroll
            for (int k = 0; k < kBTop / 2; ++k) {
                const int b2 = 2 * k + lb5;
                const bool ok = sb < kBBlk || (sb == kBBlk && b2 == 0);
                const int ip = sb >= kBBlk ? 0 : 1 + kBBlk * b2 + sb;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    float o[8];
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            o[4 * sl + r] = outv(acc[2 * k + t][sl][r], 16 * k + 8 * t + 4 * sl + r);
                    store8(ok, ip * kM2 + 16 * lb4 + 8 * t, o);
                }
            }
            {
                const int ip = 1 + kBBlk * (kBTop - 1) + (sb < kBBlk ? sb : 0);
                float o[8];
#pragma unroll
                for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        o[4 * sl + r] = outv(acc[kBTop - 1][sl][r], 48 + 4 * sl + r);
                store8(sb < kBBlk, ip * kM2 + 16 * lb4 + 8 * lb5, o);
            }
        }

        // ---- the next row into the other buffer, the one after it in flight.
        // After this row's stores, not before them: the wait for the loads
        // (issued one row ago) then counts those stores as issued after the
        // loads and does not wait for them.
        if (row + G < a.rows) {
            stage(buf ^ 1);
            sc = loaded_scale();
        }
        load_row(row + 2 * G);
        lds_barrier();  // the next row is staged; nobody reads this buffer any more
    }
}

// The operand table of paley343h_kernel: a file-scope device array, one copy
// per GPU; kernels get the address hipGetSymbolAddress returns for the
// current device.  It is built on the first k = 344 forward call on a GPU by
// one small launch, which that call waits for (the one blocking step of the
// path); every later call only reads it.
static __device__ __align__(256) u32x4 hop_table[2 * kHOps * 64];
constexpr int kMaxHopDevices = 64;
struct HopSlot {
    std::once_flag once;
    hipError_t err = hipSuccess;
    u32x4 *ptr = nullptr;
};
HopSlot g_hop[kMaxHopDevices];

hipError_t paley343h_table(const PaleyArgs &pa, const u32x4 **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxHopDevices)
        return hipErrorInvalidDevice;
    HopSlot &slot = g_hop[dev];
    std::call_once(slot.once, [&]() {
        void *p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(hop_table));
        if (slot.err != hipSuccess)
            return;
        hipLaunchKernelGGL(paley343h_build, dim3(kHOps, 2), dim3(64), 0, 0, pa, (u32x4 *)p);
        slot.err = hipGetLastError();
        if (slot.err == hipSuccess)
            slot.err = hipDeviceSynchronize();
        if (slot.err == hipSuccess)
            slot.ptr = (u32x4 *)p;
    });
    if (slot.err != hipSuccess)
        return slot.err;
    *out = slot.ptr;
    return hipSuccess;
}

}  // namespace

bool paley_mfma_available(const Request &r)
{
    if (r.op == kRotate)  // k = 344 only, 16-bit input
        return r.paley.k == kBK && r.paley.p == 7 && r.paley.e == 3 && r.paley.m2 == kM2 &&
               (r.x_dtype == kBF16 || r.x_dtype == kF16);
    if (r.op == kDequantInv)  // k = 344 only, one scale per row
        return r.group == r.n && r.paley.k == kBK && r.paley.p == 7 && r.paley.e == 3 &&
               r.paley.m2 == kM2 && (r.bits == 4 || r.bits == 8) && (r.y_dtype == kF32 || r.y_dtype == kBF16);
    return r.op == kRotateQuant && !r.dst_rows && r.group == r.n &&
           (r.x_dtype == kBF16 || r.x_dtype == kF16) && r.paley.k > 1 && r.paley.m2 == kM2 &&
           r.paley.k > 320 && r.paley.k <= 352 && r.scale_dtype == kF32;
}

hipError_t launch_paley_mfma(const Request &r, const DeviceInfo &dev)
{
    PaleyArgs pa{};
    pa.x = r.x;
    pa.s = r.s;
    pa.codes = r.codes;
    pa.scales = r.scales;
    pa.rows = r.rows;
    pa.n = r.n;
    pa.k = r.paley.k;
    pa.p = r.paley.p;
    pa.e = r.paley.e;
    pa.mod0 = r.paley.mod[0];
    pa.mod1 = r.paley.mod[1];
    pa.mod2 = r.paley.mod[2];
    const int qmax = r.bits == 8 ? 127 : 7;
    pa.kq = (float)(1.0 / (__builtin_sqrt((double)r.n) * qmax));
    if (r.op == kRotate) {
        pa.y = r.y;
        pa.rb = (float)(1.0 / __builtin_sqrt((double)r.n));
        const int64_t gr = kBOcc * (int64_t)dev.cu_count;
        const int64_t grid = r.rows < gr ? r.rows : gr;
        if (r.x_dtype == kBF16)
            hipLaunchKernelGGL((paley343_kernel<kBF16>), dim3((unsigned)grid), dim3(kBThreads), 0, r.stream, pa);
        else
            hipLaunchKernelGGL((paley343_kernel<kF16>), dim3((unsigned)grid), dim3(kBThreads), 0, r.stream, pa);
        return hipGetLastError();
    }
    if (r.op == kDequantInv) {
        pa.codes = const_cast<void *>(r.codes_in);
        pa.scales = const_cast<void *>(r.scales_in);
        pa.y = r.y;
        pa.y_bf16 = r.y_dtype == kBF16;
        pa.scale_f16 = r.scale_dtype == kF16;
        pa.rb = (float)(1.0 / __builtin_sqrt((double)r.n));
        const int64_t gi = kBOcc * (int64_t)dev.cu_count;
        const int64_t grid = r.rows < gi ? r.rows : gi;
        if (r.y_dtype == kF32) {
            if (r.bits == 4)
                hipLaunchKernelGGL((paley343_inv_kernel<4, kF32>), dim3((unsigned)grid), dim3(kBThreads), 0, r.stream, pa);
            else
                hipLaunchKernelGGL((paley343_inv_kernel<8, kF32>), dim3((unsigned)grid), dim3(kBThreads), 0, r.stream, pa);
        } else {
            if (r.bits == 4)
                hipLaunchKernelGGL((paley343_inv_kernel<4, kBF16>), dim3((unsigned)grid), dim3(kBThreads), 0, r.stream, pa);
            else
                hipLaunchKernelGGL((paley343_inv_kernel<8, kBF16>), dim3((unsigned)grid), dim3(kBThreads), 0, r.stream, pa);
        }
        return hipGetLastError();
    }
    if (r.paley.k == kBK && r.paley.p == 7 && r.paley.e == 3) {
        const u32x4 *tab = nullptr;
        const hipError_t te = paley343h_table(pa, &tab);
        if (te != hipSuccess)
            return te;
        pa.hop = tab + (r.x_dtype == kBF16 ? 0 : kHOps * 64);
        const int64_t g3 = kBOcc * (int64_t)dev.cu_count;
        const int64_t grid3 = r.rows < g3 ? r.rows : g3;
        if (r.x_dtype == kBF16) {
            if (r.bits == 4)
                hipLaunchKernelGGL((paley343h_kernel<kBF16, 4>), dim3((unsigned)grid3), dim3(kHThreads), 0, r.stream, pa);
            else
                hipLaunchKernelGGL((paley343h_kernel<kBF16, 8>), dim3((unsigned)grid3), dim3(kHThreads), 0, r.stream, pa);
        } else {
            if (r.bits == 4)
                hipLaunchKernelGGL((paley343h_kernel<kF16, 4>), dim3((unsigned)grid3), dim3(kHThreads), 0, r.stream, pa);
            else
                hipLaunchKernelGGL((paley343h_kernel<kF16, 8>), dim3((unsigned)grid3), dim3(kHThreads), 0, r.stream, pa);
        }
        return hipGetLastError();
    }
    const int64_t grid = r.rows < dev.cu_count ? r.rows : dev.cu_count;
    if (r.x_dtype == kBF16) {
        if (r.bits == 4)
            hipLaunchKernelGGL((paley_mfma_kernel<11, kBF16, 4>), dim3((unsigned)grid), dim3(kThreads), 0,
                               r.stream, pa);
        else
            hipLaunchKernelGGL((paley_mfma_kernel<11, kBF16, 8>), dim3((unsigned)grid), dim3(kThreads), 0,
                               r.stream, pa);
    } else {
        if (r.bits == 4)
            hipLaunchKernelGGL((paley_mfma_kernel<11, kF16, 4>), dim3((unsigned)grid), dim3(kThreads), 0,
                               r.stream, pa);
        else
            hipLaunchKernelGGL((paley_mfma_kernel<11, kF16, 8>), dim3((unsigned)grid), dim3(kThreads), 0,
                               r.stream, pa);
    }
    return hipGetLastError();
}

}  // namespace hq
