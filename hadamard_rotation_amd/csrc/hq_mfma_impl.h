// hq_mfma_impl.h -- the matrix-core kernel template of libhq.so for gfx950:
// rotation (+ quantisation) of 16-bit rows with the first five butterfly
// stages of every block done as one exact 32-point product on the MFMA
// unit, the rest as in the register-resident kernel.
//
// Pages cited: [RQ] "旋转量化：大模型低比特量化中的离群值克星" section 2.1 (the
// Hadamard matrix of order 2^k is the Kronecker product of H_2 factors,
// H_2n = [[H_n, H_n], [H_n, -H_n]], so an index-bit subset of the transform
// can be done as a dense product of a smaller Hadamard matrix; blockwise
// rotation for widths that are not one block) and section 2.2 (per-row
// absmax scale, round and clip); [QT] "手把手教你用QuaRot实现LLM的4位量化：从原
// 理到代码实践" section 2.1 (signs, then Hadamard).
//
// Why a matrix unit in a memory-bound path.  The butterfly kernel needs
// about 16 VALU instructions per element for 4096-point rows, and wave64
// VALU issue (not HBM) is what limits it.  A 32-point Hadamard transform of
// 16-bit data is exact on the matrix core: every product of an input with
// +-1 is exact, and the 32-term sums are accumulated in fp32 like the
// butterflies' own adds.  One v_mfma_f32_16x16x32 on 8 inputs per lane
// replaces the widening, the sign flip (now one XOR per pair) and five
// butterfly stages, i.e. about 6.5 VALU instructions per element, with
// about one eighth of an MFMA issue slot.  Later stages stay fp32 on the
// VALU (their inputs are fp32 and the matrix core would round them).
//
// Tile layout.  The rows are viewed as one stream of 512-element tiles
// (rows of n < 512 elements pack 512/n rows per tile; rows of n >= 512
// elements are n/512 whole tiles).  In a tile, lane l (L0..L5 its bits)
// loads the 16 bytes of elements P = j + 8*(L4 + 2*L5) + 32*(l & 15),
// j = 0..7, so a wave load covers 1 KB of contiguous memory.  For the
// 16x16x32 product the tile is the B operand: k = j + 8*(l >> 4) runs over
// the element bits P0..P4, the column n = l & 15 over P5..P8.  The A
// operand is a 16-row slice of H_32 (two slices, h = 0, 1, give the 32
// outputs); output row m of slice h is the transformed index
// Q = (m & 3) + 4*h + 8*(m >> 2) in the bits P0..P4, so the lane ends up
// with 8 consecutive outputs (j' = (m & 3) + 4*h) at the same lane
// position: its codes are one 32-bit store.
//
// Block bits above P4: P5..P8 live on lane bits 0..3 and are finished with
// the DPP butterflies of the register-resident kernel (same sign tracking
// and output permutation); bits above P8 (b > 512) are tile bits and are
// finished between registers.  Rows narrower than 512 elements keep their
// row index in the high lane bits.
#pragma once

#include "hq_fast_impl.h"

namespace hq {
namespace mfma {

using fast::u32x2;
using fast::u32x4;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));


struct MfmaArgs {
    const void *x;
    const int8_t *s;
    void *codes;
    void *scales;
    void *y;
    int64_t rows;
    int64_t total;    // rows * n elements
    int64_t groups;   // groups of T tiles
    int64_t ngroups;  // scale groups: rows * n / group (rows when per row)
    int logg;         // log2 of the scale group (the kernel's run-time LOGG)
    const int64_t *dst_rows;  // append: cache row of each input row
    int64_t cache_rows;       // append: rows of the cache
    uint64_t pi;      // output chunk of lane l & 15 after the DPP stages
    uint32_t neg;     // bit l set: lane l holds the negated value
    int n;
    int bits;
    int scale_f16;
    float kq;         // 1 / (sqrt(b) * qmax)
    float rb;         // 1 / sqrt(b)
    // inverse of rows wider than one block, run as rows of one 128-block
    // (rows and n above count blocks): blocks per real row, its inverse,
    // and whether a scale belongs to a real row (else to each block)
    int wide_div;
    double wide_rdiv;
    int wide_row_scale;
};

// Rows of several 128-blocks run as rows of one block: block row vr is
// block vr mod div of real row vr div div.  A group's first block row vr0
// is divided once (the double product is within one of the quotient, one
// step corrects it); block row vr0 + j, 0 <= j < 32, then needs only the
// quotient of c0 + j < div + 32 by div, which a float product also gives
// within one (c0 + j < 2^24 + 32, and the quotient is below 17).
struct WideSplit {
    int64_t q0;  // real row of block row vr0
    int c0;      // its block in that row
};

// (vr0 is wave-uniform: the results are moved to scalar registers.)
__device__ __forceinline__ WideSplit wide_split0(int64_t vr0, int div, double rdiv)
{
    int64_t q = (int64_t)((double)vr0 * rdiv);
    const int64_t rem = vr0 - q * div;
    q += rem < 0 ? -1 : (rem >= div ? 1 : 0);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)q);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)q >> 32));
    const int c0 = __builtin_amdgcn_readfirstlane((int)(vr0 - q * div));
    return WideSplit{(int64_t)(((uint64_t)hi << 32) | lo), c0};
}

// Block row vr0 + j: returns its real row minus q0, and its block in c.
__device__ __forceinline__ int wide_step(const WideSplit &w, int j, int div, float rdivf, int &c)
{
    const int x = w.c0 + j;
    int dq = (int)((float)x * rdivf);
    c = x - dq * div;
    if (c < 0) {
        dq -= 1;
        c += div;
    } else if (c >= div) {
        dq += 1;
        c -= div;
    }
    return dq;
}

// 16x16x32 product of the +-1 slice a with the 16-bit tile b (fp32 sums).
template <int IN>
__device__ __forceinline__ f32x4 hmma(u32x4 a, u32x4 b)
{
    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (IN == kBF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), z, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), z, 0, 0, 0);
}

// Row maximum over the lanes of one row: P3, P4 (lane bits 4, 5) always,
// and lane bits 0 .. NDPP-1 (P5 ..) for rows wider than 32 elements.  The
// values are bit patterns of non-negative floats.
template <int NDPP>
__device__ __forceinline__ uint32_t row_lane_max(uint32_t v)
{
    if constexpr (NDPP > 0) v = fast::dpp_max<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (NDPP > 1) v = fast::dpp_max<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (NDPP > 2) v = fast::dpp_max<0x141>(v);  // row_half_mirror
    if constexpr (NDPP > 3) v = fast::dpp_max<0x128>(v);  // row_ror:8
    auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = r16[0] > r16[1] ? r16[0] : r16[1];
    auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return r32[0] > r32[1] ? r32[0] : r32[1];
}

// Maximum over the lanes of one scale group of 2^logg elements, 32 <= 2^logg
// <= 256, in the transposed layout below (each 16-lane row one tile).  The
// group is the set of lanes whose output chunk pl agrees above bit logg-6.
// With D >= 3 DPP stages the chunk is a linear permutation of the lane
// index, and the lanes of a group of 64 or 128 are {l, l^6} or
// {l, l^3, l^5, l^6}; otherwise they are the low lane bits.
template <int D>
__device__ __forceinline__ uint32_t group_lane_max(uint32_t v, int logg)
{
    auto xor6 = [](uint32_t x) {  // l^7^1
        const uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xf, 0xf, true);
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t, 0xB1, 0xf, 0xf, true);
    };
    auto xor5 = [](uint32_t x) {  // l^7^2
        const uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xf, 0xf, true);
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t, 0x4E, 0xf, 0xf, true);
    };
    if (logg == 8) {
        v = fast::dpp_max<0xB1>(v);
        v = fast::dpp_max<0x4E>(v);
        v = fast::dpp_max<0x141>(v);
    } else if (logg == 7) {
        if constexpr (D >= 3) {
            v = fast::dpp_max<0x1B>(v);  // quad_perm [3,2,1,0]: l^3
            const uint32_t o = xor5(v);
            v = v > o ? v : o;
        } else {
            v = fast::dpp_max<0xB1>(v);
            v = fast::dpp_max<0x4E>(v);
        }
    } else if (logg == 6) {
        if constexpr (D >= 3) {
            const uint32_t o = xor6(v);
            v = v > o ? v : o;
        } else {
            v = fast::dpp_max<0xB1>(v);
        }
    }
    return v;
}

// OP    kRotateQuant or kRotate
// IN    kBF16 or kF16
// T     tiles per wave and iteration
// LOGB  log2 b, 5..12
// LOGN  log2 n, LOGB..12
// LOGG  log2 of the scale group: LOGN (one scale per row), 9..LOGN-1 (groups
//       of whole tiles), or 0: a run-time group of 32..256 elements
//       (MfmaArgs::logg) reduced in the transposed layout
// APPEND  one scale per row, and row r's codes and scale go to cache row
//       MfmaArgs::dst_rows[r] (skipped outside [0, cache_rows))
// WIDE  rows of several 128-blocks with one scale per block, run as rows of
//       one block (LOGB = LOGN = LOGG = 7): each block row takes the signs of
//       its place in the real row (MfmaArgs::wide_div blocks per real row)
// GRID  one group of T tiles per wave and one wave per workgroup (the launch
//       has a workgroup per group); otherwise persistent workgroups, one per
//       CU, hand out groups through an LDS counter with a prefetch
template <int OP, int IN, int T, int LOGB, int LOGN, int LOGG, bool APPEND = false, bool WIDE = false,
          bool GRID = false>
__global__ __launch_bounds__(T < 8 ? 1024 : 768) void mfma_kernel(MfmaArgs a)
{
    static_assert(!WIDE || (LOGB == 7 && LOGN == 7 && LOGG == 7 && !APPEND), "wide rows run as 128-blocks");
    extern __shared__ __align__(16) u32x4 lds_mask[];  // n > 512: [tile of row][lane]
    constexpr int D = LOGB - 5 < 4 ? LOGB - 5 : 4;      // DPP stages (lane bits 0..D-1)
    constexpr int R = LOGB > 9 ? LOGB - 9 : 0;          // tile-bit stages
    constexpr int TPR = LOGN > 9 ? 1 << (LOGN - 9) : 1; // tiles per row
    static_assert(T % TPR == 0, "a group holds whole rows");
    static_assert(LOGB >= 5 && LOGB <= LOGN && LOGN <= 12, "plan");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int l16 = lane & 15;
    const int lane_off = 8 * (lane >> 4) + 32 * l16;  // element offset in a tile

    // DPP sign functionals and output permutation (as in the butterfly kernel)
    const float sig0 = ((l16 ^ (l16 >> 2)) & 1) ? -1.0f : 1.0f;
    const float sig1 = (((l16 >> 1) ^ (l16 >> 2)) & 1) ? -1.0f : 1.0f;
    const float sig2 = ((l16 >> 2) & 1) ? -1.0f : 1.0f;
    const float sig3 = ((l16 >> 3) & 1) ? -1.0f : 1.0f;
    const bool lane_neg = (a.neg >> l16) & 1;
    int pl = l16;
    if constexpr (D > 0) {
        const int c = (int)((a.pi >> (4 * l16)) & 15);
        constexpr int mask = (1 << D) - 1;
        pl = (l16 & ~mask) | (c & mask);
    }
    const int out_off = 8 * (lane >> 4) + 32 * pl;  // element offset of the 8 outputs
    // store of the 8 codes of tile t of the group at element e0: a uniform
    // tile base plus the lane's fixed byte offset; non-temporal (16384 x
    // 4096: 29.35 -> 28.85 us; 131072 x 128 10.05 -> 9.75)
    auto store_codes = [&](int64_t e0, int t, int bits, const float (&vt)[8], float inv) {
        uint32_t f[8];
        if (bits == 4) {
#pragma unroll
            for (int j = 0; j < 8; ++j)  // 1.5*2^23 + 8
                f[j] = __float_as_uint(__builtin_fmaf(vt[j], inv, 12582920.0f));
            const auto rs = rsrc((uint8_t *)a.codes + (e0 >> 1), T * 256);
            __builtin_amdgcn_raw_buffer_store_b32(fast::pack_int4(f), rs, out_off >> 1, t * 256, kNonTemporal);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)  // 1.5*2^23 + 128
                f[j] = __float_as_uint(__builtin_fmaf(vt[j], inv, 12583040.0f));
            const auto rs = rsrc((int8_t *)a.codes + e0, T * 512);
            const u32x2 pk = {fast::pack_int8(f[0], f[1], f[2], f[3]), fast::pack_int8(f[4], f[5], f[6], f[7])};
            __builtin_amdgcn_raw_buffer_store_b64(pk, rs, out_off, t * 512, kNonTemporal);
        }
    };

    // The two +-1 slices of H_32 as A operands: lane l holds row m = l & 15
    // at k = 8*(l >> 4) + j; row m of slice h is output Q(m, h).  (GRID:
    // built after the row loads are issued.)
    u32x4 amat[2];
    auto make_amat = [&]() {
        const uint32_t one = IN == kF16 ? 0x3C00u : 0x3F80u;
        const int m = l16;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = (m & 3) | (h << 2) | ((m >> 2) << 3);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                uint32_t w = 0;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int k = 8 * (lane >> 4) + 2 * c + e;
                    const uint32_t sgn = __builtin_popcount(q & k) & 1;
                    w |= (one | (sgn << 15)) << (16 * e);
                }
                amat[h][c] = w;
            }
        }
    };
    if constexpr (!GRID)
        make_amat();
    // Wide groups keep the operand in LDS and read it back for the products
    // only, so that its 8 registers are free while the butterflies and the
    // quantiser run (what lets 8-tile groups fit four waves per SIMD).
    constexpr bool kAmatInLds = T == 8 && !GRID;
    __shared__ u32x4 lds_amat[kAmatInLds ? 2 : 1][64];
    if constexpr (kAmatInLds) {
        if (wave == 0) {
            lds_amat[0][lane] = amat[0];
            lds_amat[1][lane] = amat[1];
        }
    }

    // ---- work split.  GRID: every wave takes one group of T tiles (group
    // blockIdx.x * waves + wave) and ends; the hardware dispatcher starts
    // the next workgroups as waves retire.  Otherwise one persistent
    // workgroup per CU hands out groups through an LDS counter (groups
    // strided across workgroups), with the next group prefetched.
    __shared__ int pool_next;
    const int nwaves = blockDim.x >> 6;
    int64_t pool_size, first;
    if constexpr (GRID) {
        first = (int64_t)blockIdx.x * nwaves + wave;
        pool_size = first < a.groups ? first + 1 : 0;
    } else {
        pool_size = (a.groups - blockIdx.x + gridDim.x - 1) / gridDim.x;
        first = wave;
        if (threadIdx.x == 0)
            pool_next = nwaves;
    }
    const bool has_work = first < pool_size;
    auto grab = [&]() -> int64_t {
        if constexpr (GRID) {
            return pool_size;
        } else {
            int v = 0;
            if (lane == 0)
                v = atomicAdd(&pool_next, 1);
            return __builtin_amdgcn_readfirstlane(v);
        }
    };
    // first element of group g (wave-uniform)
    auto group_elem0 = [&](int64_t g) {
        if constexpr (GRID)
            return g * (int64_t)(T * 512);
        else
            return ((int64_t)blockIdx.x + g * gridDim.x) * (int64_t)(T * 512);
    };

    // Addresses: a wave-uniform tile base (scalar registers) plus the lane's
    // 32-bit byte offset, which is the same for every tile.
    const uint32_t lane_byte = 2u * (uint32_t)lane_off;
    auto load = [&](int64_t g, u32x4 (&raw)[T]) {
        const int64_t e0 = group_elem0(g);
        if constexpr (LOGN >= 9) {
            // whole tiles: a tile past the end rereads the last one
            const int64_t last = a.total - 512;  // first element of the last tile
            const int64_t base = e0 < last ? e0 : last;
            const auto rs = rsrc((const uint16_t *)a.x + base, T * 1024);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                int64_t tb = e0 + t * 512;
                tb = tb < last ? tb : last;
                const int sofs = (int)(2 * (tb - base));  // wave-uniform
                raw[t] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)lane_byte, sofs, kNonTemporal);
            }
        } else {
            const int64_t left = a.total - 8 - e0;  // >= 0 for every group
            if (left >= T * 512) {  // wave-uniform: a full group
                const auto rs = rsrc((const uint16_t *)a.x + e0, T * 1024);
#pragma unroll
                for (int t = 0; t < T; ++t)
                    raw[t] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)lane_byte, t * 1024,
                                                                   kNonTemporal);
            } else {
                const int lim = (int)left;
                const uint16_t *gp = (const uint16_t *)a.x + e0;
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    int eo = t * 512 + lane_off;
                    eo = eo < lim ? eo : lim;  // the ragged end reads valid memory
                    raw[t] = fast::stream_load((const u32x4 *)(gp + eo));
                }
            }
        }
    };

    // ---- sign masks (bit 15 of each 16-bit element).  Rows of up to 512
    // elements: the lane's 8 row positions are the same in every tile, so
    // the masks live in 4 registers.  Wider rows: GRID loads the lane's 8
    // sign bytes of every tile of the row (cache hits: s is n bytes) and
    // turns them into masks as each tile is used; the persistent kernel
    // builds one 16-byte mask per (tile of the row, lane) in LDS once.
    u32x4 smask = {0, 0, 0, 0};
    if constexpr (TPR == 1) {
        const int p = lane_off & ((1 << LOGN) - 1);
        const u32x2 sb = *(const u32x2 *)(a.s + p);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t w = sb[c >> 1] >> (16 * (c & 1));
            smask[c] = ((w >> 7) & 1) << 15 | ((w >> 15) & 1) << 31;
        }
    }

    // Wider rows: the sign bytes (the lane's own, or this thread's entries of
    // the mask table), requested before the rows, so that waiting for them
    // leaves the rows' loads in flight
    u32x2 tsb[TPR > 1 ? TPR : 1];
    constexpr bool kLaneSigns = GRID && TPR > 1;
    if constexpr (kLaneSigns) {
        // the lane's own 8 sign bytes of every tile of the row
#pragma unroll
        for (int i = 0; i < TPR; ++i)
            tsb[i] = *(const u32x2 *)(a.s + i * 512 + lane_off);
    } else if constexpr (TPR > 1) {
#pragma unroll
        for (int i = 0; i < TPR; ++i) {
            const int idx = threadIdx.x + i * (int)blockDim.x;
            if (idx < TPR * 64) {
                const int ln = idx & 63;
                const int p = (idx >> 6) * 512 + 8 * (ln >> 4) + 32 * (ln & 15);
                tsb[i] = *(const u32x2 *)(a.s + p);
            }
        }
    }

    // WIDE: the sign bytes of the lane's 8 inputs of each tile, loaded with
    // the tile; the lane's block row in tile t is vr0 + 4t + (l16 >> 2),
    // clamped to the last one for a ragged end
    u32x2 csg[WIDE ? T : 1];
    auto load_signs = [&](int64_t g) {
        if constexpr (WIDE) {
            static_assert(!WIDE || T <= 8, "block rows vr0 .. vr0 + 31");
            const int64_t vr0 = group_elem0(g) >> 7;
            const WideSplit ws = wide_split0(vr0, a.wide_div, a.wide_rdiv);
            const int64_t jl64 = a.rows - 1 - vr0;
            const int jl = jl64 < 31 ? (int)jl64 : 31;
            const float rdivf = (float)a.wide_rdiv;
            const auto rs_sg = rsrc(a.s, a.wide_div * 128);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                int j = 4 * t + (l16 >> 2);
                j = j < jl ? j : jl;
                int c;
                wide_step(ws, j, a.wide_div, rdivf, c);
                csg[t] = __builtin_amdgcn_raw_buffer_load_b64(rs_sg, (c << 7) + (lane_off & 127), 0, 0);
            }
        }
    };
    if constexpr (GRID)
        load_signs(has_work ? first : 0);

    u32x4 cur[T];
    load(has_work ? first : 0, cur);
    if constexpr (GRID) {
        // every row load is issued before anything waits for the sign loads
        // (left alone, the scheduler interleaves the mask arithmetic with the
        // loads and waits for the signs with most of the row not yet
        // requested)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (OP == kRotate && LOGN == 7) {
            // The rotation alone of 128-element rows writes fp32, four
            // bytes out per two in; spacing the waves' requests out helps
            // it (1048576 x 128 138.4 -> 133.7 us, 131072 x 128 18.7 ->
            // 18.2 with 512 cycles here; wider rows and the quantising
            // kernels gained nothing or lost a little)
            __builtin_amdgcn_s_sleep(8);
            __builtin_amdgcn_sched_barrier(0);
        }
        make_amat();
    } else {
        load_signs(has_work ? first : 0);
    }

    if constexpr (TPR > 1 && !kLaneSigns) {
#pragma unroll
        for (int i = 0; i < TPR; ++i) {
            const int idx = threadIdx.x + i * (int)blockDim.x;
            if (idx >= TPR * 64)
                break;
            const u32x2 sb = tsb[i];
            u32x4 m;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t w = sb[c >> 1] >> (16 * (c & 1));
                m[c] = ((w >> 7) & 1) << 15 | ((w >> 15) & 1) << 31;
            }
            lds_mask[idx] = m;
        }
    }
    // LDS-only release: the barrier must not wait for the row loads
    if constexpr (!GRID)
        lds_barrier();

    // Loads and stores share one completion counter; this empty asm fixes
    // where the wait for a prefetch happens (see the butterfly kernel).
    auto take_delivery = [&](u32x4 (&raw)[T]) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                asm volatile("" : "+v"(raw[t][c]));
        if constexpr (WIDE) {
#pragma unroll
            for (int t = 0; t < T; ++t)
                asm volatile("" : "+v"(csg[t][0]), "+v"(csg[t][1]));
        }
    };
    if constexpr (!GRID)
        take_delivery(cur);

    int64_t g = first;
    while (g < pool_size) {
        const int64_t g_next = grab();
        float v[T][8];
        // ------------------------------------------ signs + 32-point product
        // One lane index per iteration, passed through an empty asm so that
        // the (row-independent) LDS reads stay in the loop; every tile's read
        // is then an immediate offset from it.
        int lofs = lane;
        asm volatile("" : "+v"(lofs));
        u32x4 am0 = amat[0], am1 = amat[1];
        if constexpr (kAmatInLds) {
            am0 = lds_amat[0][lofs];
            am1 = lds_amat[1][lofs];
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            u32x4 m = smask;
            if constexpr (TPR > 1)
            {
                if constexpr (kLaneSigns) {
                    const u32x2 sb = tsb[t % TPR];
#pragma unroll
                    for (int c = 0; c < 4; ++c)  // sign bits of bytes 2c, 2c+1 to bits 15, 31
                        m[c] = __builtin_amdgcn_perm(0u, sb[c >> 1], (c & 1) ? 0x030c020cu : 0x010c000cu) &
                               0x80008000u;
                } else {
                    m = lds_mask[lofs + (t % TPR) * 64];
                }
            }
            if constexpr (WIDE) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t w = csg[t][c >> 1] >> (16 * (c & 1));
                    m[c] = ((w >> 7) & 1) << 15 | ((w >> 15) & 1) << 31;
                }
            }
            u32x4 b;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                b[c] = cur[t][c] ^ m[c];
            const f32x4 d0 = hmma<IN>(am0, b);
            const f32x4 d1 = hmma<IN>(am1, b);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[t][i] = d0[i];
                v[t][4 + i] = d1[i];
            }
        }
        // ------------------------------------ prefetch the next tile group
        if (g_next < pool_size) {  // wave-uniform
            load(g_next, cur);
            load_signs(g_next);
        }

        // ------------------------------------------ tile-bit stages (b > 512)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t) {
                if ((t >> r) & 1)
                    continue;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    fast::bfly(v[t][j], v[t + (1 << r)][j]);
            }

        // ------------------------------------- DPP stages (lane bits 0..D-1)
        if constexpr (D > 0) {
            // The DPP blocks are inline asm, which the compiler does not pad
            // against the matrix unit's write latency.  Every product result
            // is first passed through an empty asm (in program order), then
            // 20 wait states cover the longest MFMA-write -> VALU hazard.
            if constexpr (R == 0) {
#pragma unroll
                for (int t = 0; t < T; ++t)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        asm volatile("" : "+v"(v[t][j]));
                asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::);
            }
#pragma unroll
            for (int t = 0; t < T; ++t)
                fast::dpp_stages<D>(v[t], sig0, sig1, sig2, sig3);
        }

        // Take delivery of the prefetched group before this group's stores.
        if constexpr (!GRID)
            take_delivery(cur);

        // ------------------------------------------------------------ outputs
        const int64_t e0 = group_elem0(g);
        if constexpr (OP == kRotate) {
            const float mul = lane_neg ? -a.rb : a.rb;
            // Whole tiles: lanes l and l ^ 8 trade the second halves of
            // their 32 output bytes, so that each of a tile's two 16-byte
            // stores writes 8 whole 128-byte lines (those of the lanes with
            // bit 3 clear, then those with it set), not half of each of 16
            // lines.  The partner's output offset follows from its lane
            // index as out_off does.
            // No branch around the stores: past the tensor's end they are
            // dropped by a descriptor cut there (the whole offset in the
            // checked vector operand).  At a branch join the compiler once
            // left out the wait state that a VALU write needs right after a
            // 16-byte store of the same registers.
            const int64_t left = a.total - e0;
            const auto ry = rsrc((float *)a.y + e0, (int)(left < T * 512 ? left : T * 512) * 4);
            const bool hi8 = (lane >> 3) & 1;
            int pl8 = l16 ^ 8;
            if constexpr (D > 0) {
                const int c = (int)((a.pi >> (4 * (l16 ^ 8))) & 15);
                constexpr int mask = (1 << D) - 1;
                pl8 = ((l16 ^ 8) & ~mask) | (c & mask);
            }
            const int out_off8 = 8 * (lane >> 4) + 32 * pl8;
            const int s0 = 4 * (hi8 ? out_off8 + 4 : out_off);  // byte offsets of the two stores
            const int s1 = 4 * (hi8 ? out_off : out_off8 + 4);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                u32x4 p0, p1;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    p0[q] = __float_as_uint(v[t][q] * mul);
                    p1[q] = __float_as_uint(v[t][4 + q] * mul);
                }
                u32x4 r, d0, d1;  // r: the partner's second half (row_ror:8 in rows of 16 lanes)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    r[q] = (uint32_t)__builtin_amdgcn_mov_dpp((int)p1[q], 0x128, 0xF, 0xF, false);
                    d0[q] = hi8 ? r[q] : p0[q];
                    d1[q] = hi8 ? p0[q] : r[q];
                }
                // (non-temporal: 1048576 x 128 148.2 -> 140.8 us, 16384 x 4096
                // 72.3 -> 69.1, 16384 x 11008 in 128-blocks 186.7 -> 180.0)
                __builtin_amdgcn_raw_buffer_store_b128(d0, ry, t * 2048 + s0, 0, kNonTemporal);
                __builtin_amdgcn_raw_buffer_store_b128(d1, ry, t * 2048 + s1, 0, kNonTemporal);
            }
        } else if constexpr (LOGG == 0) {
            // ---- scale groups of 32..256 elements: each lies in one tile.
            // Transposed reduction: permlane16_swap of the chunk maxima of
            // tiles (2p, 2p+1) reduces lane bit 4 of both at once and leaves
            // rows [2p, 2p+1, 2p, 2p+1]; permlane32_swap of two such
            // registers reduces lane bit 5 and leaves one tile per 16-lane
            // row.  The in-row DPP steps, the reciprocal and the scale
            // stores then run once per four tiles, and the same swaps in
            // reverse hand every lane its group's multiplier.
            const int qmax = a.bits == 4 ? 7 : 127;
            const int logg = a.logg;
            uint32_t mt[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                float m = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; j += 2)
                    m = fmaxf(fmaxf(m, fabsf(v[t][j])), fabsf(v[t][j + 1]));
                mt[t] = __float_as_uint(m);
            }
            constexpr int NX = T / 2;
            constexpr int NZ = T >= 4 ? T / 4 : 1;
            uint32_t x[NX], z[NZ];
#pragma unroll
            for (int p = 0; p < NX; ++p) {
                const auto r = __builtin_amdgcn_permlane16_swap(mt[2 * p], mt[2 * p + 1], false, false);
                x[p] = r[0] > r[1] ? r[0] : r[1];
            }
#pragma unroll
            for (int q = 0; q < NZ; ++q) {
                const auto r = __builtin_amdgcn_permlane32_swap(x[T >= 4 ? 2 * q : 0],
                                                                x[T >= 4 ? 2 * q + 1 : 0], false, false);
                z[q] = r[0] > r[1] ? r[0] : r[1];
            }
            // z[q], row rho: tile 4q + rho (T >= 4) or rho & 1 (T == 2)
            const int rho = lane >> 4;
            const bool rep_lane = (pl & ((1 << (logg - 5)) - 1)) == 0 && (T >= 4 || rho < 2);
            float iz[NZ], bz[NZ];
            bool boosted = false;
#pragma unroll
            for (int q = 0; q < NZ; ++q) {
                const uint32_t mb = group_lane_max<D>(z[q], logg);
                const RowQuant rq = row_quant(__uint_as_float(mb), a.kq, qmax);
                bz[q] = rq.boost;
                boosted |= rq.boost != 1.0f;
                const int t = T >= 4 ? 4 * q + rho : (rho & 1);
                const int64_t gi = (e0 + t * 512 + 32 * pl) >> logg;
                if (rep_lane && gi < a.ngroups) {
                    if (a.scale_f16)
                        ((uint16_t *)a.scales)[gi] = f32_to_f16(rq.scale);
                    else
                        ((float *)a.scales)[gi] = rq.scale;
                }
                iz[q] = lane_neg ? -rq.inv : rq.inv;
            }
            // un-transpose: a value per tile at every lane of the tile
            auto untranspose = [&](const float (&zv)[NZ], float (&out)[T]) {
                if constexpr (T >= 4) {
#pragma unroll
                    for (int q = 0; q < NZ; ++q) {
                        const uint32_t zi = __float_as_uint(zv[q]);
                        const auto w = __builtin_amdgcn_permlane32_swap(zi, zi, false, false);
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const auto u = __builtin_amdgcn_permlane16_swap(w[h], w[h], false, false);
                            out[4 * q + 2 * h] = __uint_as_float(u[0]);
                            out[4 * q + 2 * h + 1] = __uint_as_float(u[1]);
                        }
                    }
                } else {
                    const uint32_t zi = __float_as_uint(zv[0]);
                    const auto u = __builtin_amdgcn_permlane16_swap(zi, zi, false, false);
                    out[0] = __uint_as_float(u[0]);
                    out[1] = __uint_as_float(u[1]);
                }
            };
            float inv[T];
            untranspose(iz, inv);
            // groups too small for qmax / max: magnify their values exactly
            if (__builtin_amdgcn_ballot_w64(boosted) != 0) {
                float boost[T];
                untranspose(bz, boost);
#pragma unroll
                for (int t = 0; t < T; ++t)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        v[t][j] *= boost[t];
            }
            const int bits = a.bits;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                if (e0 + t * 512 + out_off >= a.total)
                    continue;
                store_codes(e0, t, bits, v[t], inv[t]);
            }
        } else {
            // ---- one scale per row (LOGG == LOGN) or per group of whole
            // tiles (9 <= LOGG < LOGN): TPG tiles of a group are reduced in
            // registers, then over the group's lanes
            constexpr int TPG = LOGG > 9 ? 1 << (LOGG - 9) : 1;  // tiles per group
            static_assert(T % TPG == 0, "a tile group holds whole scale groups");
            const int qmax = a.bits == 4 ? 7 : 127;
#pragma unroll
            for (int rr = 0; rr < T / TPG; ++rr) {
                // tiles t0 .. t0+TPG-1 hold 512/n rows (TPG == 1) or one group
                const int t0 = rr * TPG;
                float m = 0.0f;
#pragma unroll
                for (int t = t0; t < t0 + TPG; ++t)
#pragma unroll
                    for (int j = 0; j < 8; j += 2)
                        m = fmaxf(fmaxf(m, fabsf(v[t][j])), fabsf(v[t][j + 1]));
                constexpr int NDPP = LOGG - 5 < 4 ? LOGG - 5 : 4;
                const uint32_t mb = row_lane_max<NDPP>(__float_as_uint(m));
                const RowQuant rq = row_quant(__uint_as_float(mb), a.kq, qmax);
                if (wave_any_boost(rq)) {  // rows too small for qmax / max
#pragma unroll
                    for (int t = t0; t < t0 + TPG; ++t)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            v[t][j] *= rq.boost;
                }
                // the lane's group: first element of its outputs >> LOGG
                const int64_t grp = (e0 + t0 * 512 + out_off) >> LOGG;
                bool grp_ok = grp < a.ngroups;
                int64_t orow = grp;  // where the group's scale goes
                if constexpr (APPEND) {
                    orow = grp_ok ? a.dst_rows[grp] : -1;
                    grp_ok = grp_ok && orow >= 0 && orow < a.cache_rows;
                }
                // one lane per group writes the scale: lane bits 4, 5 and the
                // group-internal low lane bits all zero
                constexpr int grp_lanes_mask = (1 << NDPP) - 1;
                if (grp_ok && lane < 16 && (l16 & grp_lanes_mask) == 0) {
                    if (a.scale_f16)
                        ((uint16_t *)a.scales)[orow] = f32_to_f16(rq.scale);
                    else
                        ((float *)a.scales)[orow] = rq.scale;
                }
                const float inv = lane_neg ? -rq.inv : rq.inv;
                if (grp_ok) {
                    const int bits = a.bits;
#pragma unroll
                    for (int t = t0; t < t0 + TPG; ++t) {
                        if constexpr (APPEND) {
                            // the lane's 8 codes at their place in cache row orow
                            const int in_row = (int)((e0 + t * 512 + out_off) & ((1 << LOGN) - 1));
                            uint32_t f[8];
                            if (bits == 4) {
#pragma unroll
                                for (int j = 0; j < 8; ++j)  // 1.5*2^23 + 8
                                    f[j] = __float_as_uint(__builtin_fmaf(v[t][j], inv, 12582920.0f));
                                uint8_t *dst = (uint8_t *)a.codes + orow * (int64_t)(a.n >> 1);
                                *(uint32_t *)(dst + (in_row >> 1)) = fast::pack_int4(f);
                            } else {
#pragma unroll
                                for (int j = 0; j < 8; ++j)  // 1.5*2^23 + 128
                                    f[j] = __float_as_uint(__builtin_fmaf(v[t][j], inv, 12583040.0f));
                                int8_t *dst = (int8_t *)a.codes + orow * (int64_t)a.n;
                                *(uint2 *)(dst + in_row) =
                                    make_uint2(fast::pack_int8(f[0], f[1], f[2], f[3]),
                                               fast::pack_int8(f[4], f[5], f[6], f[7]));
                            }
                        } else {
                            store_codes(e0, t, bits, v[t], inv);
                        }
                    }
                }
            }
        }
        g = g_next;
    }
}

}  // namespace mfma
}  // namespace hq

namespace hq {
namespace mfma {

// Host side (hq_mfma.hip): plan check, argument setup and the launch.
bool plan_ok(const Request &r);
bool wide_inv_ok(const Request &r);
bool wide_fwd_ok(const Request &r);
bool long_fwd_ok(const Request &r);
void fill_args(MfmaArgs &ma, const Request &r, int tiles_per_group);
int occupancy_waves(const void *fn, size_t lds);

// Launches with at least this many 4096-element groups per CU take the grid
// form of the kernel (one group of tiles per single-wave workgroup; rows of
// up to 512 elements in groups of 4 tiles, wider rows in groups of 8);
// smaller ones the persistent form.  Measured on MI355X (steady state, us
// per launch, persistent -> grid):
//   16384 x 4096 (64 per CU)       31.6 -> 29.5   (8-tile groups)
//   65536 x 1024 (64 per CU)       31.4 -> 28.8   (8-tile groups)
//   1048576 x 128 (128 per CU)     55.6 -> 55.0   (4-tile groups)
//   131072 x 512 (64 per CU)       29.5 -> 28.4   (4-tile groups)
//   131072 x 128 (16 per CU)       10.0 ->  9.8   (4-tile groups; 10.9 with 8)
// In the grid form the dispatcher starts workgroups on whichever CU frees
// first and a wave holds one group of loads, not two.  Wide rows keep the
// persistent form below 32 per CU (not measured there).
constexpr int kGridPerCuShort = 4;
constexpr int kGridPerCuWide = 32;

inline bool grid_launch(const Request &r, const DeviceInfo &dev)
{
    const int64_t groups = (r.rows * (int64_t)r.n + 8 * 512 - 1) / (8 * 512);
    const int per_cu = r.n <= 512 ? kGridPerCuShort : kGridPerCuWide;
    return r.dst_rows == nullptr && groups >= (int64_t)dev.cu_count * per_cu;
}

template <int OP, int IN, int T, int LOGB, int LOGN, int LOGG, bool APPEND = false, bool WIDE = false,
          bool GRID = false>
hipError_t launch_one(const Request &r, const DeviceInfo &dev, int wide_div = 1)
{
    MfmaArgs ma;
    fill_args(ma, r, T);
    ma.wide_div = wide_div;
    ma.wide_rdiv = 1.0 / (double)wide_div;
    ma.wide_row_scale = 0;
    auto fn = mfma_kernel<OP, IN, T, LOGB, LOGN, LOGG, APPEND, WIDE, GRID>;
    if constexpr (GRID) {
        // one group per single-wave workgroup; no LDS (the signs of wide
        // rows are per lane)
        hipLaunchKernelGGL(fn, dim3((unsigned)ma.groups), dim3(64), 0, r.stream, ma);
        return hipGetLastError();
    }
    constexpr int TPR = LOGN > 9 ? 1 << (LOGN - 9) : 1;
    const size_t lds = TPR > 1 ? (size_t)TPR * 64 * 16 : 0;
    // One workgroup per CU with every wave the CU can hold, at most 16 for
    // groups of 2 tiles and 12 otherwise (steady-state timings: 131072 x 128
    // rows 9.8 us with 16 waves, 10.4 with 12; 1048576 x 128 rows, groups of
    // 4 tiles, 54.6 us with 12, 55.1 with 16; 16384 x 4096, 8 tiles, 31.3 us
    // with 12, 31.7 with 16, 31.8 with 8).
    const int max_threads = T == 2 ? 1024 : 768;
    int waves_cu = occupancy_waves((const void *)fn, lds);
    if (waves_cu > max_threads / 64)
        waves_cu = max_threads / 64;
    int64_t grid = dev.cu_count;
    if (grid > ma.groups)
        grid = ma.groups;
    // small launches (a decode step's few rows): no more waves per
    // workgroup than it has groups of tiles
    const int64_t per_wg = (ma.groups + grid - 1) / grid;
    if (waves_cu > per_wg)
        waves_cu = (int)per_wg;
    const int threads = 64 * waves_cu;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(threads), lds, r.stream, ma);
    return hipGetLastError();
}

// Launch modes of the forward kernels: one scale per row, group-wise scales,
// or rows appended into a cache.
enum Mode : int { kPerRow = 0, kGrouped = 1, kAppend = 2 };

// The scale grouping of a (T, LOGB, LOGN) plan: one scale per row, or
// (kGrouped, forward only) a run-time group of 32..256 elements, or whole-tile
// groups of 512 .. n/2 elements; kAppend: one scale per row, written to the
// cache rows the caller names.
template <int OP, int IN, int MODE, int T, int LOGB, int LOGN, bool GRID>
hipError_t launch_g(const Request &r, const DeviceInfo &dev)
{
    if constexpr (MODE == kAppend && OP == kRotateQuant) {
        return launch_one<OP, IN, T, LOGB, LOGN, LOGN, true, false, false>(r, dev);
    } else if constexpr (MODE == kGrouped && OP == kRotateQuant) {
        if (r.logg < 9)
            return launch_one<OP, IN, T, LOGB, LOGN, 0, false, false, GRID>(r, dev);
        if constexpr (LOGN > 9)
            if (r.logg == 9) return launch_one<OP, IN, T, LOGB, LOGN, 9, false, false, GRID>(r, dev);
        if constexpr (LOGN > 10)
            if (r.logg == 10) return launch_one<OP, IN, T, LOGB, LOGN, 10, false, false, GRID>(r, dev);
        if constexpr (LOGN > 11)
            if (r.logg == 11) return launch_one<OP, IN, T, LOGB, LOGN, 11, false, false, GRID>(r, dev);
        return hipErrorInvalidValue;
    } else {
        return launch_one<OP, IN, T, LOGB, LOGN, LOGN, false, false, GRID>(r, dev);
    }
}

// Grid or persistent form of a (T, LOGB, LOGN) plan (appends are always
// persistent: a decode step's few rows).
template <int OP, int IN, int MODE, int T, int LOGB, int LOGN>
hipError_t launch_gp(const Request &r, const DeviceInfo &dev, bool grid)
{
    if constexpr (MODE != kAppend && T == 8)
        if (grid)
            return launch_g<OP, IN, MODE, T, LOGB, LOGN, true>(r, dev);
    return launch_g<OP, IN, MODE, T, LOGB, LOGN, false>(r, dev);
}

// Full rotations of n = 32..4096 and 128-blocks of n = 256..4096.
// Rows of up to 512 elements take groups of 4 tiles in the grid form; in the
// persistent form groups of 4 tiles, or of 2 tiles when that would leave
// fewer than 4 groups per wave (the last round of groups then idles less of
// the machine; measured on 131072 x 128).
template <int OP, int IN, int MODE, int T, bool GRID>
hipError_t dispatch_short(const Request &r, const DeviceInfo &dev)
{
    const bool full = r.b == r.n;
    switch (r.n) {
    case 32: return launch_g<OP, IN, MODE, T, 5, 5, GRID>(r, dev);
    case 64: return launch_g<OP, IN, MODE, T, 6, 6, GRID>(r, dev);
    case 128: return launch_g<OP, IN, MODE, T, 7, 7, GRID>(r, dev);
    case 256:
        return full ? launch_g<OP, IN, MODE, T, 8, 8, GRID>(r, dev)
                    : launch_g<OP, IN, MODE, T, 7, 8, GRID>(r, dev);
    default:
        return full ? launch_g<OP, IN, MODE, T, 9, 9, GRID>(r, dev)
                    : launch_g<OP, IN, MODE, T, 7, 9, GRID>(r, dev);
    }
}

template <int OP, int IN, int MODE>
hipError_t dispatch_op(const Request &r, const DeviceInfo &dev)
{
    const bool full = r.b == r.n;
    const bool grid = MODE != kAppend && grid_launch(r, dev);
    if (r.n <= 512) {
        if constexpr (MODE != kAppend)
            if (grid)
                return dispatch_short<OP, IN, MODE, 4, true>(r, dev);
        const int64_t groups4 = (r.rows * (int64_t)r.n + 4 * 512 - 1) / (4 * 512);
        if (groups4 < (int64_t)dev.cu_count * 16 * 4)
            return dispatch_short<OP, IN, MODE, 2, false>(r, dev);
        return dispatch_short<OP, IN, MODE, 4, false>(r, dev);
    }
    switch (r.n) {
    case 1024:
        return full ? launch_gp<OP, IN, MODE, 8, 10, 10>(r, dev, grid)
                    : launch_gp<OP, IN, MODE, 8, 7, 10>(r, dev, grid);
    case 2048:
        return full ? launch_gp<OP, IN, MODE, 8, 11, 11>(r, dev, grid)
                    : launch_gp<OP, IN, MODE, 8, 7, 11>(r, dev, grid);
    default:
        return full ? launch_gp<OP, IN, MODE, 8, 12, 12>(r, dev, grid)
                    : launch_gp<OP, IN, MODE, 8, 7, 12>(r, dev, grid);
    }
}

}  // namespace mfma
}  // namespace hq
