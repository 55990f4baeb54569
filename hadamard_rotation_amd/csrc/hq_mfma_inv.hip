// hq_mfma_inv.hip -- matrix-core kernel of the inverse path (dequantise +
// inverse rotation, one scale per row) for gfx950, and its host side.
//
// Pages cited: [MS] "QuaRot：基于旋转的离群值抑制算法说明" principle section
// (the normalised Hadamard matrix is orthogonal and symmetric, so the same
// transform undoes the rotation); [RQ] "旋转量化：大模型低比特量化中的离群值克星"
// section 2.1 (H_2n = H_2 (x) H_n, so five index bits of the transform can be
// one dense 32-point product) and section 2.2 (dequantisation x = q * scale).
//
// With one scale per row the scale commutes with the transform:
//   x_hat = s * (q . H_b) * (scale / sqrt(b)),
// and q . H_b of integer codes is an integer of magnitude at most
// b * 127 < 2^24, exact in fp32 at every stage.  The codes are also exact in
// fp16, so the first five stages run as one 16x16x32 f16 product against the
// +-1 slices of H_32, like the forward kernel.  A code becomes an f16 operand
// in a byte permute and one bit operation: 0x6400 | c is 1024 + c for
// c < 1024, and c = q + 8 (INT4 nibble ^ 8) or q + 128 (INT8 byte ^ 0x80).
// The offset o = 1032 or 1152 is the same for all 32 inputs of a product, and
// the rows of H_32 other than row 0 sum to zero, so only output 0 of every
// 32-point block is shifted, by exactly 32 * o; one subtraction restores it.
// The remaining stages, the output permutation and the DPP sign tracking are
// those of the forward kernel; the per-row scale, 1/sqrt(b) and the lane's
// DPP sign form one multiplier, and the sign vector s is an XOR of the
// output sign bits (a table in LDS for rows wider than one tile).
#include "hq_mfma_impl.h"


namespace hq {
namespace mfma {

namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// OUT   output dtype (kF32 or kBF16)
// BITS  4 or 8
// T, LOGB, LOGN as in mfma_kernel
// WIDE  rows wider than one block, run as rows of one 128-block (LOGB =
//       LOGN = 7): each block row takes the scale of its real row (or its
//       own, one scale per block) and the signs of its place in the real row
// GRID  one group of T tiles per wave (group blockIdx.x * waves + wave), a
//       workgroup per few groups; otherwise persistent workgroups, one per
//       CU, with an LDS work counter and a prefetch
// GRP   one scale per group of 2^logg >= 32 elements: a lane's 8 inputs of a
//       tile lie in one 32-element chunk, hence in one group, so its scale
//       is applied to the 8 outputs of the chunk's 32-point product, which
//       are still exact integers; the later stages mix chunks of different
//       groups in fp32, as the butterflies of scaled codes would
template <int OUT, int BITS, int T, int LOGB, int LOGN, bool WIDE = false, bool GRID = false,
          bool GRP = false>
__global__ __launch_bounds__(T < 8 || (OUT == kF32 && !GRP) ? 1024 : 768) void mfma_inv_kernel(MfmaArgs a)
{
    static_assert(!WIDE || (LOGB == 7 && LOGN == 7), "wide rows run as 128-blocks");
    static_assert(!(WIDE && GRP), "wide rows carry their own scale mode");
    extern __shared__ __align__(16) u32x4 lds_osg[];   // n > 512: [tile of row][lane][2]
    constexpr int D = LOGB - 5 < 4 ? LOGB - 5 : 4;      // DPP stages (lane bits 0..D-1)
    constexpr int R = LOGB > 9 ? LOGB - 9 : 0;          // tile-bit stages
    constexpr int TPR = LOGN > 9 ? 1 << (LOGN - 9) : 1; // tiles per row
    constexpr int RPG = T / TPR;                        // rows per group (n >= 512)
    constexpr int CB = BITS == 4 ? 256 : 512;           // code bytes per tile
    constexpr int OB = OUT == kF32 ? 4 : 2;             // output bytes per element
    constexpr float kShift = 32.0f * (BITS == 4 ? 1032.0f : 1152.0f);
    // Output stores: non-temporal, except in the persistent form for fp32
    // rows of 8-tile groups, whose stores are half lines (see kFullLine):
    // there the hint cost a third of the throughput (16384 x 4096, 70 us
    // plain vs 106-115 us non-temporal).  With whole-line stores it helps
    // (grid form, 16384 x 4096 58.0 -> 55.9 us, 65536 x 1024 56.7 -> 54.5).
    constexpr int kStoreAux = (OUT == kF32 && T == 8 && !GRID) ? 0 : kNonTemporal;
    // fp32 output of whole tiles as whole 128-byte lines (see below): every
    // instance but the persistent 8-tile ones, whose 128 registers the
    // exchange would overflow
    constexpr bool kFullLine = OUT == kF32 && (GRID || T < 8);
    static_assert(T % TPR == 0, "a group holds whole rows");
    static_assert(LOGB >= 5 && LOGB <= LOGN && LOGN <= 12, "plan");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int l16 = lane & 15;
    const int lane_off = 8 * (lane >> 4) + 32 * l16;  // element offset in a tile
    const uint32_t code_byte = (uint32_t)(lane_off * BITS / 8);

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
    // fp32 output of whole tiles: lanes l and l ^ 8 trade the second halves
    // of their 32 output bytes, so that each of the two 16-byte stores of a
    // tile writes 8 whole 128-byte lines (those of the lanes with bit 3
    // clear, then those with it set) instead of half of each of 16 lines.
    // (MI355X, fp32 out: 1048576 x 128 139.5 -> 127.8 us, 131072 x 128
    // 22.6 -> 16.6, 131072 x 512 70.8 -> 64.3, 16384 x 4096 60.5 -> 58.6,
    // 16384 x 11008 in 128-blocks 186.4 -> 179.6.)
    const bool hi8 = (lane >> 3) & 1;
    int pl8 = l16 ^ 8;
    if constexpr (D > 0) {
        const int c = (int)((a.pi >> (4 * (l16 ^ 8))) & 15);
        constexpr int mask = (1 << D) - 1;
        pl8 = ((l16 ^ 8) & ~mask) | (c & mask);
    }
    const int out_off8 = 8 * (lane >> 4) + 32 * pl8;  // the partner's
    // lanes 0..15 hold transformed index 0 of their 32-point block in v[t][0]
    const float shift0 = lane < 16 ? kShift : 0.0f;
    const float rbs = lane_neg ? -a.rb : a.rb;

    // +-1 slices of H_32 in f16 (see the forward kernel)
    u32x4 amat[2];
    {
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
                    w |= (0x3C00u | (sgn << 15)) << (16 * e);
                }
                amat[h][c] = w;
            }
        }
    }

    // ---- work split (as in the forward kernel)
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
    auto group_elem0 = [&](int64_t g) {
        if constexpr (GRID)
            return g * (int64_t)(T * 512);
        else
            return ((int64_t)blockIdx.x + g * gridDim.x) * (int64_t)(T * 512);
    };

    // ---- raw input of a group: the lane's code bytes per tile and the
    // scale of each of its rows (RPG rows per group for n >= 512, else the
    // row of each tile)
    constexpr int CW = BITS == 4 ? 1 : 2;     // code words per tile
    constexpr int NS = GRP ? T : (LOGN >= 9 ? RPG : T);  // scales per lane and group
    struct Raw {
        uint32_t c[T][CW];
        uint32_t s[NS];
        u32x2 sg[WIDE ? T : 1];  // WIDE: sign bytes of the lane's 8 outputs per tile
    };
    auto load = [&](int64_t g, Raw &raw) {
        const int64_t e0 = group_elem0(g);
        const int64_t left = a.total - 8 - e0;  // >= 0 for every group
        const uint8_t *cb = (const uint8_t *)a.codes + e0 * BITS / 8;
        if (left >= T * 512) {  // wave-uniform: a full group
            const auto rs = rsrc(cb, T * CB);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                if constexpr (BITS == 4) {
                    raw.c[t][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)code_byte, t * CB,
                                                                       kNonTemporal);
                } else {
                    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)code_byte, t * CB,
                                                                         kNonTemporal);
                    raw.c[t][0] = w[0];
                    raw.c[t][1] = w[1];
                }
            }
        } else {
            const int lim = (int)left;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                int eo = t * 512 + lane_off;
                eo = eo < lim ? eo : lim;  // the ragged end reads valid memory
                if constexpr (BITS == 4) {
                    raw.c[t][0] = fast::stream_load((const uint32_t *)(cb + eo / 2));
                } else {
                    const u32x2 w = fast::stream_load((const u32x2 *)(cb + eo));
                    raw.c[t][0] = w[0];
                    raw.c[t][1] = w[1];
                }
            }
        }
        if constexpr (GRP) {
            // the scale of the group of the lane's chunk in each tile (a
            // group never straddles rows, so its index is the element
            // index >> logg), clamped into the tensor for a ragged end
            const int64_t glast = a.ngroups - 1;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                int64_t gi = (e0 + t * 512 + lane_off) >> a.logg;
                gi = gi < glast ? gi : glast;
                raw.s[t] = a.scale_f16 ? (uint32_t)((const uint16_t *)a.scales)[gi]
                                       : ((const uint32_t *)a.scales)[gi];
            }
            return;
        }
        const int64_t row_last = a.rows - 1;
        if constexpr (WIDE) {
            // the lane's block row in tile i is vr0 + 4i + (l16 >> 2) (input
            // and output positions of a lane share it), clamped to the last
            // one for a ragged end
            static_assert(!WIDE || T <= 8, "block rows vr0 .. vr0 + 31");
            const int64_t vr0 = e0 >> 7;
            const WideSplit ws = wide_split0(vr0, a.wide_div, a.wide_rdiv);
            const int64_t jl64 = row_last - vr0;
            const int jl = jl64 < 31 ? (int)jl64 : 31;
            const float rdivf = (float)a.wide_rdiv;
            // scales from row q0 (one per real row) or block row vr0 on:
            // at most 17 real rows, or 32 block rows
            const int ss = a.scale_f16 ? 2 : 4;
            const auto rs_sc = rsrc((const uint8_t *)a.scales + (a.wide_row_scale ? ws.q0 : vr0) * ss,
                                    32 * ss);
            const auto rs_sg = rsrc(a.s, a.wide_div * 128);
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                int j = 4 * i + (l16 >> 2);
                j = j < jl ? j : jl;
                int c;
                const int dq = wide_step(ws, j, a.wide_div, rdivf, c);
                const int so = (a.wide_row_scale ? dq : j) * ss;
                raw.sg[i] = __builtin_amdgcn_raw_buffer_load_b64(rs_sg, (c << 7) + (out_off & 127), 0, 0);
                raw.s[i] = a.scale_f16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs_sc, so, 0, 0)
                                       : __builtin_amdgcn_raw_buffer_load_b32(rs_sc, so, 0, 0);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            int64_t row = LOGN >= 9 ? (e0 >> LOGN) + i : (e0 + i * 512 + lane_off) >> LOGN;
            row = row < row_last ? row : row_last;
            raw.s[i] = a.scale_f16 ? (uint32_t)((const uint16_t *)a.scales)[row]
                                   : ((const uint32_t *)a.scales)[row];
        }
    };

    // ---- output signs: bit 31 of word j is the sign of output out_off + j.
    // Rows of up to 512 elements: the same 8 positions in every tile (8
    // registers); wider rows: two 16-byte words per (tile of the row, lane)
    // in LDS.
    uint32_t osg_r[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto sign_words = [&](int p, uint32_t (&w)[8]) {
        const u32x2 sb = *(const u32x2 *)(a.s + p);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            w[j] = ((sb[j >> 2] >> (8 * (j & 3) + 7)) & 1u) << 31;
    };
    if constexpr (TPR == 1 && !WIDE)
        sign_words(out_off & ((1 << LOGN) - 1), osg_r);

    Raw cur;
    load(has_work ? first : 0, cur);
    if constexpr (GRID)
        __builtin_amdgcn_sched_barrier(0);  // every load issued before the sign table

    if constexpr (TPR > 1) {
        for (int idx = threadIdx.x; idx < TPR * 64; idx += blockDim.x) {
            const int ln = idx & 63;
            const int l = ln & 15;
            int p16 = l;
            if constexpr (D > 0) {
                const int c = (int)((a.pi >> (4 * l)) & 15);
                constexpr int mask = (1 << D) - 1;
                p16 = (l & ~mask) | (c & mask);
            }
            uint32_t w[8];
            sign_words((idx >> 6) * 512 + 8 * (ln >> 4) + 32 * p16, w);
            lds_osg[2 * idx] = u32x4{w[0], w[1], w[2], w[3]};
            lds_osg[2 * idx + 1] = u32x4{w[4], w[5], w[6], w[7]};
        }
    }
    // LDS-only release: the barrier must not wait for the first loads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    // loads and stores share one completion counter: wait for the prefetch
    // right before this group's stores (see the forward kernel)
    auto take_delivery = [&](Raw &raw) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int c = 0; c < CW; ++c)
                asm volatile("" : "+v"(raw.c[t][c]));
#pragma unroll
        for (int i = 0; i < NS; ++i)
            asm volatile("" : "+v"(raw.s[i]));
        if constexpr (WIDE) {
#pragma unroll
            for (int i = 0; i < T; ++i)
                asm volatile("" : "+v"(raw.sg[i][0]), "+v"(raw.sg[i][1]));
        }
    };
    if constexpr (!GRID)
        take_delivery(cur);

    int64_t g = first;
    while (g < pool_size) {
        const int64_t g_next = grab();
        float v[T][8];
        float sc[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i)
            sc[i] = a.scale_f16 ? f16_to_f32((uint16_t)cur.s[i]) : __uint_as_float(cur.s[i]);
        // ---------------------------------- codes -> f16 + 32-point product
#pragma unroll
        for (int t = 0; t < T; ++t) {
            u32x4 b;
            if constexpr (BITS == 4) {
                // byte c of w holds codes 2c (low nibble) and 2c+1 (high)
                const uint32_t w = cur.c[t][0];
                const uint32_t w4 = w >> 4;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t sel = (uint32_t)c | (0x0Cu << 8) | ((uint32_t)(4 + c) << 16) | (0x0Cu << 24);
                    const uint32_t x = __builtin_amdgcn_perm(w4, w, sel);  // [w.b_c, 0, w4.b_c, 0]
                    b[c] = (x & 0x000F000Fu) ^ 0x64086408u;
                }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t wd = cur.c[t][c >> 1];
                    const uint32_t lo = (uint32_t)(2 * (c & 1));
                    const uint32_t sel = lo | (0x0Cu << 8) | ((lo + 1) << 16) | (0x0Cu << 24);
                    b[c] = __builtin_amdgcn_perm(0u, wd, sel) ^ 0x64806480u;
                }
            }
            const f32x4 d0 = hmma<kF16>(amat[0], b);
            const f32x4 d1 = hmma<kF16>(amat[1], b);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[t][i] = d0[i];
                v[t][4 + i] = d1[i];
            }
            if constexpr (GRP) {
                // the f16 operands' offset (index 0 of the chunk, lanes
                // 0..15), then the group's scale, while the sums are exact
                v[t][0] -= shift0;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v[t][j] *= sc[t];
            }
        }
        u32x2 sgt[WIDE ? T : 1];
        if constexpr (WIDE) {
#pragma unroll
            for (int t = 0; t < T; ++t)
                sgt[t] = cur.sg[t];
        }
        // ------------------------------------ prefetch the next tile group
        if (g_next < pool_size)  // wave-uniform
            load(g_next, cur);

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
        // the offset of the f16 operands, on index 0 of every block; placed
        // after the tile stages, which carry it only into index 0 of tile 0
        // of each block (sums of blocks' index 0 entries with signs +1)
        if constexpr (!GRP) {
#pragma unroll
            for (int t = 0; t < T; t += (1 << R))
                v[t][0] -= (float)(1 << R) * shift0;
        }

        // ------------------------------------- DPP stages (lane bits 0..D-1)
        if constexpr (D > 0) {
            // product results pass through empty asm, then 20 wait states
            // cover the matrix unit's write latency before the DPP asm
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

        if constexpr (!GRID)
            take_delivery(cur);

        // ------------------------------------------------------------ outputs
        const int64_t e0 = group_elem0(g);
        const bool full = a.total - e0 >= T * 512;  // wave-uniform
        const auto ry = rsrc((uint8_t *)a.y + e0 * OB, T * 512 * OB);
        // (the same memory cut at the tensor's end, for stores that are
        // issued by every lane and dropped past the end)
        const auto ryc = rsrc((uint8_t *)a.y + e0 * OB, (full ? T * 512 : (int)(a.total - e0)) * OB);
        int lofs = lane;
        asm volatile("" : "+v"(lofs));  // keep the sign-table reads in the loop
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float mul = GRP ? rbs : (LOGN >= 9 ? sc[t / TPR] : sc[t]) * rbs;
            uint32_t osg[8];
            if constexpr (WIDE) {
                // (the signs of this tile's block row, loaded with the codes;
                // cur was refilled by the prefetch, so they were kept aside)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    osg[j] = ((sgt[t][j >> 2] >> (8 * (j & 3) + 7)) & 1u) << 31;
            } else if constexpr (TPR > 1) {
                const u32x4 w0 = lds_osg[2 * (lofs + (t % TPR) * 64)];
                const u32x4 w1 = lds_osg[2 * (lofs + (t % TPR) * 64) + 1];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    osg[j] = w0[j];
                    osg[4 + j] = w1[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    osg[j] = osg_r[j];
            }
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                o[j] = __uint_as_float(__float_as_uint(v[t][j] * mul) ^ osg[j]);
            const bool ok = full || e0 + t * 512 + out_off < a.total;
            if constexpr (OUT == kF32) {
                const u32x4 p0 = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                                  __float_as_uint(o[3])};
                const u32x4 p1 = {__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]),
                                  __float_as_uint(o[7])};
                if constexpr (kFullLine) {
                    // No branch around these stores (a partial tile's stores
                    // past the end are dropped by the cut descriptor, the
                    // whole offset being in the checked vector operand): at
                    // a branch join the compiler once left out the wait
                    // state that a VALU write needs right after a 16-byte
                    // store of the same registers.
                    u32x4 r;  // the partner's second half (row_ror:8 within rows of 16 lanes)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        r[q] = (uint32_t)__builtin_amdgcn_mov_dpp((int)p1[q], 0x128, 0xF, 0xF, false);
                    u32x4 d0, d1;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        d0[q] = hi8 ? r[q] : p0[q];
                        d1[q] = hi8 ? p0[q] : r[q];
                    }
                    const int a0 = t * 2048 + (hi8 ? out_off8 * 4 + 16 : out_off * 4);
                    const int a1 = t * 2048 + (hi8 ? out_off * 4 : out_off8 * 4 + 16);
                    __builtin_amdgcn_raw_buffer_store_b128(d0, ryc, a0, 0, kStoreAux);
                    __builtin_amdgcn_raw_buffer_store_b128(d1, ryc, a1, 0, kStoreAux);
                    continue;
                }
                if (!ok)
                    continue;
                __builtin_amdgcn_raw_buffer_store_b128(p0, ry, out_off * 4, t * 2048, kStoreAux);
                __builtin_amdgcn_raw_buffer_store_b128(p1, ry, out_off * 4 + 16, t * 2048, kStoreAux);
            } else {
                if (!ok)
                    continue;
                u32x4 p;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x2 f = {o[2 * q], o[2 * q + 1]};
                    p[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
                }
                __builtin_amdgcn_raw_buffer_store_b128(p, ry, out_off * 2, t * 1024, kStoreAux);
            }
        }
        g = g_next;
    }
}

template <int OUT, int BITS, int T, int LOGB, int LOGN, bool WIDE = false, bool GRP = false>
hipError_t launch_inv_one(const Request &r, const DeviceInfo &dev, int wide_div = 1, int wide_row_scale = 0)
{
    MfmaArgs ma;
    fill_args(ma, r, T);
    ma.codes = const_cast<void *>(r.codes_in);
    ma.scales = const_cast<void *>(r.scales_in);
    ma.wide_div = wide_div;
    ma.wide_rdiv = 1.0 / (double)wide_div;
    ma.wide_row_scale = wide_row_scale;
    constexpr int TPR = LOGN > 9 ? 1 << (LOGN - 9) : 1;
    const size_t lds = TPR > 1 ? (size_t)TPR * 64 * 32 : 0;
    // The grid form (steady-state timings, whole-line fp32 stores):
    //  - narrow groups (2 or 4 tiles), 4 waves per workgroup: fp32 out from
    //    4 groups of 8 tiles per CU (1048576 x 128 131.2 -> 105.5 us,
    //    131072 x 128 17.2 -> 14.2, 131072 x 512 65.7 -> 52.1; with the
    //    half-line fp32 stores of before, the grid form had been the slower
    //    one here), bf16 out from 32 per CU (1048576 x 128 63.4 -> 57.7;
    //    131072 x 128 9.5 -> 10.3 us in the grid form, so it stays
    //    persistent);
    //  - 128-block rows of wide rows, from 32 per CU, 4 waves per
    //    workgroup: 16384 x 11008 fp32 out 198 -> 187 us, bf16 101.5 -> 90
    //    (one wave per workgroup, half-line stores; with whole-line stores
    //    4 waves per workgroup: 170.1 -> 166.2 us);
    //  - 8-tile groups with fp32 out, from 32 per CU, 8 waves per workgroup
    //    sharing the sign table: 16384 x 4096 64.7 -> 61.0 us, 65536 x 1024
    //    67.8 -> 58.6.  Not for bf16 out with 8-tile groups (16384 x 4096
    //    33.2 -> 38.2 us).
    constexpr bool kGridForm = WIDE || T < 8 || OUT == kF32;
    const int64_t groups8 = (ma.total + 4095) / 4096;
    const int per_cu_min = (T < 8 && !WIDE && OUT == kF32) ? kGridPerCuShort : kGridPerCuWide;
    if (kGridForm && groups8 >= (int64_t)dev.cu_count * per_cu_min) {
        const int wpb = T == 8 ? 8 : 4;
        hipLaunchKernelGGL((mfma_inv_kernel<OUT, BITS, T, LOGB, LOGN, WIDE, true, GRP>),
                           dim3((unsigned)((ma.groups + wpb - 1) / wpb)), dim3(64 * wpb), lds,
                           r.stream, ma);
        return hipGetLastError();
    }
    auto fn = mfma_inv_kernel<OUT, BITS, T, LOGB, LOGN, WIDE, false, GRP>;
    // every wave the CU holds, up to a cap per case (steady-state timings):
    // fp32 out 16 (131072 x 128: 15.6 us at 16, 17.2 at 8, with whole-line
    // stores; 16384 x 4096: 65.5 us at 16, 68.1 at 12, 74.5 at 8), 12 for
    // 8-tile groups with group scales (their launch bound); bf16 out 16 for
    // narrow groups and 12 for 8-tile groups (33.0 us at 12, 33.2 at 16)
    int waves_cu = occupancy_waves((const void *)fn, lds);
    const int cap = OUT == kF32 ? (T == 8 && GRP ? 12 : 16) : (T < 8 ? 16 : 12);
    if (waves_cu > cap)
        waves_cu = cap;
    int64_t grid = dev.cu_count;
    if (grid > ma.groups)
        grid = ma.groups;
    const int64_t per_wg = (ma.groups + grid - 1) / grid;
    if (waves_cu > per_wg)
        waves_cu = (int)per_wg;
    const int threads = 64 * waves_cu;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(threads), lds, r.stream, ma);
    return hipGetLastError();
}

template <int OUT, int BITS, int T, bool GRP>
hipError_t inv_short(const Request &r, const DeviceInfo &dev)
{
    const bool full = r.b == r.n;
    switch (r.n) {
    case 32: return launch_inv_one<OUT, BITS, T, 5, 5, false, GRP>(r, dev);
    case 64: return launch_inv_one<OUT, BITS, T, 6, 6, false, GRP>(r, dev);
    case 128: return launch_inv_one<OUT, BITS, T, 7, 7, false, GRP>(r, dev);
    case 256:
        return full ? launch_inv_one<OUT, BITS, T, 8, 8, false, GRP>(r, dev)
                    : launch_inv_one<OUT, BITS, T, 7, 8, false, GRP>(r, dev);
    default:
        return full ? launch_inv_one<OUT, BITS, T, 9, 9, false, GRP>(r, dev)
                    : launch_inv_one<OUT, BITS, T, 7, 9, false, GRP>(r, dev);
    }
}

// GRP: one scale per group of 2^logg >= 32 elements (see the kernel)
template <int OUT, int BITS, bool GRP>
hipError_t inv_dispatch(const Request &r, const DeviceInfo &dev)
{
    const bool full = r.b == r.n;
    if (r.n <= 512) {
        const int64_t groups4 = (r.rows * (int64_t)r.n + 4 * 512 - 1) / (4 * 512);
        if (groups4 < (int64_t)dev.cu_count * 8 * 4)
            return inv_short<OUT, BITS, 2, GRP>(r, dev);
        return inv_short<OUT, BITS, 4, GRP>(r, dev);
    }
    switch (r.n) {
    case 1024:
        return full ? launch_inv_one<OUT, BITS, 8, 10, 10, false, GRP>(r, dev)
                    : launch_inv_one<OUT, BITS, 8, 7, 10, false, GRP>(r, dev);
    case 2048:
        return full ? launch_inv_one<OUT, BITS, 8, 11, 11, false, GRP>(r, dev)
                    : launch_inv_one<OUT, BITS, 8, 7, 11, false, GRP>(r, dev);
    default:
        return full ? launch_inv_one<OUT, BITS, 8, 12, 12, false, GRP>(r, dev)
                    : launch_inv_one<OUT, BITS, 8, 7, 12, false, GRP>(r, dev);
    }
}

template <bool GRP>
hipError_t inv_by_type(const Request &r, const DeviceInfo &dev)
{
    if (r.y_dtype == kF32)
        return r.bits == 4 ? inv_dispatch<kF32, 4, GRP>(r, dev) : inv_dispatch<kF32, 8, GRP>(r, dev);
    return r.bits == 4 ? inv_dispatch<kBF16, 4, GRP>(r, dev) : inv_dispatch<kBF16, 8, GRP>(r, dev);
}

// Rows of several 128-blocks (see wide_inv_ok) as rows of one block.
template <int OUT, int BITS>
hipError_t inv_wide(const Request &r, const DeviceInfo &dev)
{
    const int blocks = r.n / 128;
    Request w = r;
    w.rows = r.rows * blocks;
    w.n = 128;
    w.group = 128;
    w.logg = 7;
    const int row_scale = r.group == r.n ? 1 : 0;
    const int64_t groups4 = (w.rows * 128 + 4 * 512 - 1) / (4 * 512);
    if (groups4 < (int64_t)dev.cu_count * 8 * 4)
        return launch_inv_one<OUT, BITS, 2, 7, 7, true>(w, dev, blocks, row_scale);
    return launch_inv_one<OUT, BITS, 4, 7, 7, true>(w, dev, blocks, row_scale);
}

}  // namespace

hipError_t launch_inv(const Request &r, const DeviceInfo &dev)
{
    if (wide_inv_ok(r)) {
        if (r.y_dtype == kF32)
            return r.bits == 4 ? inv_wide<kF32, 4>(r, dev) : inv_wide<kF32, 8>(r, dev);
        return r.bits == 4 ? inv_wide<kBF16, 4>(r, dev) : inv_wide<kBF16, 8>(r, dev);
    }
    return r.group == r.n ? inv_by_type<false>(r, dev) : inv_by_type<true>(r, dev);
}

}  // namespace mfma
}  // namespace hq
