// hq_device.h -- device-side numeric helpers shared by every kernel of
// libhq.so.  All arithmetic is IEEE binary32; the library is compiled with
// -ffp-contract=off so that every fused multiply-add below is explicit.
//
// Pages cited: [RQ] "旋转量化：大模型低比特量化中的离群值克星" section 2.2
// (symmetric absmax quantisation with round-to-nearest and clipping to
// +-(2^(bits-1)-1)); [HQA] "哈特曼旋转，轻量级QAT，流式注意力" section 1 (scale
// = max|x| / qmax).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>

namespace hq {

// Buffer resource over `bytes` bytes at the wave-uniform address p (raw
// buffer, 32-bit elements; dword 3 as every gfx9 target wants it).  The
// base lives in scalar registers, so the lane's offset is the only vector
// part of an address; a load whose lane offset is at or past `bytes` returns
// 0 without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}
constexpr int kNonTemporal = 2;  // buffer cache-policy bit: nt

// Workgroup barrier for LDS traffic only.  __syncthreads() also orders
// global memory, which makes every wave wait for all of its loads and
// stores in flight first (prefetched rows, earlier rows' stores).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 1.5 * 2^23: adding it to a value v with |v| < 2^22 leaves round_half_even(v)
// in the low mantissa bits, because the sum's unit in the last place is 1.
constexpr float kRoundMagic = 12582912.0f;
constexpr int kRoundMagicBits = 0x4B400000;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h)
{
    return __half2float(__ushort_as_half(h));
}

__device__ __forceinline__ uint16_t f32_to_f16(float f)
{
    return __half_as_ushort(__float2half_rn(f));
}

// Quantisation code of an unnormalised rotated value y, given
// inv = qmax / max|y| of its row: round_half_even(y * inv) with the product
// kept exact inside one fma, clamped to [-qmax, qmax].  (y * inv equals
// x'/scale because the 1/sqrt(b) normalisation cancels.)
__device__ __forceinline__ int quant_code(float y, float inv, int qmax)
{
    float t = __builtin_fmaf(y, inv, kRoundMagic);
    int q = (int)__float_as_uint(t) - kRoundMagicBits;
    q = q > qmax ? qmax : q;
    q = q < -qmax ? -qmax : q;
    return q;
}

// Per-row constants of the quantiser.  m = max|y| over the row (unnormalised
// rotated values); kq = 1 / (sqrt(b) * qmax) rounded to fp32 on the host.
struct RowQuant {
    float inv;    // qmax / (m * boost), or 0 for a zero row
    float scale;  // m * kq = max|x'| / qmax
    float boost;  // 1, or kBoost for a row below kBoostBelow
};

// qmax / m overflows binary32 once m drops below about 2^-121.  The codes
// depend only on y / m, so a row whose maximum is below kBoostBelow is
// quantised from its values magnified by kBoost, an exact power of two:
// y * kBoost and m * kBoost are exact (a subnormal becomes normal), and
// code = round(y * kBoost * qmax / (m * kBoost)).  Every finite row, down
// to the smallest subnormal, thus gets the codes of its exact quotients;
// the scale still comes from m itself.
constexpr float kBoostBelow = 0x1p-100f;
constexpr float kBoost = 0x1p+64f;

// inv from the hardware reciprocal refined by one residual step (within
// about half an ulp of the correctly rounded quotient; a handful of
// instructions instead of the full IEEE division sequence, which every lane
// of a row would otherwise run).
__device__ __forceinline__ RowQuant row_quant(float m, float kq, int qmax)
{
    const float fq = (float)qmax;
    const bool live = m > 0.0f;
    RowQuant rq;
    rq.boost = live && m < kBoostBelow ? kBoost : 1.0f;
    const float mb = m * rq.boost;
    const float r = __builtin_amdgcn_rcpf(live ? mb : 1.0f);
    const float q0 = fq * r;
    const float e = __builtin_fmaf(-mb, q0, fq);
    rq.inv = live ? __builtin_fmaf(e, r, q0) : 0.0f;
    rq.scale = m * kq;
    return rq;
}

// True on every lane when any lane of the wave holds a magnified row
// (wave-uniform, so the magnification can sit behind a scalar branch).
__device__ __forceinline__ bool wave_any_boost(const RowQuant &rq)
{
    return __builtin_amdgcn_ballot_w64(rq.boost != 1.0f) != 0;
}

}  // namespace hq
