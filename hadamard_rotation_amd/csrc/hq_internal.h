// hq_internal.h -- declarations shared by the host dispatcher and the kernel
// translation units of libhq.so.  Not part of the public ABI (include/hq.h).
#pragma once

#include <hip/hip_runtime.h>

#include "hq.h"

#include <cstdint>

namespace hq {

// Element types, numbered like the public hq_dtype.
enum Dtype : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

// Which path a launch computes.
enum Op : int {
    kRotateQuant = 0,  // x -> codes + scales
    kRotate = 1,       // x -> fp32 rotated rows
    kDequantInv = 2    // codes + scales -> rows (inverse rotation)
};

// The Hadamard matrix of a width n that is not a power of two:
// H_n = H_k (x) H_m2, m2 = n / k a power of two, H_k Paley's first
// construction over GF(q), q = k - 1 = p^e = 3 (mod 4), e <= 3.  GF(p^e) is
// GF(p)[x] modulo x^e + mod[e-1] x^(e-1) + ... + mod[0], the first monic
// polynomial of degree e without a root in GF(p) by the index
// mod[0] + p mod[1] + p^2 mod[2]; an element c0 + c1 x + c2 x^2 has index
// c0 + p c1 + p^2 c2.  k is the smallest order of the form
// (odd part of n) * 2^a.  k = 1 (and m2 = n) for a power of two.
struct PaleySpec {
    int k = 1, m2 = 0, p = 0, e = 0;
    int mod[3] = {0, 0, 0};
};

// Fills ps for a width n; false when n has no such matrix.
bool hadamard_split(int n, PaleySpec &ps);

// Everything a launcher needs; validated by the host dispatcher beforehand.
struct Request {
    Op op;
    const void *x;          // kRotateQuant / kRotate input rows
    int x_dtype;
    const void *codes_in;   // kDequantInv inputs
    const void *scales_in;
    int64_t rows;
    int n;
    int b;
    const int8_t *s;
    int bits;
    void *codes;            // kRotateQuant outputs
    void *scales;
    int scale_dtype;        // kRotateQuant output / kDequantInv input
    int group;              // elements per scale: n (one scale per row) or a
                            // power of two dividing n (scales [rows, n/group])
    int logg;               // log2(group) when group is a power of two, else -1
    const int64_t *dst_rows;  // kRotateQuant append: output row of each input
                              // row (device), or null: row r writes row r
    int64_t cache_rows;       // rows of codes / scales when dst_rows is set
    void *y;                // kRotate / kDequantInv output
    int y_dtype;
    hipStream_t stream;
    PaleySpec paley;        // b == n not a power of two: its factors
};

// Per-device facts the dispatcher uses to choose and size launches.
struct DeviceInfo {
    int cu_count;
    int lds_per_block;   // bytes of LDS one workgroup may allocate
};

// Decode attention over a rotated, quantised K/V cache (head dim 128, 4-bit
// codes, one scale per row); validated by the host dispatcher beforehand.
struct AttnRequest {
    const void *q;          // [q_heads, 128], q_dtype
    int q_dtype;
    int q_heads;
    int kv_heads;           // q_heads % kv_heads == 0, q_heads / kv_heads <= 8
    int b;                  // block size of the cache's rotation
    const int8_t *s;        // [128]
    int64_t tokens;         // >= 1
    const void *k_codes;    // [tokens, kv_heads, 64]
    const void *k_scales;   // [tokens, kv_heads]
    const void *v_codes;
    const void *v_scales;
    int scale_dtype;
    float *out;             // [q_heads, 128]
    void *workspace;        // attention_workspace() bytes
    hipStream_t stream;
};

// Work split of the decode attention, shared by the host validation and the
// kernels: kernel 1 runs workgroups of kAttnWaves waves, each wave one
// "part" (a token range of one kv head); about 3072 waves in all (12 per
// CU), whole workgroups, at most one part per 16-token block.  Each
// workgroup leaves one partial per query head in the workspace:
// o[128], max, sum and two unused floats.
constexpr int kAttnHeadDim = 128;
constexpr int kAttnPartStride = kAttnHeadDim + 4;
constexpr int kAttnWaves = 4;

inline int attention_parts(int kv_heads, int64_t tokens)
{
    const int64_t blocks = (tokens + 15) / 16;
    int64_t p = (3072 + kv_heads - 1) / kv_heads;
    p = (p + kAttnWaves - 1) / kAttnWaves * kAttnWaves;
    const int64_t pmax = (blocks + kAttnWaves - 1) / kAttnWaves * kAttnWaves;
    if (p > pmax)
        p = pmax;
    return (int)(p < kAttnWaves ? kAttnWaves : p);
}

inline size_t attention_workspace(int q_heads, int kv_heads, int64_t tokens)
{
    return (size_t)q_heads * (attention_parts(kv_heads, tokens) / kAttnWaves) * kAttnPartStride *
           sizeof(float);
}

hipError_t launch_attention(const AttnRequest &r);

// The library's own workspace for hq_decode_attention_noalloc: a file-scope
// device array of this many bytes in the attention kernels' source, one copy
// per GPU.  attention_static_workspace() returns its address on the current
// device (looked up once per device).
constexpr size_t kAttnStaticWorkspaceBytes = HQ_NOALLOC_WORKSPACE_BYTES;
hipError_t attention_static_workspace(void **ptr);

// Generic path: any supported (n, b); one workgroup per row with the row
// staged in LDS as fp32.  Requires 4*n <= dev.lds_per_block.
hipError_t launch_generic(const Request &r, const DeviceInfo &dev);
// Matrix-core path for H_k (x) H_32 rotations (k in (320, 352], 16-bit
// input, per-row fp32 scales).
bool paley_mfma_available(const Request &r);
hipError_t launch_paley_mfma(const Request &r, const DeviceInfo &dev);
// Whether the generic kernel's LDS holds a request with r.paley.k > 1.
bool generic_paley_fits(const Request &r, const DeviceInfo &dev);

// Tuned register-resident paths.  fast_plan() says whether one exists for
// the request; launch_fast() enqueues it.
bool fast_available(const Request &r);
hipError_t launch_fast(const Request &r, const DeviceInfo &dev);

// Matrix-core paths (16-bit input, forward): mfma_available() says whether
// one exists for the request; launch_mfma() enqueues it.
bool mfma_available(const Request &r);
hipError_t launch_mfma(const Request &r, const DeviceInfo &dev);

}  // namespace hq
