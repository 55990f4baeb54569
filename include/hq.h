/*
 * hq.h -- C ABI of libhq.so: randomized Hadamard rotation fused with symmetric
 * per-row low-bit quantisation, for AMD Instinct MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *   [RQ] "旋转量化：大模型低比特量化中的离群值克星" (rotation-quantization blog)
 *   [QT] "手把手教你用QuaRot实现LLM的4位量化：从原理到代码实践" (QuaRot tutorial)
 *   [HQA] "哈特曼旋转，轻量级QAT，流式注意力" (Q&A post, section 1)
 *   [MS] "QuaRot：基于旋转的离群值抑制算法说明" (msModelSlim QuaRot page)
 *
 *   Each row x (n contiguous elements) is flipped elementwise by a +-1 sign
 *   vector s shared by all rows ([QT] 2.1: the "random Hadamard" transform),
 *   then split into n/b consecutive blocks of b elements, and every block is
 *   multiplied by the Sylvester Hadamard matrix H_b normalised by 1/sqrt(b)
 *   ([RQ] 2.1: H_2 = [[1,1],[1,-1]], H_2m = H_2 (x) H_m; blockwise rotation
 *   for widths that are not a power of two; b == n is the full rotation):
 *
 *       x'[kb+i] = sum_j x[kb+j] s[kb+j] H_b[j][i] / sqrt(b)
 *
 *   The row is then quantised symmetrically with one scale per row
 *   ([HQA] 1, [RQ] 2.2):
 *
 *       scale = max_i |x'_i| / qmax,   qmax = 2^(bits-1) - 1  (7 or 127)
 *       q_i   = clamp(round_half_even(x'_i / scale), -qmax, qmax)
 *
 *   and the inverse path dequantises and rotates back with the transpose
 *   ([MS] principle: the normalised H is orthogonal, Q^T = Q^-1):
 *
 *       x_hat[kb+i] = s[kb+i] * sum_j (q[kb+j] * scale) H_b[i][j] / sqrt(b)
 *
 *   The Sylvester H_b is symmetric, so there H_b^T = H_b; the matrices of
 *   the full rotations below (H_k (x) H_m) are not, and their inverse
 *   multiplies by the transpose.
 *
 *   Full rotation of a width that is not a power of two (b == n only):
 *   H_n = H_k (x) H_(n/k), n/k a power of two and H_k Paley's first
 *   construction over GF(q), q = k - 1 = p^e = 3 (mod 4) a prime power with
 *   e <= 3; k is the smallest order of the form (odd part of n) * 2^a.
 *   Element i*(n/k) + j of a row is entry (i, j) of the Kronecker product
 *   ([RQ] 2.1: larger Hadamard matrices as Kronecker products).  Widths
 *   without such a factorisation (e.g. 496 = 31 * 16) are HQ_EINVAL.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument except `stream` is a DEVICE pointer owned by the
 *     caller.  The library allocates no memory and keeps no per-call state;
 *     it caches a few device properties per device, and, for the full-width
 *     rotation of order k = 344 (n = 11008) with one scale per row, a
 *     constant operand table in its own static device memory.  It is
 *     thread-safe.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL is the null stream).  On return with HQ_OK the work is enqueued.
 *     One exception: the first such k = 344 rotate + quantise call on a
 *     device builds that table and waits for the device to be idle before
 *     it enqueues its work (so that first call cannot be captured into a
 *     graph); every later call is asynchronous.
 *   - A row is n contiguous elements; rows are contiguous (row stride n).
 *     Head-dim-innermost layouts ([B,H,S,D], [S,H,D]) are just rows of D.
 *   - s: int8 [n]; an element < 0 means "negate", anything else "keep".
 *     The caller supplies it; the library never draws random numbers.
 *   - Supported shapes: n % 16 == 0, 16 <= n <= hq_max_n(), rows >= 0
 *     (rows == 0 is a no-op), and either
 *       b a power of two with n % b == 0 (b > 4096: HQ_EUNSUPPORTED), or
 *       b == n for a width n = k * 2^m that is not a power of two and has
 *       a Paley order k as above (e.g. 96 = 12 * 8, 11008 = 344 * 32);
 *     any other b is HQ_EINVAL.
 *   - Alignment: x, codes, y and s must be 16-byte aligned; scales must be
 *     aligned to their element size.
 *   - Outputs must not overlap inputs.  Inputs are never modified.
 *   - Every argument is validated on the host before anything is enqueued;
 *     on any error nothing is written and nothing is launched.  No C++
 *     exception crosses this boundary.
 *   - Values of x that are NaN or infinite give unspecified codes/scales.
 */
#ifndef HQ_H
#define HQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hq_status {
    HQ_OK = 0,           /* enqueued (or nothing to do)                    */
    HQ_EINVAL = 1,       /* invalid argument: null pointer, bad shape,
                            dtype, bits, or misaligned pointer             */
    HQ_EUNSUPPORTED = 2, /* valid request this library has no kernel for
                            (n above hq_max_n(), b above 4096)             */
    HQ_EHIP = 3          /* the HIP runtime reported an error (no device,
                            launch failure); see hq_last_hip_error()       */
} hq_status;

/* Under C++ the type is fixed to int32_t, so that any int32 value a caller
 * passes is a valid value of the type and is rejected as HQ_EINVAL by the
 * validation (an enum without a fixed type holds only the range of its
 * enumerators there).  C sees a plain enum of the same size. */
typedef enum hq_dtype
#ifdef __cplusplus
    : int32_t
#endif
{
    HQ_F32 = 0,  /* IEEE binary32 */
    HQ_BF16 = 1, /* bfloat16      */
    HQ_F16 = 2   /* IEEE binary16 */
} hq_dtype;

/*
 * hq_rotate_quant -- fused rotation + symmetric quantisation (forward path).
 *   x        [rows, n] input, element type x_dtype (HQ_F32, HQ_BF16, HQ_F16)
 *   s        [n] int8 signs
 *   bits     4 or 8
 *   codes    bits == 4: [rows, n/2] uint8; element 2j in the low nibble,
 *            2j+1 in the high nibble, 4-bit two's complement in [-7, 7].
 *            bits == 8: [rows, n] int8 in [-127, 127].
 *   scales   [rows], element type scale_dtype (HQ_F32 or HQ_F16), the stored
 *            value of max|x'|/qmax rounded to nearest even.  A row of zeros
 *            gets scale 0 and codes 0.  Every other finite row, down to
 *            subnormal inputs, is quantised as defined above.
 * Codes are computed from the unrounded scale, so they do not depend on
 * scale_dtype.
 */
hq_status hq_rotate_quant(const void *x, hq_dtype x_dtype, int64_t rows, int32_t n,
                          int32_t b, const int8_t *s, int32_t bits, void *codes,
                          void *scales, hq_dtype scale_dtype, void *stream);

/*
 * hq_dequant_rotate_inv -- dequantisation + inverse rotation (round trip).
 *   codes, scales, scale_dtype, bits: as written by hq_rotate_quant
 *   y        [rows, n] output, y_dtype HQ_F32 or HQ_BF16 (rounded to
 *            nearest even)
 */
hq_status hq_dequant_rotate_inv(const void *codes, const void *scales,
                                hq_dtype scale_dtype, int64_t rows, int32_t n,
                                int32_t b, const int8_t *s, int32_t bits, void *y,
                                hq_dtype y_dtype, void *stream);

/*
 * hq_rotate_quant_grouped -- hq_rotate_quant with one scale per run of
 * `group` consecutive elements of the rotated row instead of one per row
 * ([RQ] 6.2: group size 128 for 4-bit, 64 or 128 for 8-bit; [QT] 4.2: the
 * scales of a tensor are stored together, apart from the codes).  For each
 * group k of a row (elements k*group .. k*group+group-1 of x'):
 *
 *       scale_k = max_{i in k} |x'_i| / qmax
 *       q_i     = clamp(round_half_even(x'_i / scale_k), -qmax, qmax)
 *
 *   group    n (identical to hq_rotate_quant), or a power of two with
 *            2 <= group < n that divides n; anything else is HQ_EINVAL.
 *            The group size is independent of the block size b.
 *   scales   [rows, n/group] (row-major), element type scale_dtype.
 *   Everything else, including the zero rule (applied per group), is as for
 *   hq_rotate_quant.
 */
hq_status hq_rotate_quant_grouped(const void *x, hq_dtype x_dtype, int64_t rows, int32_t n,
                                  int32_t b, const int8_t *s, int32_t bits, int32_t group,
                                  void *codes, void *scales, hq_dtype scale_dtype,
                                  void *stream);

/*
 * hq_dequant_rotate_inv_grouped -- inverse of hq_rotate_quant_grouped: every
 * element is dequantised with the scale of its own group (v_i = q_i *
 * scale_k, scales [rows, n/group]) before the inverse rotation.  Arguments
 * and errors as for hq_dequant_rotate_inv plus `group` as above.
 */
hq_status hq_dequant_rotate_inv_grouped(const void *codes, const void *scales,
                                        hq_dtype scale_dtype, int64_t rows, int32_t n,
                                        int32_t b, const int8_t *s, int32_t bits,
                                        int32_t group, void *y, hq_dtype y_dtype,
                                        void *stream);

/*
 * hq_rotate_quant_append -- hq_rotate_quant of a few new rows written into a
 * preallocated per-row-scale cache at given rows: the online K/V rotation
 * into a 4-bit cache, one decode step at a time ([QT] 2.2: K and V are
 * rotated online and kept as 4-bit codes).
 *   x, x_dtype, rows, n, b, s, bits, scale_dtype: as for hq_rotate_quant
 *   dst_rows  [rows] int64, device, 8-byte aligned: input row r is written to
 *             cache row dst_rows[r].  Rows whose index lies outside
 *             [0, cache_rows) are skipped (nothing is written for them; the
 *             host cannot see device indices without synchronising).  Two
 *             input rows with the same index race: the cache row then holds
 *             one of them.
 *   codes     the cache's codes: [cache_rows, n/2] (bits 4) or [cache_rows, n]
 *   scales    the cache's scales: [cache_rows]
 * Cache rows that no input row names are not touched.
 */
hq_status hq_rotate_quant_append(const void *x, hq_dtype x_dtype, int64_t rows, int32_t n,
                                 int32_t b, const int8_t *s, int32_t bits,
                                 const int64_t *dst_rows, void *codes, void *scales,
                                 hq_dtype scale_dtype, int64_t cache_rows, void *stream);

/*
 * hq_decode_attention -- the consumer of the codes: attention of one query
 * token per head over a K/V cache written by hq_rotate_quant /
 * hq_rotate_quant_append with one scale per row ([QT] 2.2: K and V rotated
 * online, stored as 4-bit codes and dequantised when attention reads them;
 * [HQA] 1: rotating Q with the same matrix keeps Q.K^T).  For query head h
 * and its kv head kh = h / (q_heads / kv_heads):
 *
 *       q'  = (q_h * s) . H_b / sqrt(b)                 (the cache's rotation)
 *       c_t = q' . (code_k[t, kh] * scale_k[t, kh]) / sqrt(n)
 *       o'  = sum_t softmax_t(c) * code_v[t, kh] * scale_v[t, kh]
 *       out_h = (o' . H_b / sqrt(b)) * s                (the query's space)
 *
 *   q         [q_heads, n], q_dtype (HQ_F32, HQ_BF16, HQ_F16), not rotated
 *   s, b      the sign vector [n] and block size the cache was written with
 *   k_codes, v_codes    [tokens, kv_heads, n/2] uint8, 16-byte aligned
 *   k_scales, v_scales  [tokens, kv_heads], scale_dtype (one per row)
 *   out       [q_heads, n] fp32, 16-byte aligned
 *   workspace device memory of at least hq_decode_attention_workspace(...)
 *             bytes, 16-byte aligned; its contents on entry do not matter and
 *             two calls in flight on one workspace race.
 * Errors: HQ_EINVAL for invalid arguments (tokens < 1, q_heads not a
 * multiple of kv_heads, a short workspace, ...); HQ_EUNSUPPORTED for valid
 * requests outside the library's kernel: n != 128, bits != 4, or
 * q_heads / kv_heads not 1, 2, 4 or 8.
 */
int64_t hq_decode_attention_workspace(int32_t q_heads, int32_t kv_heads, int64_t tokens);
hq_status hq_decode_attention(const void *q, hq_dtype q_dtype, int32_t q_heads,
                              int32_t kv_heads, int32_t n, int32_t b, const int8_t *s,
                              int64_t tokens, int32_t bits, const void *k_codes,
                              const void *k_scales, const void *v_codes, const void *v_scales,
                              hq_dtype scale_dtype, float *out, void *workspace,
                              int64_t workspace_bytes, void *stream);

/*
 * hq_decode_attention_noalloc -- hq_decode_attention without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * allocates nothing (no hipMalloc, hipFree or allocating library routine):
 * the partials live in a device array of HQ_NOALLOC_WORKSPACE_BYTES that the
 * library holds on each GPU it runs on until the process ends.
 *   Arguments, results and errors as for hq_decode_attention, plus
 *   HQ_EUNSUPPORTED when hq_decode_attention_workspace(q_heads, kv_heads,
 *   tokens) exceeds HQ_NOALLOC_WORKSPACE_BYTES (e.g. 32 query heads over
 *   8 kv heads need 1.6 MiB at any cache length), and HQ_EHIP if the
 *   array's address cannot be obtained.
 * Every call on one GPU shares that GPU's array (it keeps the last call's
 * partials, which no call reads before writing): calls that overlap on one
 * GPU, on any streams, race.  Use one stream, or hq_decode_attention with a
 * workspace of your own per stream.
 */
#define HQ_NOALLOC_WORKSPACE_BYTES (4 * 1024 * 1024)
hq_status hq_decode_attention_noalloc(const void *q, hq_dtype q_dtype, int32_t q_heads,
                                      int32_t kv_heads, int32_t n, int32_t b, const int8_t *s,
                                      int64_t tokens, int32_t bits, const void *k_codes,
                                      const void *k_scales, const void *v_codes,
                                      const void *v_scales, hq_dtype scale_dtype, float *out,
                                      void *stream);

/*
 * hq_rotate -- rotation only: y = x' as fp32 [rows, n] (no quantisation).
 * Used to check the rotated values themselves and Q.K^T preservation
 * ([HQA] 1: rotating Q and K with the same matrix keeps Q.K^T).
 */
hq_status hq_rotate(const void *x, hq_dtype x_dtype, int64_t rows, int32_t n,
                    int32_t b, const int8_t *s, float *y, void *stream);

/* Static text for a status code (never NULL). */
const char *hq_status_str(int32_t status);

/* Text of the last HIP error seen by this thread inside the library (empty
 * string if none).  Valid until the next library call on the same thread. */
const char *hq_last_hip_error(void);

/* Largest supported row width n on the current device (needs a device;
 * returns 0 if none is present). */
int32_t hq_max_n(void);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int32_t hq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HQ_H */
