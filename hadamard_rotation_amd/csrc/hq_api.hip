// hq_api.hip -- the C ABI of libhq.so (declared in include/hq.h): argument
// validation, per-device property cache and dispatch to the kernels.
//
// Every check happens on the host before anything is enqueued, so an
// invalid call writes nothing and launches nothing.  Calls with rows == 0
// return HQ_OK without touching the HIP runtime.
#include "hq.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "hq_internal.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxB = 4096;

thread_local char g_hip_error[256] = "";

struct DeviceSlot {
    std::once_flag once;
    hipError_t err = hipSuccess;
    hq::DeviceInfo info{};
};
DeviceSlot g_devices[kMaxDevices];

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

hq_status hip_fail(hipError_t e, const char *where)
{
    std::snprintf(g_hip_error, sizeof g_hip_error, "%s: %s", where, hipGetErrorString(e));
    return HQ_EHIP;
}

// Properties of the current device, queried once per device.
hq_status current_device(const hq::DeviceInfo **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return hip_fail(hipErrorInvalidDevice, "device ordinal");
    DeviceSlot &slot = g_devices[dev];
    std::call_once(slot.once, [&]() {
        int v = 0;
        slot.err = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (slot.err != hipSuccess)
            return;
        slot.info.cu_count = v;
        slot.err = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (slot.err != hipSuccess)
            return;
        slot.info.lds_per_block = v;
    });
    if (slot.err != hipSuccess)
        return hip_fail(slot.err, "hipDeviceGetAttribute");
    *out = &slot.info;
    return HQ_OK;
}

int max_n_for(const hq::DeviceInfo &d)
{
    // the generic kernel stages a row in LDS as fp32 next to <= 256 B of its own
    int by_lds = (d.lds_per_block - 256) / (int)sizeof(float);
    int cap = 65536;
    int m = by_lds < cap ? by_lds : cap;
    return m & ~15;
}

// Checks shared by all entry points.  Pointer checks skip nulls when
// rows == 0.
hq_status check_shape(int64_t rows, int32_t n, int32_t b, const int8_t *s)
{
    if (rows < 0)
        return HQ_EINVAL;
    if (n < 16 || n % 16 != 0)
        return HQ_EINVAL;
    if (is_pow2(b)) {
        if (n % b != 0)
            return HQ_EINVAL;
    } else {
        // a width that is not a power of two: the full rotation by
        // H_k (x) H_(n/k), when n has such a factorisation
        hq::PaleySpec ps;
        if (b != n || !hq::hadamard_split(n, ps))
            return HQ_EINVAL;
    }
    if (rows > 0 && !s)
        return HQ_EINVAL;
    if (s && !aligned(s, 16))
        return HQ_EINVAL;
    if (is_pow2(b) && b > kMaxB)
        return HQ_EUNSUPPORTED;
    return HQ_OK;
}

bool valid_scale_dtype(int d) { return d == HQ_F32 || d == HQ_F16; }

bool valid_in_dtype(int d) { return d == HQ_F32 || d == HQ_BF16 || d == HQ_F16; }

hq_status dispatch(const hq::Request &r)
{
    const hq::DeviceInfo *dev = nullptr;
    hq_status st = current_device(&dev);
    if (st != HQ_OK)
        return st;
    if (r.n > max_n_for(*dev))
        return HQ_EUNSUPPORTED;
    hipError_t e;
    if (!is_pow2(r.b)) {
        // H_k (x) H_m2: the matrix-core kernel where it has a plan, else the
        // generic kernel
        hq::Request rp = r;
        if (!hq::hadamard_split(r.b, rp.paley))
            return HQ_EINVAL;
        if (hq::paley_mfma_available(rp))
            e = hq::launch_paley_mfma(rp, *dev);
        else if (!hq::generic_paley_fits(rp, *dev))
            return HQ_EUNSUPPORTED;
        else
            e = hq::launch_generic(rp, *dev);
    } else if (hq::mfma_available(r))
        e = hq::launch_mfma(r, *dev);
    else if (hq::fast_available(r))
        e = hq::launch_fast(r, *dev);
    else
        e = hq::launch_generic(r, *dev);
    if (e != hipSuccess)
        return hip_fail(e, "kernel launch");
    return HQ_OK;
}

// Group size check: n itself (one scale per row) or a power of two >= 2
// that divides n.  Returns -2 when invalid, else log2(group) (-1 when
// group == n is not a power of two).
int group_log2(int32_t n, int32_t group)
{
    if (group == n)
        return is_pow2(n) ? __builtin_ctz((unsigned)n) : -1;
    if (group < 2 || !is_pow2(group) || n % group != 0)
        return -2;
    return __builtin_ctz((unsigned)group);
}

hq_status rotate_quant_impl(const void *x, hq_dtype x_dtype, int64_t rows, int32_t n,
                            int32_t b, const int8_t *s, int32_t bits, int32_t group,
                            void *codes, void *scales, hq_dtype scale_dtype, void *stream,
                            const int64_t *dst_rows = nullptr, int64_t cache_rows = 0)
{
    g_hip_error[0] = '\0';
    hq_status st = check_shape(rows, n, b, s);
    if (st == HQ_EINVAL)
        return st;
    const int logg = group_log2(n, group);
    if (logg == -2)
        return HQ_EINVAL;
    if (!valid_in_dtype(x_dtype) || !valid_scale_dtype(scale_dtype))
        return HQ_EINVAL;
    if (bits != 4 && bits != 8)
        return HQ_EINVAL;
    if (rows > 0 && (!x || !codes || !scales))
        return HQ_EINVAL;
    if ((x && !aligned(x, 16)) || (codes && !aligned(codes, 16)))
        return HQ_EINVAL;
    if (scales && !aligned(scales, scale_dtype == HQ_F32 ? 4 : 2))
        return HQ_EINVAL;
    if (st != HQ_OK)
        return st;
    if (rows == 0)
        return HQ_OK;
    hq::Request r{};
    r.op = hq::kRotateQuant;
    r.x = x;
    r.x_dtype = x_dtype;
    r.rows = rows;
    r.n = n;
    r.b = b;
    r.s = s;
    r.bits = bits;
    r.codes = codes;
    r.scales = scales;
    r.scale_dtype = scale_dtype;
    r.group = group;
    r.logg = logg;
    r.dst_rows = dst_rows;
    r.cache_rows = cache_rows;
    r.stream = (hipStream_t)stream;
    return dispatch(r);
}

hq_status dequant_inv_impl(const void *codes, const void *scales, hq_dtype scale_dtype,
                           int64_t rows, int32_t n, int32_t b, const int8_t *s, int32_t bits,
                           int32_t group, void *y, hq_dtype y_dtype, void *stream)
{
    g_hip_error[0] = '\0';
    hq_status st = check_shape(rows, n, b, s);
    if (st == HQ_EINVAL)
        return st;
    const int logg = group_log2(n, group);
    if (logg == -2)
        return HQ_EINVAL;
    if (!valid_scale_dtype(scale_dtype) || (y_dtype != HQ_F32 && y_dtype != HQ_BF16))
        return HQ_EINVAL;
    if (bits != 4 && bits != 8)
        return HQ_EINVAL;
    if (rows > 0 && (!codes || !scales || !y))
        return HQ_EINVAL;
    if ((codes && !aligned(codes, 16)) || (y && !aligned(y, 16)))
        return HQ_EINVAL;
    if (scales && !aligned(scales, scale_dtype == HQ_F32 ? 4 : 2))
        return HQ_EINVAL;
    if (st != HQ_OK)
        return st;
    if (rows == 0)
        return HQ_OK;
    hq::Request r{};
    r.op = hq::kDequantInv;
    r.codes_in = codes;
    r.scales_in = scales;
    r.scale_dtype = scale_dtype;
    r.rows = rows;
    r.n = n;
    r.b = b;
    r.s = s;
    r.bits = bits;
    r.y = y;
    r.y_dtype = y_dtype;
    r.group = group;
    r.logg = logg;
    r.stream = (hipStream_t)stream;
    return dispatch(r);
}

// Validation shared by both decode attention entry points (everything but
// the workspace); fills r on success.
hq_status attention_request(const void *q, hq_dtype q_dtype, int32_t q_heads, int32_t kv_heads,
                            int32_t n, int32_t b, const int8_t *s, int64_t tokens, int32_t bits,
                            const void *k_codes, const void *k_scales, const void *v_codes,
                            const void *v_scales, hq_dtype scale_dtype, float *out,
                            void *stream, hq::AttnRequest &r)
{
    if (q_heads <= 0 || kv_heads <= 0 || q_heads % kv_heads != 0 || tokens < 1)
        return HQ_EINVAL;
    if (n < 16 || n % 16 != 0 || !is_pow2(b) || n % b != 0)
        return HQ_EINVAL;
    if (bits != 4 && bits != 8)
        return HQ_EINVAL;
    if (!valid_in_dtype(q_dtype) || !valid_scale_dtype(scale_dtype))
        return HQ_EINVAL;
    if (!q || !s || !k_codes || !k_scales || !v_codes || !v_scales || !out)
        return HQ_EINVAL;
    if (!aligned(q, q_dtype == HQ_F32 ? 4 : 2) || !aligned(s, 16) || !aligned(k_codes, 16) ||
        !aligned(v_codes, 16) || !aligned(out, 16))
        return HQ_EINVAL;
    const uintptr_t sa = scale_dtype == HQ_F32 ? 4 : 2;
    if (!aligned(k_scales, sa) || !aligned(v_scales, sa))
        return HQ_EINVAL;
    const int g = q_heads / kv_heads;
    if (n != 128 || bits != 4 || (g != 1 && g != 2 && g != 4 && g != 8))
        return HQ_EUNSUPPORTED;
    r.q = q;
    r.q_dtype = q_dtype;
    r.q_heads = q_heads;
    r.kv_heads = kv_heads;
    r.b = b;
    r.s = s;
    r.tokens = tokens;
    r.k_codes = k_codes;
    r.k_scales = k_scales;
    r.v_codes = v_codes;
    r.v_scales = v_scales;
    r.scale_dtype = scale_dtype;
    r.out = out;
    r.stream = (hipStream_t)stream;
    return HQ_OK;
}

hq_status attention_launch(hq::AttnRequest &r, void *workspace)
{
    const hq::DeviceInfo *dev = nullptr;
    hq_status st = current_device(&dev);
    if (st != HQ_OK)
        return st;
    r.workspace = workspace;
    const hipError_t e = hq::launch_attention(r);
    if (e != hipSuccess)
        return hip_fail(e, "kernel launch");
    return HQ_OK;
}

}  // namespace

extern "C" {

hq_status hq_rotate_quant(const void *x, hq_dtype x_dtype, int64_t rows, int32_t n,
                          int32_t b, const int8_t *s, int32_t bits, void *codes,
                          void *scales, hq_dtype scale_dtype, void *stream)
{
    return rotate_quant_impl(x, x_dtype, rows, n, b, s, bits, n, codes, scales, scale_dtype,
                             stream);
}

hq_status hq_rotate_quant_grouped(const void *x, hq_dtype x_dtype, int64_t rows, int32_t n,
                                  int32_t b, const int8_t *s, int32_t bits, int32_t group,
                                  void *codes, void *scales, hq_dtype scale_dtype, void *stream)
{
    return rotate_quant_impl(x, x_dtype, rows, n, b, s, bits, group, codes, scales,
                             scale_dtype, stream);
}

hq_status hq_rotate_quant_append(const void *x, hq_dtype x_dtype, int64_t rows, int32_t n,
                                 int32_t b, const int8_t *s, int32_t bits,
                                 const int64_t *dst_rows, void *codes, void *scales,
                                 hq_dtype scale_dtype, int64_t cache_rows, void *stream)
{
    if (cache_rows < 0 || (rows > 0 && !dst_rows))
        return HQ_EINVAL;
    if (dst_rows && !aligned(dst_rows, 8))
        return HQ_EINVAL;
    return rotate_quant_impl(x, x_dtype, rows, n, b, s, bits, n, codes, scales, scale_dtype,
                             stream, dst_rows, cache_rows);
}

hq_status hq_dequant_rotate_inv(const void *codes, const void *scales,
                                hq_dtype scale_dtype, int64_t rows, int32_t n,
                                int32_t b, const int8_t *s, int32_t bits, void *y,
                                hq_dtype y_dtype, void *stream)
{
    return dequant_inv_impl(codes, scales, scale_dtype, rows, n, b, s, bits, n, y, y_dtype,
                            stream);
}

hq_status hq_dequant_rotate_inv_grouped(const void *codes, const void *scales,
                                        hq_dtype scale_dtype, int64_t rows, int32_t n,
                                        int32_t b, const int8_t *s, int32_t bits,
                                        int32_t group, void *y, hq_dtype y_dtype,
                                        void *stream)
{
    return dequant_inv_impl(codes, scales, scale_dtype, rows, n, b, s, bits, group, y,
                            y_dtype, stream);
}

int64_t hq_decode_attention_workspace(int32_t q_heads, int32_t kv_heads, int64_t tokens)
{
    if (q_heads <= 0 || kv_heads <= 0 || tokens < 1)
        return 0;
    return (int64_t)hq::attention_workspace(q_heads, kv_heads, tokens);
}

hq_status hq_decode_attention(const void *q, hq_dtype q_dtype, int32_t q_heads,
                              int32_t kv_heads, int32_t n, int32_t b, const int8_t *s,
                              int64_t tokens, int32_t bits, const void *k_codes,
                              const void *k_scales, const void *v_codes, const void *v_scales,
                              hq_dtype scale_dtype, float *out, void *workspace,
                              int64_t workspace_bytes, void *stream)
{
    g_hip_error[0] = '\0';
    hq::AttnRequest r{};
    hq_status st = attention_request(q, q_dtype, q_heads, kv_heads, n, b, s, tokens, bits,
                                     k_codes, k_scales, v_codes, v_scales, scale_dtype, out,
                                     stream, r);
    if (st != HQ_OK)
        return st;
    if (!workspace || !aligned(workspace, 16))
        return HQ_EINVAL;
    if (workspace_bytes < (int64_t)hq::attention_workspace(q_heads, kv_heads, tokens))
        return HQ_EINVAL;
    return attention_launch(r, workspace);
}

hq_status hq_decode_attention_noalloc(const void *q, hq_dtype q_dtype, int32_t q_heads,
                                      int32_t kv_heads, int32_t n, int32_t b, const int8_t *s,
                                      int64_t tokens, int32_t bits, const void *k_codes,
                                      const void *k_scales, const void *v_codes,
                                      const void *v_scales, hq_dtype scale_dtype, float *out,
                                      void *stream)
{
    g_hip_error[0] = '\0';
    hq::AttnRequest r{};
    hq_status st = attention_request(q, q_dtype, q_heads, kv_heads, n, b, s, tokens, bits,
                                     k_codes, k_scales, v_codes, v_scales, scale_dtype, out,
                                     stream, r);
    if (st != HQ_OK)
        return st;
    if (hq::attention_workspace(q_heads, kv_heads, tokens) > hq::kAttnStaticWorkspaceBytes)
        return HQ_EUNSUPPORTED;
    void *ws = nullptr;
    const hipError_t e = hq::attention_static_workspace(&ws);
    if (e != hipSuccess)
        return hip_fail(e, "static workspace");
    return attention_launch(r, ws);
}

hq_status hq_rotate(const void *x, hq_dtype x_dtype, int64_t rows, int32_t n,
                    int32_t b, const int8_t *s, float *y, void *stream)
{
    g_hip_error[0] = '\0';
    hq_status st = check_shape(rows, n, b, s);
    if (st == HQ_EINVAL)
        return st;
    if (!valid_in_dtype(x_dtype))
        return HQ_EINVAL;
    if (rows > 0 && (!x || !y))
        return HQ_EINVAL;
    if ((x && !aligned(x, 16)) || (y && !aligned(y, 16)))
        return HQ_EINVAL;
    if (st != HQ_OK)
        return st;
    if (rows == 0)
        return HQ_OK;
    hq::Request r{};
    r.op = hq::kRotate;
    r.x = x;
    r.x_dtype = x_dtype;
    r.rows = rows;
    r.n = n;
    r.b = b;
    r.s = s;
    r.y = y;
    r.y_dtype = HQ_F32;
    r.bits = 4;
    r.scale_dtype = HQ_F32;
    r.group = n;
    r.logg = group_log2(n, n);
    r.stream = (hipStream_t)stream;
    return dispatch(r);
}

const char *hq_status_str(int32_t status)
{
    switch (status) {
    case HQ_OK: return "HQ_OK: success";
    case HQ_EINVAL: return "HQ_EINVAL: invalid argument";
    case HQ_EUNSUPPORTED: return "HQ_EUNSUPPORTED: valid request without a kernel in this library";
    case HQ_EHIP: return "HQ_EHIP: HIP runtime error";
    default: return "unknown hq_status";
    }
}

const char *hq_last_hip_error(void) { return g_hip_error; }

int32_t hq_max_n(void)
{
    const hq::DeviceInfo *dev = nullptr;
    if (current_device(&dev) != HQ_OK)
        return 0;
    return max_n_for(*dev);
}

int32_t hq_version(void) { return 10300; }

}  // extern "C"
