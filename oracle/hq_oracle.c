/*
 * hq_oracle.c -- plain, slow CPU oracle for the randomized Hadamard rotation
 * fused with symmetric per-row low-bit quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP kernels.
 *
 * Everything is computed in fp64 with explicit loops and no blocking, fusion
 * or reordering beyond the definitions below.  Pages cited:
 *   [HQA] "哈特曼旋转，轻量级QAT，流式注意力" (Q&A post on Hadamard rotation of
 *         Q/K), section 1.
 *   [QT]  "手把手教你用QuaRot实现LLM的4位量化：从原理到代码实践" (QuaRot
 *         tutorial), sections 2.1, 2.2 and 4.2.
 *   [RQ]  "旋转量化：大模型低比特量化中的离群值克星" (rotation-quantization
 *         blog), sections 1.1, 2.1 and 2.2.
 *   [MS]  "QuaRot：基于旋转的离群值抑制算法说明" (msModelSlim QuaRot page),
 *         section "原理" (principle) and the YAML field table.
 *
 * Definitions followed (all readings of the pages are listed in the
 * repository's design notes):
 *   H_1 = [1];  H_2m = [[H_m, H_m], [H_m, -H_m]]     Sylvester doubling,
 *        entries +-1, normalised once by 1/sqrt(b)     ([RQ] 2.1, [HQA] 1)
 *   u = x * s (elementwise sign flip, s shared by every row)   ([QT] 2.1)
 *   for each block k of b consecutive elements:  x'_blk = u_blk . H_b / sqrt(b)
 *        (block-diagonal rotation for widths that are not one power of two,
 *         [RQ] 2.1; b == n is the full rotation)
 *   m = max_i |x'_i| over the whole row; scale = m / qmax, qmax = 2^(bits-1)-1
 *   q_i = clamp(round_half_even(x'_i / scale), -qmax, qmax)   ([RQ] 2.2, [HQA] 1)
 *   Group-wise scales: the same, with m taken over each run of `group`
 *   consecutive elements of the rotated row and one scale per run, stored
 *   row by row ([RQ] 6.2 recommends group size 128 for 4 bits; [QT] 4.2
 *   keeps the scales of one group together).  group == n is the per-row
 *   case above.
 *   INT4 storage: two codes per byte, element 2j in the low nibble, 4-bit
 *   two's complement ([QT] 2.2 gives the 4x size reduction; the nibble
 *   order is this library's convention).
 *   Inverse: v = q * scale_stored (the scale of the element's group);
 *        x_hat_blk = (v_blk . H_b^T / sqrt(b)) * s
 *        (the normalised H is orthogonal, so its transpose undoes it: [MS]
 *         principle, [HQA] 1; the Sylvester matrix is also symmetric).
 *   Orders that are not a power of two: H_b = H_k (x) H_(b/k) with H_k from
 *   Paley's first construction (see hqo_hadamard_split / hqo_paley).
 *
 * Parity pins for every function are in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* Input / scale element types understood by the oracle (its own numbering). */
#define HQO_F32 0
#define HQO_BF16 1
#define HQO_F16 2

/* ---------------------------------------------------------------- helpers */

static int is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

/* IEEE binary16 -> double, exact.  value = (1024+M) * 2^(E-25) for normals,
 * M * 2^-24 for subnormals. */
double hqo_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* double -> IEEE binary16 with one round-half-to-even step (no double
 * rounding through float).  nearbyint() uses the default rounding mode,
 * which is round-to-nearest-even. */
uint16_t hqo_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return sign | 0x7e00;
    if (a >= 65520.0) /* halfway between 65504 and 2^16 rounds to even -> inf */
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) { /* subnormal quantum 2^-24 */
        double r = nearbyint(ldexp(a, 24));
        return sign | (uint16_t)r; /* r == 1024 is the smallest normal */
    }
    int e2;
    (void)frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;      /* a = 1.m * 2^E */
    double r = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7c00;
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(r - 1024.0);
}

/* bfloat16 -> double, exact (bf16 is the upper half of a binary32). */
static double bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

int hqo_decode(const void *src, int dtype, int64_t count, double *dst)
{
    if (count < 0 || (count > 0 && (!src || !dst)))
        return -1;
    for (int64_t i = 0; i < count; ++i) {
        if (dtype == HQO_F32)
            dst[i] = (double)((const float *)src)[i];
        else if (dtype == HQO_BF16)
            dst[i] = bf16_to_f64(((const uint16_t *)src)[i]);
        else if (dtype == HQO_F16)
            dst[i] = hqo_f16_to_f64(((const uint16_t *)src)[i]);
        else
            return -1;
    }
    return 0;
}

/* ------------------------------------------------------ Sylvester matrix */

/* Fills H (b*b, row-major) with the Sylvester Hadamard matrix of order b,
 * entries +1/-1, by repeated doubling H_2m = [[H_m, H_m], [H_m, -H_m]]
 * ([RQ] 2.1 prints H_2 and H_4 = H_2 (x) H_2; [HQA] 1 builds the same
 * recursion).  Returns 0, or -1 if b is not a power of two. */
static int sylvester(int b, int8_t *H)
{
    if (!is_pow2(b) || !H)
        return -1;
    H[0] = 1;
    for (int m = 1; m < b; m *= 2) {
        for (int i = 0; i < m; ++i) {
            for (int j = 0; j < m; ++j) {
                int8_t v = H[(int64_t)i * b + j];
                H[(int64_t)i * b + (j + m)] = v;
                H[(int64_t)(i + m) * b + j] = v;
                H[(int64_t)(i + m) * b + (j + m)] = (int8_t)-v;
            }
        }
    }
    return 0;
}

/* ------------------------------------- Paley matrices (non-power-of-two) */

/* Widths that are not a power of two ([MS] YAML table: the block size is a
 * power of two or the full width; [RQ] 2.1: H_4 = H_2 (x) H_2, larger orders
 * by Kronecker products).  Reading: H_n = H_k (x) H_(n/k), where n/k is a
 * power of two and H_k is Paley's first construction of order k = q + 1,
 * q = p^e a prime power with q = 3 (mod 4), k the smallest such order of the
 * form (odd part of n) * 2^a.  Element (i, j) of the Kronecker product has
 * index i * (n/k) + j.
 *
 * Paley's first construction: with GF(q) and its quadratic character chi
 * (chi(0) = 0, chi(a) = 1 if a is a nonzero square, -1 otherwise), the
 * Jacobsthal matrix Q[a][b] = chi(a - b) is skew-symmetric for q = 3 (mod 4)
 * and H = I + [[0, 1^T], [-1, Q]] has H H^T = (q + 1) I.  Conventions this
 * library fixes: GF(p^e) is GF(p)[x] modulo the monic irreducible polynomial
 * x^e + c_(e-1) x^(e-1) + ... + c_0 with the smallest index
 * c_0 + p c_1 + ... (e <= 3, where irreducible means "has no root"); an
 * element c_0 + c_1 x + c_2 x^2 has index c_0 + p c_1 + p^2 c_2; row and
 * column 0 of H belong to the extra point, row and column a + 1 to element a. */

/* q = p^e with p prime; returns 0, or -1 if q is not a prime power. */
static int prime_power(int q, int *p, int *e)
{
    if (q < 2)
        return -1;
    int f = 2;
    while (q % f != 0)
        ++f;
    int r = q, k = 0;
    while (r % f == 0) {
        r /= f;
        ++k;
    }
    if (r != 1)
        return -1;
    *p = f;
    *e = k;
    return 0;
}

static int ipow(int b, int e)
{
    int r = 1;
    while (e-- > 0)
        r *= b;
    return r;
}

/* the e coefficients of an element / of the modulus, lowest first */
static void digits(int a, int p, int e, int *c)
{
    for (int i = 0; i < e; ++i) {
        c[i] = a % p;
        a /= p;
    }
}

static int undigits(const int *c, int p, int e)
{
    int a = 0;
    for (int i = e - 1; i >= 0; --i)
        a = a * p + c[i];
    return a;
}

/* a * b in GF(p^e) = GF(p)[x] / (x^e + mod[e-1] x^(e-1) + ... + mod[0]) */
static int gf_mul(int a, int b, int p, int e, const int *mod)
{
    int ca[3], cb[3], prod[5] = {0, 0, 0, 0, 0};
    digits(a, p, e, ca);
    digits(b, p, e, cb);
    for (int i = 0; i < e; ++i)
        for (int j = 0; j < e; ++j)
            prod[i + j] = (prod[i + j] + ca[i] * cb[j]) % p;
    /* x^d = x^(d-e) * x^e and x^e = -(mod[e-1] x^(e-1) + ... + mod[0]) */
    for (int d = 2 * e - 2; d >= e; --d) {
        int c = prod[d];
        prod[d] = 0;
        for (int i = 0; i < e; ++i)
            prod[d - e + i] = ((prod[d - e + i] - c * mod[i]) % p + p) % p;
    }
    return undigits(prod, p, e);
}

static int gf_sub(int a, int b, int p, int e)
{
    int ca[3], cb[3], c[3];
    digits(a, p, e, ca);
    digits(b, p, e, cb);
    for (int i = 0; i < e; ++i)
        c[i] = ((ca[i] - cb[i]) % p + p) % p;
    return undigits(c, p, e);
}

/* the modulus of GF(p^e): the first monic polynomial of degree e (e <= 3)
 * without a root in GF(p), by the index of its lower coefficients */
static int gf_modulus(int p, int e, int *mod)
{
    if (e == 1) {
        mod[0] = 0; /* GF(p): arithmetic mod p; x^1 = 0 never used */
        return 0;
    }
    for (int c = 0; c < ipow(p, e); ++c) {
        digits(c, p, e, mod);
        int has_root = 0;
        for (int r = 0; r < p && !has_root; ++r) {
            int v = ipow(r, e) % p;
            for (int i = 0; i < e; ++i)
                v = (v + mod[i] * ipow(r, i)) % p;
            has_root = v == 0;
        }
        if (!has_root)
            return 0;
    }
    return -1;
}

/* Paley's first construction of order k (k - 1 = p^e = 3 mod 4, e <= 3):
 * H (k*k, row-major, +1/-1).  Returns 0, or -1 if k is not such an order. */
int hqo_paley(int k, int8_t *H)
{
    int q = k - 1, p = 0, e = 0, mod[3] = {0, 0, 0};
    if (!H || prime_power(q, &p, &e) != 0 || q % 4 != 3 || e > 3 || gf_modulus(p, e, mod) != 0)
        return -1;
    int8_t *square = (int8_t *)calloc((size_t)q, 1);
    if (!square)
        return -1;
    for (int a = 1; a < q; ++a)
        square[e == 1 ? (int)((int64_t)a * a % q) : gf_mul(a, a, p, e, mod)] = 1;
    for (int j = 0; j < k; ++j)
        H[j] = 1; /* row of the extra point: 1 on the diagonal, 1 elsewhere */
    for (int a = 0; a < q; ++a) {
        int8_t *row = H + (int64_t)(a + 1) * k;
        row[0] = -1;
        for (int b = 0; b < q; ++b) {
            int d = e == 1 ? ((a - b) % q + q) % q : gf_sub(a, b, p, e);
            int chi = d == 0 ? 0 : (square[d] ? 1 : -1);
            row[b + 1] = (int8_t)(chi + (a == b ? 1 : 0));
        }
    }
    free(square);
    return 0;
}

/* n = k * m2 as above (m2 a power of two, k a Paley order or k = 1 when n
 * itself is a power of two).  Returns 0, or -1 when n has no such split. */
int hqo_hadamard_split(int n, int *k, int *m2)
{
    if (n <= 0)
        return -1;
    if (is_pow2(n)) {
        *k = 1;
        *m2 = n;
        return 0;
    }
    int odd = n, twos = 1;
    while (odd % 2 == 0) {
        odd /= 2;
        twos *= 2;
    }
    for (int a = 1; a <= twos; a *= 2) {
        int kk = odd * a, q = kk - 1, p = 0, e = 0, mod[3];
        if (prime_power(q, &p, &e) == 0 && q % 4 == 3 && e <= 3 && gf_modulus(p, e, mod) == 0) {
            *k = kk;
            *m2 = twos / a;
            return 0;
        }
    }
    return -1;
}

/* The Hadamard matrix of order b this library rotates with: Sylvester for a
 * power of two, H_k (x) H_(b/k) otherwise (see above).  H is b*b, row-major,
 * +1/-1.  Returns 0, or -1 when b has no such matrix. */
int hqo_hadamard(int b, int8_t *H)
{
    int k = 0, m2 = 0;
    if (!H || hqo_hadamard_split(b, &k, &m2) != 0)
        return -1;
    if (k == 1)
        return sylvester(b, H);
    int8_t *P = (int8_t *)malloc((size_t)k * k);
    int8_t *S = (int8_t *)malloc((size_t)m2 * m2);
    int rc = -1;
    if (P && S && hqo_paley(k, P) == 0 && sylvester(m2, S) == 0) {
        for (int i = 0; i < k; ++i)
            for (int j = 0; j < m2; ++j)
                for (int i2 = 0; i2 < k; ++i2)
                    for (int j2 = 0; j2 < m2; ++j2)
                        H[((int64_t)i * m2 + j) * b + (int64_t)i2 * m2 + j2] =
                            (int8_t)(P[(int64_t)i * k + i2] * S[(int64_t)j * m2 + j2]);
        rc = 0;
    }
    free(P);
    free(S);
    return rc;
}

/* Builds H and Ht[i][j] = H[j][i].  The forward rotation u.H walks Ht
 * contiguously; the inverse v.H^T walks H.  (The Sylvester matrix is
 * symmetric and Paley matrices are not; the oracle transposes explicitly in
 * both cases.) */
static int make_mats(int b, int8_t **Hp, int8_t **Htp)
{
    int8_t *H = (int8_t *)malloc((size_t)b * b);
    int8_t *Ht = (int8_t *)malloc((size_t)b * b);
    if (!H || !Ht || hqo_hadamard(b, H) != 0) {
        free(H);
        free(Ht);
        return -1;
    }
    for (int i = 0; i < b; ++i)
        for (int j = 0; j < b; ++j)
            Ht[(int64_t)i * b + j] = H[(int64_t)j * b + i];
    *Hp = H;
    *Htp = Ht;
    return 0;
}

/* One row: out[kb+i] = sum_j (x[kb+j]*s[kb+j]) * M[i][j] / sqrt(b), with M
 * = Ht for the forward rotation u.H and M = H for the inverse v.H^T.  When
 * sums is not NULL it receives the same sums before the division by
 * sqrt(b). */
static void rotate_row(const double *x, const int8_t *s, int n, int b,
                       const int8_t *Ht, double *u, double *out, double *sums)
{
    double norm = sqrt((double)b);
    for (int i = 0; i < n; ++i)
        u[i] = s[i] < 0 ? -x[i] : x[i];
    for (int k = 0; k < n; k += b) {
        for (int i = 0; i < b; ++i) {
            const int8_t *hrow = Ht + (int64_t)i * b;
            double acc = 0.0;
            for (int j = 0; j < b; ++j)
                acc += u[k + j] * (double)hrow[j];
            if (sums)
                sums[k + i] = acc;
            out[k + i] = acc / norm;
        }
    }
}

/* ---------------------------------------------------------- quantisation */

static int qmax_of(int bits) { return (1 << (bits - 1)) - 1; }

/* Quantises one rotated row in groups of `group` consecutive elements (one
 * scale each; group == n is one scale per row).  xr is the rotated row x'
 * and sums the same values before the division by sqrt(b).  Writes the
 * packed codes, the stored scales [row * (n/group) + k] and optionally the
 * exact (fp64) scales (same index) and the pre-rounding values x'/scale.
 *
 * x'_i / scale = qmax * x'_i / max|x'| = qmax * sums_i / max|sums|: the
 * 1/sqrt(b) cancels, and the quotient is taken in that last form, so that a
 * value lying exactly on a .5 boundary (integer inputs, for instance) stays
 * exactly on it for every block size, irrational sqrt(b) included. */
static void quantize_row(const double *xr, const double *sums, int n, int group, int bits,
                         int scale_dtype, uint8_t *codes, void *scale_out, int64_t row,
                         double *scale_exact, double *preround)
{
    int qmax = qmax_of(bits);
    int ngroups = n / group;
    for (int k = 0; k < ngroups; ++k) {
        int i0 = k * group;
        int64_t si = row * ngroups + k;
        double m = 0.0, ms = 0.0;
        for (int i = i0; i < i0 + group; ++i) {
            if (fabs(xr[i]) > m)
                m = fabs(xr[i]);
            if (fabs(sums[i]) > ms)
                ms = fabs(sums[i]);
        }
        double scale = m / (double)qmax;
        if (scale_exact)
            scale_exact[si] = scale;
        if (scale_dtype == HQO_F32)
            ((float *)scale_out)[si] = (float)scale; /* C cast: round to nearest even */
        else
            ((uint16_t *)scale_out)[si] = hqo_f64_to_f16(scale);

        for (int i = i0; i < i0 + group; ++i) {
            /* all-zero group: codes 0 */
            double r = (ms > 0.0) ? ((double)qmax * sums[i]) / ms : 0.0;
            if (preround)
                preround[(int64_t)row * n + i] = r;
            double qd = nearbyint(r); /* round half to even */
            if (qd > qmax)
                qd = qmax;
            if (qd < -qmax)
                qd = -qmax;
            int q = (int)qd;
            if (bits == 8) {
                codes[(int64_t)row * n + i] = (uint8_t)(int8_t)q;
            } else {
                uint8_t *byte = codes + (int64_t)row * (n / 2) + i / 2;
                uint8_t nib = (uint8_t)(q & 0xf);
                if ((i & 1) == 0)
                    *byte = nib;
                else
                    *byte = (uint8_t)(*byte | (nib << 4));
            }
        }
    }
}

static int unpack_code(const uint8_t *codes, int64_t row, int n, int bits, int i)
{
    if (bits == 8)
        return (int)(int8_t)codes[row * n + i];
    uint8_t byte = codes[row * (n / 2) + i / 2];
    int nib = (i & 1) ? (byte >> 4) : (byte & 0xf);
    return nib >= 8 ? nib - 16 : nib;
}

static double stored_scale(const void *scales, int scale_dtype, int64_t index)
{
    if (scale_dtype == HQO_F32)
        return (double)((const float *)scales)[index];
    return hqo_f16_to_f64(((const uint16_t *)scales)[index]);
}

/* ------------------------------------------------------------- threading */

typedef struct {
    int kind; /* 0 rotate, 1 rotate+quant, 2 dequant+inverse */
    const void *x;
    int x_dtype;
    int64_t rows;
    int n, b, group, bits, scale_dtype;
    const int8_t *s;
    const int8_t *H, *Ht;
    double *xr;
    uint8_t *codes;
    void *scales;
    const uint8_t *codes_in;
    const void *scales_in;
    double *scale_exact, *preround, *y;
    int64_t r0, r1;
    int err;
} job_t;

static void *worker(void *arg)
{
    job_t *j = (job_t *)arg;
    int n = j->n;
    double *xin = (double *)malloc(sizeof(double) * n);
    double *u = (double *)malloc(sizeof(double) * n);
    double *out = (double *)malloc(sizeof(double) * n);
    double *sums = (double *)malloc(sizeof(double) * n);
    int8_t *ones = (int8_t *)malloc((size_t)n); /* unit signs for the inverse */
    if (!xin || !u || !out || !sums || !ones) {
        j->err = -2;
        goto done;
    }
    memset(ones, 1, (size_t)n);
    for (int64_t r = j->r0; r < j->r1; ++r) {
        if (j->kind == 0) {
            rotate_row((const double *)j->x + r * n, j->s, n, j->b, j->Ht, u,
                       j->xr + r * n, NULL);
        } else if (j->kind == 1) {
            size_t esz = j->x_dtype == HQO_F32 ? 4 : 2;
            hqo_decode((const char *)j->x + (size_t)r * n * esz, j->x_dtype, n, xin);
            rotate_row(xin, j->s, n, j->b, j->Ht, u, out, sums);
            if (j->xr)
                memcpy(j->xr + r * n, out, sizeof(double) * n);
            quantize_row(out, sums, n, j->group, j->bits, j->scale_dtype, j->codes, j->scales, r,
                         j->scale_exact, j->preround);
        } else {
            /* v = q * scale_stored (of the element's group), then v.H/sqrt(b)
             * per block, then * s. */
            int ngroups = n / j->group;
            for (int i = 0; i < n; ++i) {
                double sc = stored_scale(j->scales_in, j->scale_dtype,
                                         r * ngroups + i / j->group);
                xin[i] = (double)unpack_code(j->codes_in, r, n, j->bits, i) * sc;
            }
            rotate_row(xin, ones, n, j->b, j->H, u, out, NULL);
            for (int i = 0; i < n; ++i)
                j->y[r * n + i] = j->s[i] < 0 ? -out[i] : out[i];
        }
    }
done:
    free(ones);
    free(xin);
    free(u);
    free(out);
    free(sums);
    return NULL;
}

static int run_jobs(job_t *tmpl, int threads)
{
    if (tmpl->rows == 0)
        return 0;
    if (threads <= 0)
        threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (threads < 1)
        threads = 1;
    if ((int64_t)threads > tmpl->rows)
        threads = (int)tmpl->rows;
    int8_t *H = NULL, *Ht = NULL;
    if (make_mats(tmpl->b, &H, &Ht) != 0)
        return -2;
    tmpl->H = H;
    tmpl->Ht = Ht;
    job_t *jobs = (job_t *)calloc((size_t)threads, sizeof(job_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    int rc = 0;
    if (!jobs || !tids) {
        rc = -2;
        goto out;
    }
    for (int t = 0; t < threads; ++t) {
        jobs[t] = *tmpl;
        jobs[t].r0 = tmpl->rows * t / threads;
        jobs[t].r1 = tmpl->rows * (t + 1) / threads;
        if (pthread_create(&tids[t], NULL, worker, &jobs[t]) != 0) {
            jobs[t].err = -3;
            tids[t] = 0;
        }
    }
    for (int t = 0; t < threads; ++t) {
        if (tids[t])
            pthread_join(tids[t], NULL);
        if (jobs[t].err)
            rc = jobs[t].err;
    }
out:
    free(jobs);
    free(tids);
    free(H);
    free(Ht);
    return rc;
}

static int check_shape(int64_t rows, int n, int b, const int8_t *s)
{
    int k = 0, m2 = 0;
    if (rows < 0 || n <= 0 || b <= 0 || n % b != 0 || !s || hqo_hadamard_split(b, &k, &m2) != 0)
        return -1;
    return 0;
}

/* ------------------------------------------------------------ public API */

/* Rotation only: xr = blockwise (x*s).H_b/sqrt(b), x already decoded to fp64. */
int hqo_rotate(const double *x, int64_t rows, int n, int b, const int8_t *s,
               double *xr, int threads)
{
    if (check_shape(rows, n, b, s) || (rows > 0 && (!x || !xr)))
        return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.kind = 0;
    j.x = x;
    j.rows = rows;
    j.n = n;
    j.b = b;
    j.s = s;
    j.xr = xr;
    return run_jobs(&j, threads);
}

/* Rotation + quantisation straight from the raw input bytes, one scale per
 * run of `group` consecutive rotated elements (group must divide n).
 * codes: [rows, n/2] (bits 4) or [rows, n] (bits 8);  scales: [rows, n/group]
 * fp32 or fp16 bits.  scale_exact [rows, n/group], preround [rows*n] and
 * xr [rows*n] are optional diagnostics (NULL to skip). */
int hqo_rotate_quant_g(const void *x, int x_dtype, int64_t rows, int n, int b,
                       const int8_t *s, int bits, int group, uint8_t *codes, void *scales,
                       int scale_dtype, double *scale_exact, double *preround,
                       double *xr, int threads)
{
    if (check_shape(rows, n, b, s))
        return -1;
    if (group <= 0 || n % group != 0 || (bits == 4 && group % 2 != 0))
        return -1;
    if (bits != 4 && bits != 8)
        return -1;
    if (bits == 4 && n % 2 != 0)
        return -1;
    if (x_dtype != HQO_F32 && x_dtype != HQO_BF16 && x_dtype != HQO_F16)
        return -1;
    if (scale_dtype != HQO_F32 && scale_dtype != HQO_F16)
        return -1;
    if (rows > 0 && (!x || !codes || !scales))
        return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.kind = 1;
    j.x = x;
    j.x_dtype = x_dtype;
    j.rows = rows;
    j.n = n;
    j.b = b;
    j.group = group;
    j.bits = bits;
    j.scale_dtype = scale_dtype;
    j.s = s;
    j.codes = codes;
    j.scales = scales;
    j.scale_exact = scale_exact;
    j.preround = preround;
    j.xr = xr;
    return run_jobs(&j, threads);
}

/* Per-row scales: the group-wise function with group == n. */
int hqo_rotate_quant(const void *x, int x_dtype, int64_t rows, int n, int b,
                     const int8_t *s, int bits, uint8_t *codes, void *scales,
                     int scale_dtype, double *scale_exact, double *preround,
                     double *xr, int threads)
{
    return hqo_rotate_quant_g(x, x_dtype, rows, n, b, s, bits, n, codes, scales,
                              scale_dtype, scale_exact, preround, xr, threads);
}

/* Dequantisation + inverse rotation with group-wise scales [rows, n/group]:
 * y = ((q*scale_stored) . H_b/sqrt(b)) * s. */
int hqo_dequant_rotate_inv_g(const uint8_t *codes, const void *scales,
                             int scale_dtype, int64_t rows, int n, int b,
                             const int8_t *s, int bits, int group, double *y, int threads)
{
    if (check_shape(rows, n, b, s))
        return -1;
    if (group <= 0 || n % group != 0 || (bits == 4 && group % 2 != 0))
        return -1;
    if (bits != 4 && bits != 8)
        return -1;
    if (bits == 4 && n % 2 != 0)
        return -1;
    if (scale_dtype != HQO_F32 && scale_dtype != HQO_F16)
        return -1;
    if (rows > 0 && (!codes || !scales || !y))
        return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.kind = 2;
    j.codes_in = codes;
    j.scales_in = scales;
    j.scale_dtype = scale_dtype;
    j.rows = rows;
    j.n = n;
    j.b = b;
    j.group = group;
    j.bits = bits;
    j.s = s;
    j.y = y;
    return run_jobs(&j, threads);
}

/* Per-row scales: the group-wise inverse with group == n. */
int hqo_dequant_rotate_inv(const uint8_t *codes, const void *scales,
                           int scale_dtype, int64_t rows, int n, int b,
                           const int8_t *s, int bits, double *y, int threads)
{
    return hqo_dequant_rotate_inv_g(codes, scales, scale_dtype, rows, n, b, s, bits, n, y,
                                    threads);
}

/* Decode attention over a rotated, quantised K/V cache: the consumer of the
 * codes written above.  [QT] 2.2: K and V are rotated online, stored as 4-bit
 * codes and dequantised when attention reads them; [HQA] 1: rotating Q and K
 * with the same orthogonal matrix leaves Q.K^T unchanged, so the query is
 * rotated with the cache's rotation.  One query token per head:
 *   q        [q_heads, n] (q_dtype), not rotated
 *   k_codes, v_codes   [tokens, kv_heads, n/2] (bits 4) or [.., n] (bits 8)
 *   k_scales, v_scales [tokens, kv_heads] (scale_dtype), one per row
 *   query head h reads kv head h / (q_heads / kv_heads)
 *   q'   = (q * s) . H_b / sqrt(b)              the cache's rotation
 *   k_t  = code_k[t] * scale_k[t], v_t likewise  (rotated, dequantised)
 *   a_t  = exp(c_t - max c) / sum_u exp(c_u - max c),  c_t = q'.k_t / sqrt(n)
 *   o'   = sum_t a_t v_t                          (rotated space)
 *   o    = (o' . H_b / sqrt(b)) * s               back to the query's space
 * out [q_heads, n], double.  Returns 0, or -1 on invalid arguments. */
int hqo_decode_attention(const void *q, int q_dtype, int q_heads, int kv_heads, int n, int b,
                         const int8_t *s, int64_t tokens, int bits, const uint8_t *k_codes,
                         const void *k_scales, const uint8_t *v_codes, const void *v_scales,
                         int scale_dtype, double *out)
{
    if (check_shape(1, n, b, s) || q_heads <= 0 || kv_heads <= 0 || q_heads % kv_heads != 0)
        return -1;
    if (tokens <= 0 || (bits != 4 && bits != 8) || (bits == 4 && n % 2 != 0))
        return -1;
    if (scale_dtype != HQO_F32 && scale_dtype != HQO_F16)
        return -1;
    if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !out)
        return -1;
    int8_t *H = NULL, *Ht = NULL;
    if (make_mats(b, &H, &Ht) != 0)
        return -2;
    double *qin = (double *)malloc(sizeof(double) * n);
    double *qr = (double *)malloc(sizeof(double) * n);
    double *u = (double *)malloc(sizeof(double) * n);
    double *o = (double *)malloc(sizeof(double) * n);
    double *c = (double *)malloc(sizeof(double) * (size_t)tokens);
    int8_t *ones = (int8_t *)malloc((size_t)n);
    int err = 0;
    if (!Ht || !qin || !qr || !u || !o || !c || !ones) {
        err = -2;
        goto done;
    }
    memset(ones, 1, (size_t)n);
    size_t qsz = q_dtype == HQO_F32 ? 4 : 2;
    int group = q_heads / kv_heads;
    for (int h = 0; h < q_heads; ++h) {
        int kh = h / group;
        if (hqo_decode((const char *)q + (size_t)h * n * qsz, q_dtype, n, qin)) {
            err = -1;
            goto done;
        }
        rotate_row(qin, s, n, b, Ht, u, qr, NULL);
        double cmax = -INFINITY;
        for (int64_t t = 0; t < tokens; ++t) {
            int64_t row = t * kv_heads + kh; /* the row of (token t, kv head kh) */
            double sc = stored_scale(k_scales, scale_dtype, row);
            double dot = 0.0;
            for (int i = 0; i < n; ++i)
                dot += qr[i] * ((double)unpack_code(k_codes, row, n, bits, i) * sc);
            c[t] = dot / sqrt((double)n);
            if (c[t] > cmax)
                cmax = c[t];
        }
        double denom = 0.0;
        for (int64_t t = 0; t < tokens; ++t) {
            c[t] = exp(c[t] - cmax);
            denom += c[t];
        }
        for (int i = 0; i < n; ++i)
            o[i] = 0.0;
        for (int64_t t = 0; t < tokens; ++t) {
            int64_t row = t * kv_heads + kh;
            double w = c[t] / denom * stored_scale(v_scales, scale_dtype, row);
            for (int i = 0; i < n; ++i)
                o[i] += w * (double)unpack_code(v_codes, row, n, bits, i);
        }
        /* back to the query's space: o . H_b^T / sqrt(b), then * s */
        rotate_row(o, ones, n, b, H, u, qin, NULL);
        for (int i = 0; i < n; ++i)
            out[(int64_t)h * n + i] = s[i] < 0 ? -qin[i] : qin[i];
    }
done:
    free(H);
    free(Ht);
    free(qin);
    free(qr);
    free(u);
    free(o);
    free(c);
    free(ones);
    return err;
}

/* Number of worker threads a call with threads<=0 would use. */
int hqo_default_threads(void) { return (int)sysconf(_SC_NPROCESSORS_ONLN); }
