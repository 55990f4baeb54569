// hq_paley.hip -- host side of the rotations whose width is not a power of
// two: the factorisation n = k * m2 and the field GF(k - 1) behind Paley's
// first construction of H_k.
//
// Pages cited: [RQ] "旋转量化：大模型低比特量化中的离群值克星" section 2.1 (larger
// Hadamard matrices as Kronecker products of smaller ones); [MS]
// "QuaRot：基于旋转的离群值抑制算法说明" YAML field table (the block size is a power of
// two or the whole width).  The matrix of order k itself is Paley's (1933):
// H = I + [[0, 1^T], [-1, Q]], Q[a][b] = chi(a - b) over GF(q), q = 3 mod 4.
#include "hq_internal.h"

namespace hq {
namespace {

// q = p^e with p prime (trial division; q is at most a few thousand)
bool prime_power(int q, int &p, int &e)
{
    if (q < 2)
        return false;
    int d = 2;
    for (; d * d <= q; ++d)
        if (q % d == 0)
            break;
    if (d * d > q)
        d = q;  // q is prime
    int r = q;
    e = 0;
    while (r % d == 0) {
        r /= d;
        ++e;
    }
    p = d;
    return r == 1;
}

// value of x^e + mod[e-1] x^(e-1) + ... + mod[0] at x = r, mod p
int poly_at(int r, int p, int e, const int *mod)
{
    int v = 1;
    for (int i = 0; i < e; ++i)
        v = v * r % p;
    int xi = 1;
    for (int i = 0; i < e; ++i) {
        v = (v + mod[i] * xi) % p;
        xi = xi * r % p;
    }
    return v;
}

// the first monic polynomial of degree e (e <= 3) without a root in GF(p);
// for degree 2 and 3 that is irreducibility
bool field_modulus(int p, int e, int *mod)
{
    if (e == 1)
        return true;
    int count = 1;
    for (int i = 0; i < e; ++i)
        count *= p;
    for (int idx = 0; idx < count; ++idx) {
        int t = idx;
        for (int i = 0; i < e; ++i) {
            mod[i] = t % p;
            t /= p;
        }
        bool root = false;
        for (int r = 0; r < p && !root; ++r)
            root = poly_at(r, p, e, mod) == 0;
        if (!root)
            return true;
    }
    return false;
}

}  // namespace

bool hadamard_split(int n, PaleySpec &ps)
{
    ps = PaleySpec{};
    if (n <= 0)
        return false;
    int odd = n, twos = 1;
    while ((odd & 1) == 0) {
        odd >>= 1;
        twos <<= 1;
    }
    if (odd == 1) {
        ps.m2 = n;
        return true;
    }
    for (int a = 1; a <= twos; a <<= 1) {
        const int k = odd * a, q = k - 1;
        int p = 0, e = 0;
        if (q % 4 != 3 || !prime_power(q, p, e) || e > 3)
            continue;
        int mod[3] = {0, 0, 0};
        if (!field_modulus(p, e, mod))
            continue;
        ps.k = k;
        ps.m2 = twos / a;
        ps.p = p;
        ps.e = e;
        for (int i = 0; i < 3; ++i)
            ps.mod[i] = mod[i];
        return true;
    }
    return false;
}

}  // namespace hq
