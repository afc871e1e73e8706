/* Scalar CPU emulation of the FP32 instruction sequence the HIP kernels use
 * for PS(mu) arithmetic (test code, checked against the oracle):
 *
 *   product  p = fl(q*k); C = sign(p) * 2^exponent(p) (sign and exponent
 *            bits of p); r_s = fma(q_s, k, C) - C, where q_s = q * 2^(mu-23).
 *            The fma adds the exact scaled product to C (same sign, so the
 *            magnitude stays in C's binade) with one rounding at C's ulp,
 *            which is the PS(mu) ulp of the product scaled by 2^(mu-23); C is
 *            2^23 ulps (even), so ties go to even.  Result: RN_mu(q*k) *
 *            2^(mu-23), exactly.
 *   sum      s = fl(acc_s + r_s), then RNE of s to mu fraction bits by
 *            Veltkamp's splitting with the constant 2^(23-mu) + 1:
 *            g = fl(C s), hi = fl(g + fl(s - g)) (innocuous double rounding for
 *            mu <= 10).  check_split_exhaustive compares that splitting with
 *            the integer RNE of the bits over every FP32 input.
 *   score    fl(acc_s * (scale * 2^(23-mu))).
 *
 * Valid when every nonzero |q|, |k| lies in [2^-40, 2^40] (products and sums
 * stay normal in the scaled domain) and mu <= 10. */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef double (*rn_fn)(double, int);

static inline uint32_t fb(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static inline float bf(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float emu_prod_scaled(float q, float k, int mu)
{
    float qs = ldexpf(q, mu - 23);
    float p = q * k;
    float C = bf(fb(p) & 0xff800000u);
    float t = fmaf(qs, k, C);
    return t - C;
}

/* integer RNE of s's bits to mu fraction bits */
static float emu_round_bits(float s, int mu)
{
    uint32_t u = fb(s);
    int sh = 23 - mu;
    uint32_t half = 1u << (sh - 1);
    u = (u + ((u >> sh) & 1u) + (half - 1u)) & ~((1u << sh) - 1u);
    return bf(u);
}

/* the kernels' form: Veltkamp's splitting (three separately rounded FP32 ops) */
float emu_round(float s, int mu)
{
    const float C = (float)((1u << (23 - mu)) + 1u);
    volatile float g = C * s;
    volatile float d = s - g;
    return g + d;
}

/* Every FP32 pattern with a finite normal value of magnitude below 2^100, and
 * +0 (the fast path's sums: never -0, nonzero magnitudes far above the
 * subnormals, below 2^75): the splitting against the integer RNE.  Returns
 * the number of mismatches; the first one in *first. */
int64_t check_split_exhaustive(int mu, uint32_t *first)
{
    int64_t bad = 0;
    uint32_t fst = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = 0; i < (1LL << 32); ++i) {
        const uint32_t u = (uint32_t)i;
        const uint32_t e = (u >> 23) & 0xffu;
        if (e >= 127 + 100 || (e == 0 && u != 0u))
            continue;
        const float x = bf(u);
        if (fb(emu_round(x, mu)) != fb(emu_round_bits(x, mu))) {
            if (bad == 0) {
#pragma omp critical
                fst = u;
            }
            bad++;
        }
    }
    *first = fst;
    return bad;
}

float emu_ps_score(const float *q, const float *k, int D, int mu, float scale)
{
    float acc = 0.0f;
    for (int d = 0; d < D; ++d) {
        float r = emu_prod_scaled(q[d], k[d], mu);
        float s = acc + r;
        acc = emu_round(s, mu);
    }
    float sc = ldexpf(scale, 23 - mu);
    return acc * sc;
}

/* xorshift64* stream for test inputs */
static inline uint64_t nextr(uint64_t *s)
{
    uint64_t x = *s;
    x ^= x >> 12; x ^= x << 25; x ^= x >> 27;
    *s = x;
    return x * 0x2545f4914f6cdd1dULL;
}

static float rand_operand(uint64_t *st, int emin, int emax)
{
    uint64_t r = nextr(st);
    int e = emin + (int)(r % (uint64_t)(emax - emin + 1));
    uint32_t mant = (uint32_t)(r >> 40) & 0x7fffffu;
    uint32_t sign = (uint32_t)(r >> 63) << 31;
    return bf(sign | ((uint32_t)(e + 127) << 23) | mant);
}

/* Products: n random pairs with exponents in [emin, emax].  Returns the
 * number of mismatches against rn(q*k); *traps counts pairs whose FP32
 * product sits exactly on a PS(mu) midpoint while the exact product does not
 * (where rounding the FP32 product again would be wrong). */
int64_t check_products(uint64_t seed, int64_t n, int mu, int emin, int emax, rn_fn rn,
                       int64_t *traps)
{
    int64_t bad = 0, tr = 0;
    uint64_t st = seed | 1;
    int sh = 23 - mu;
    for (int64_t i = 0; i < n; ++i) {
        float q = rand_operand(&st, emin, emax);
        float k = rand_operand(&st, emin, emax);
        double exact = (double)q * (double)k;
        float want = (float)rn(exact, mu);
        float got = ldexpf(emu_prod_scaled(q, k, mu), 23 - mu);
        if (fb(got) != fb(want))
            bad++;
        float p = q * k;
        uint32_t low = fb(p) & ((1u << sh) - 1u);
        if (low == (1u << (sh - 1)) && (double)p != exact)
            tr++;
    }
    *traps = tr;
    return bad;
}

/* Sums: all ordered pairs of PS(mu) values with binade exponents in
 * [emin, emax] (both signs, all mantissas), fp32 add + integer RNE compared
 * with rn(exact double sum).  Returns mismatches. */
int64_t check_sums_exhaustive(int mu, int emin, int emax, rn_fn rn)
{
    int nm = 1 << mu;
    int64_t nv = (int64_t)(emax - emin + 1) * nm * 2;
    int64_t bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bad)
    for (int64_t a = 0; a < nv; ++a) {
        int64_t ia = a;
        uint32_t sa = (uint32_t)(ia & 1) << 31; ia >>= 1;
        uint32_t ma = (uint32_t)(ia % nm) << (23 - mu); ia /= nm;
        float x = bf(sa | ((uint32_t)(emin + ia + 127) << 23) | ma);
        for (int64_t b = 0; b < nv; ++b) {
            int64_t ib = b;
            uint32_t sb = (uint32_t)(ib & 1) << 31; ib >>= 1;
            uint32_t mb = (uint32_t)(ib % nm) << (23 - mu); ib /= nm;
            float y = bf(sb | ((uint32_t)(emin + ib + 127) << 23) | mb);
            float got = emu_round(x + y, mu);
            float want = (float)rn((double)x + (double)y, mu);
            if (fb(got) != fb(want))
                bad++;
        }
    }
    return bad;
}

/* Random sums with wide exponent gaps (double sum not exact): compared with
 * rn(double sum).  Returns mismatches. */
int64_t check_sums_random(uint64_t seed, int64_t n, int mu, int emin, int emax, rn_fn rn)
{
    uint64_t st = seed | 1;
    int64_t bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        float x = (float)rn((double)rand_operand(&st, emin, emax), mu);
        float y = (float)rn((double)rand_operand(&st, emin, emax), mu);
        float got = emu_round(x + y, mu);
        float want = (float)rn((double)x + (double)y, mu);
        if (fb(got) != fb(want))
            bad++;
    }
    return bad;
}
