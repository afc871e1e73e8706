/* Scalar CPU emulation of the shortened double exponentials of the HIP
 * kernels (exp64_crit: Taylor degree 4; exp64_sum: degree 3), test code:
 *
 *   n = rint(x * 64/ln2),  r = fma(-n, ln2/64 (one double), x),
 *   exp(x) = 2^(n >> 6) * T[n & 63] * (1 + p(r)),  T[k] = 2^(k/64),
 *
 * with p the Taylor polynomial of exp(r) - 1 to the given degree (Horner, as
 * the kernels evaluate it).  T is formed here from the long double exp2, not
 * copied from the kernels' table.  max_rel_error compares the emulation with
 * the long double expl at seeded random arguments. */
#include <math.h>
#include <stdint.h>

static double tab[64];
static int tab_ready = 0;

static void fill(void)
{
    if (tab_ready)
        return;
    for (int k = 0; k < 64; ++k)
        tab[k] = (double)exp2l((long double)k / 64.0L);
    tab_ready = 1;
}

double emu_exp64_short(double x, int deg)
{
    fill();
    const double k64Log2e = 0x1.71547652b82fep+6;
    const double kLn2_64 = 0x1.62e42fefa39efp-7;
    if (x == x)
        x = fmin(fmax(x, -750.0), 712.0);
    const double n = rint(x * k64Log2e);
    const double r = fma(-n, kLn2_64, x);
    double q;
    if (deg >= 4) {
        q = fma(r, 1.0 / 24.0, 1.0 / 6.0);
        q = fma(q, r, 0.5);
    } else {
        q = fma(r, 1.0 / 6.0, 0.5);
    }
    q = fma(q, r, 1.0);
    const double p = q * r;
    const int ni = (int)n;
    const double t = tab[ni & 63];
    return ldexp(fma(t, p, t), ni >> 6);
}

static inline uint64_t nextr(uint64_t *s)
{
    uint64_t z = (*s += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* Largest relative error over n arguments drawn uniformly from [lo, hi]
 * (results below the normal range are skipped). */
double max_rel_error(int deg, uint64_t seed, int64_t n, double lo, double hi)
{
    double worst = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double u = (double)(nextr(&seed) >> 11) * 0x1p-53;
        const double x = lo + (hi - lo) * u;
        const long double want = expl((long double)x);
        if (want < 0x1p-1022L)
            continue;
        const double got = emu_exp64_short(x, deg);
        const double rel = (double)fabsl(((long double)got - want) / want);
        if (rel > worst)
            worst = rel;
    }
    return worst;
}
