/* Integer RNE of FP32 bit patterns to mu fraction bits, compared with a
 * rounding function passed in by pointer (the oracle's).  Test code. */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef double (*rn_fn)(double, int);

static uint32_t rn_bits(uint32_t u, int mu)
{
    int sh = 23 - mu;
    if (sh == 0)
        return u;
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return u;                                   /* NaN: unchanged */
    uint32_t half = 1u << (sh - 1);
    uint32_t lsb = (u >> sh) & 1u;
    return (u + half - 1u + lsb) & ~((1u << sh) - 1u);
}

/* Returns the number of mismatching patterns in [start, start+count);
 * the first one is stored in *first. */
int64_t rn_check_range(uint64_t start, uint64_t count, int mu, rn_fn rn, uint32_t *first)
{
    int64_t bad = 0;
    uint32_t fb = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (uint64_t i = 0; i < count; ++i) {
        uint32_t u = (uint32_t)(start + i);
        float f;
        memcpy(&f, &u, 4);
        float g = (float)rn((double)f, mu);
        uint32_t gu;
        memcpy(&gu, &g, 4);
        uint32_t w = rn_bits(u, mu);
        int ok = isnan(f) ? isnan(g) : (gu == w);
        if (!ok) {
            bad++;
#pragma omp critical
            fb = u;
        }
    }
    if (bad && first)
        *first = fb;
    return bad;
}
