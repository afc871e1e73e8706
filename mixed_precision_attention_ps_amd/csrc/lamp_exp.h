// lamp_exp.h -- exponentials for the softmax, criterion and KL sums.
//
// exp64: double exp by table-driven range reduction (Tang, "Table-driven
// implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989, with a 64-entry table):
//   n = rint(x * 64 / ln 2),  r = x - n (ln2/64)_hi - n (ln2/64)_lo,
//   |r| <= ln 2 / 128,
//   exp(x) = 2^(n >> 6) * T[n & 63] * (1 + p(r)),  T[k] = 2^(k/64),
// p(r) = r + r^2/2 + ... + r^5/120 (Taylor; the first omitted term is below
// 3.6e-17 relative).  (ln2/64)_hi has 29 significant bits, so n (ln2/64)_hi
// is exact for |n| < 2^24.  Twelve double operations, one LDS read and a
// power-of-two scale; relative error within about one unit of the last place,
// far inside the 1e-12 tie band of the strict and relaxed criteria.
//
// The table T lives in LDS: every kernel that calls exp64 declares a
// 64-double shared array, fills it with exp_table_fill and synchronises its
// block before the first call.
//
// exp64_crit / exp64_sum: shorter forms of exp64 for the hot loops, with the
// same table and range reduction except that ln 2 / 64 is taken as one double
// (its rounding error, 3.6e-19, times |n| <= 7e4 moves r by at most 2.5e-14)
// and the Taylor polynomial stops earlier:
//   exp64_crit, degree 4: remainder below r^5/120 <= 3.9e-14 relative (6.4e-14
//     with the reduction's error at the ends of the range), for
//     values that decide a look-ahead criterion (a decision must agree with an
//     exact evaluation outside a 1e-12 relative band around the threshold);
//   exp64_sum, degree 3: remainder below r^4/24 <= 3.6e-11 relative, for sums
//     that only normalise probabilities or enter a KL (1e-7 bars).
//
// exp_f32: an FP32-accurate exp of a double argument (probabilities): the
// argument is split in double into n + f, |f| <= 1/2, f is rounded to FP32
// (absolute error <= 2^-25) and 2^f is taken by the hardware exp2
// (v_exp_f32), then scaled by 2^n.  Relative error about 2e-7.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace lamp {

// 2^(k/64), k = 0..63, each correctly rounded to double.
static __constant__ double kExp2Frac64[64] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0,
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0,
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0,
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0,
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0,
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0,
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0,
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0,
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0,
};

// Copies the table into a block's LDS array (the caller then synchronises
// the block).
__device__ __forceinline__ void exp_table_fill(double *s_tab)
{
    for (unsigned k = threadIdx.x; k < 64; k += blockDim.x)
        s_tab[k] = kExp2Frac64[k];
}

// The reduction, polynomial and scale, for x in [-750, 712].
__device__ __forceinline__ double exp64_core(double x, const double *s_tab)
{
    const double k64Log2e = 0x1.71547652b82fep+6;    // 64 / ln 2
    const double kLn2Hi = 0x1.62e42ff000000p-7;      // (ln 2 / 64), 29 bits
    const double kLn2Lo = -0x1.718432a1b0e26p-41;    // the rest of ln 2 / 64
    const double n = rint(x * k64Log2e);
    double r = fma(-n, kLn2Hi, x);
    r = fma(-n, kLn2Lo, r);
    double q = fma(r, 1.0 / 120.0, 1.0 / 24.0);
    q = fma(q, r, 1.0 / 6.0);
    q = fma(q, r, 0.5);
    q = fma(q, r, 1.0);
    const double p = q * r;   // exp(r) - 1
    const int ni = (int)n;
    const double t = s_tab[ni & 63];
    return ldexp(fma(t, p, t), ni >> 6);
}

__device__ __forceinline__ double exp64(double x, const double *s_tab)
{
    // exp underflows to 0 below -745.2 and overflows above 709.8: clamping the
    // argument keeps the reduction exact and lets the final scale saturate
    // (NaN passes through)
    if (!(x != x))
        x = fmin(fmax(x, -750.0), 712.0);
    return exp64_core(x, s_tab);
}

// exp of an argument that is <= 0 or -inf (a score minus its row maximum);
// a NaN argument gives 0, so a caller that must propagate NaN checks for it.
__device__ __forceinline__ double exp64_nonpos(double x, const double *s_tab)
{
    return exp64_core(fmax(x, -750.0), s_tab);
}

template <int DEG>
__device__ __forceinline__ double exp64_short_core(double x, const double *s_tab)
{
    const double k64Log2e = 0x1.71547652b82fep+6;    // 64 / ln 2
    const double kLn2_64 = 0x1.62e42fefa39efp-7;     // ln 2 / 64, rounded to double
    const double n = rint(x * k64Log2e);
    const double r = fma(-n, kLn2_64, x);
    double q;
    if constexpr (DEG >= 4) {
        q = fma(r, 1.0 / 24.0, 1.0 / 6.0);
        q = fma(q, r, 0.5);
    } else {
        q = fma(r, 1.0 / 6.0, 0.5);
    }
    q = fma(q, r, 1.0);
    const double p = q * r;   // exp(r) - 1
    const int ni = (int)n;
    const double t = s_tab[ni & 63];
    return ldexp(fma(t, p, t), ni >> 6);
}

// (argument handling as exp64 and exp64_nonpos)
__device__ __forceinline__ double exp64_crit(double x, const double *s_tab)
{
    if (!(x != x))
        x = fmin(fmax(x, -750.0), 712.0);
    return exp64_short_core<4>(x, s_tab);
}

__device__ __forceinline__ double exp64_crit_nonpos(double x, const double *s_tab)
{
    return exp64_short_core<4>(fmax(x, -750.0), s_tab);
}

__device__ __forceinline__ double exp64_sum(double x, const double *s_tab)
{
    if (!(x != x))
        x = fmin(fmax(x, -750.0), 712.0);
    return exp64_short_core<3>(x, s_tab);
}

__device__ __forceinline__ double exp64_sum_nonpos(double x, const double *s_tab)
{
    return exp64_short_core<3>(fmax(x, -750.0), s_tab);
}

__device__ __forceinline__ float exp_f32(double x)
{
    const double kLog2e = 0x1.71547652b82fep+0;
    double t = x * kLog2e;
    t = fmin(fmax(t, -300.0), 300.0);
    const double n = rint(t);
    const float f = (float)(t - n);
    const float r = __builtin_amdgcn_exp2f(f);
    return ldexpf(r, (int)n);
}

}  // namespace lamp
