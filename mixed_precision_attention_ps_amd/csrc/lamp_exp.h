// lamp_exp.h -- exponentials for the softmax, criterion and KL sums.
//
// exp64: double exp with Cody & Waite range reduction (Cody & Waite,
// "Software Manual for the Elementary Functions", 1980): n = rint(x / ln 2),
// r = x - n ln2_hi - n ln2_lo with a two-part ln 2 (ln2_hi has 32 significant
// bits, so n ln2_hi is exact for |n| < 2^21), then the Taylor polynomial of
// exp(r) to degree 12 for |r| <= ln2 / 2 (truncation < 1.7e-16 relative), then
// a power-of-two scale.  About 17 double operations; relative error within a
// few units of the last place, which keeps the strict criterion's double
// evaluation far inside the 1e-12 tie band the parity tests allow.
//
// exp_f32: an FP32-accurate exp of a double argument (probabilities): the
// argument is split in double into n + f, |f| <= 1/2, f is rounded to FP32
// (absolute error <= 2^-25) and 2^f is taken by the hardware exp2
// (v_exp_f32), then scaled by 2^n.  Relative error about 2e-7.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace lamp {

// Taylor coefficients 1/12!, 1/11!, ..., 1/2!, 1, 1 (Horner order).  They
// travel in every kernel's arguments so that they sit in scalar registers
// and each Horner step is one v_fma_f64 with a scalar operand.
struct ExpCoef {
    double c[13];
};

inline ExpCoef make_exp_coef()
{
    const ExpCoef k = {{0x1.1eed8eff8d898p-29, 0x1.ae64567f544e4p-26, 0x1.27e4fb7789f5cp-22,
                        0x1.71de3a556c734p-19, 0x1.a01a01a01a01ap-16, 0x1.a01a01a01a01ap-13,
                        0x1.6c16c16c16c17p-10, 0x1.1111111111111p-7, 0x1.5555555555555p-5,
                        0x1.5555555555555p-3, 0.5, 1.0, 1.0}};
    return k;
}

__device__ __forceinline__ double exp64(double x, const ExpCoef &k)
{
    const double kLog2e = 0x1.71547652b82fep+0;
    const double kLn2Hi = 0x1.62e42ff000000p-1;
    const double kLn2Lo = -0x1.718432a1b0e26p-35;
    // exp underflows to 0 below -745.2 and overflows above 709.8: clamping the
    // argument keeps the reduction exact and lets the final scale saturate
    // (NaN passes through)
    if (!(x != x))
        x = fmin(fmax(x, -750.0), 712.0);
    const double n = rint(x * kLog2e);
    double r = fma(-n, kLn2Hi, x);
    r = fma(-n, kLn2Lo, r);
    double p = k.c[0];
#pragma unroll
    for (int i = 1; i < 13; ++i)
        p = fma(p, r, k.c[i]);
    return ldexp(p, (int)n);
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
