// Device math shared by the GEMM epilogues.
#pragma once
#include <hip/hip_runtime.h>

namespace zo {

// GELU in its exact form x Phi(x), Phi the standard normal CDF, evaluated
// through the complementary error function, Phi(x) = erfc(-x / sqrt 2) / 2:
//   x >= 0:  x (1 - erfc(a) / 2),   x < 0:  x erfc(a) / 2,   a = |x| / sqrt 2.
// erfc(a) = t exp(-a^2 + P(t)), t = 1 / (1 + a / 2), with P the degree-9
// Chebyshev fit of Press, Teukolsky, Vetterling and Flannery (Numerical
// Recipes in C, 2nd ed., section 6.2, routine erfcc), whose fractional error
// is below 1.2e-7 for every a >= 0.  Working with erfc instead of 1 + erf
// keeps the negative tail relatively accurate (no cancellation), and
// a^2 = x^2 / 2 is carried as an exact two-term fp32 sum, so the exponent's
// rounding stays at fp32 level.  Relative error in fp32: below 1e-6 for
// x > -3 and below 3e-6 down to x = -6 (checked against fp64 on a dense grid);
// no branches, about 20 VALU operations.
__device__ __forceinline__ float gelu_erf(float x)
{
    const float a = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, a, 1.0f));
    float p = 0.17087277f;
    p = fmaf(p, t, -0.82215223f);
    p = fmaf(p, t, 1.48851587f);
    p = fmaf(p, t, -1.13520398f);
    p = fmaf(p, t, 0.27886807f);
    p = fmaf(p, t, -0.18628806f);
    p = fmaf(p, t, 0.09678418f);
    p = fmaf(p, t, 0.37409196f);
    p = fmaf(p, t, 1.00002368f);
    p = fmaf(p, t, -1.26551223f);
    const float sh = x * x;
    const float sl = fmaf(x, x, -sh);            // x^2 = sh + sl exactly
    const float arg = fmaf(-0.5f, sh, p) - 0.5f * sl;
    const float e = t * __builtin_amdgcn_exp2f(arg * 1.44269504088896341f);
    return x * (x >= 0.0f ? fmaf(-0.5f, e, 1.0f) : 0.5f * e);
}

}  // namespace zo
