// 8-bit packed directions, device side (gfx950).
//
// The ZOO blog ("Backprop 없이 Transformer를 학습시킨다", section "첫 번째 논문:
// probe-space 사전조건화(1.5-SPSA)") trains OPT-30B in place with an 8-bit
// packing random generator and a fused unpack/apply kernel; the pages give no
// format.  Here one Philox4x32-10 block yields sixteen 8-bit codes, one per
// element, and a code k stands for the k-th of 256 equal-probability Gaussian
// quantiles, scaled to unit variance:
//
//   element j of direction i under seed s: byte (j mod 4) (least significant
//   first) of word ((j / 4) mod 4) of Philox4x32-10 with key (s lo, s hi) and
//   counter (q lo, q hi, i, 1), q = j / 16;
//   T[k] = x_k / r,  x_k = Phi^-1((k + 1/2) / 256),  r^2 = (1/256) sum_k x_k^2,
//   rounded once to fp32.
//
// The counter's last word (1) keeps these streams apart from the Gaussian
// directions (last word 0).  Codes are uniform over 0..255, so the values are
// symmetric with mean 0 and variance 1, which keeps E[z z^T] = I for the
// estimator.  The table is evaluated at compile time in fp64 from the series
// below and placed in the code object: no device-side state to initialise.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zo_rng.hpp"

namespace zo {
namespace dirs8 {

constexpr double kLn2d = 0.693147180559945309417232121458176568;
constexpr double kInvSqrt2Pi = 0.398942280401432677939946059934381868;

// exp(x) for x <= 0 of moderate size: x = m ln2 + t, |t| <= ln2 / 2, Taylor
// series of exp(t), then the power of two applied by halving.
constexpr double c_exp(double x)
{
    const double f = x / kLn2d;
    const int m = (int)(f < 0 ? f - 0.5 : f + 0.5);
    const double t = x - m * kLn2d;
    double term = 1.0, sum = 1.0;
    for (int n = 1; n < 30; ++n) {
        term *= t / n;
        sum += term;
    }
    for (int i = 0; i < (m < 0 ? -m : m); ++i) sum = m < 0 ? sum * 0.5 : sum * 2.0;
    return sum;
}

// standard normal density
constexpr double c_pdf(double x) { return kInvSqrt2Pi * c_exp(-0.5 * x * x); }

// Phi(x) for x >= 0: 1/2 + pdf(x) * sum_n x^(2n+1) / (1 3 5 ... (2n+1)), a
// series of positive terms (no cancellation).
constexpr double c_cdf(double x)
{
    double term = x, sum = x;
    for (int n = 1; n < 200; ++n) {
        term *= x * x / (2 * n + 1);
        sum += term;
        if (term < sum * 1e-20) break;
    }
    return 0.5 + c_pdf(x) * sum;
}

// Phi^-1(p) for p in (1/2, 1): Newton from 0.  Phi is concave on x > 0, so
// the iterates increase monotonically to the root.
constexpr double c_quantile(double p)
{
    double x = 0.0;
    for (int it = 0; it < 60; ++it) {
        const double dx = (c_cdf(x) - p) / c_pdf(x);
        x -= dx;
        if (dx > -1e-17 && dx < 1e-17) break;
    }
    return x;
}

constexpr double c_sqrt(double v)
{
    double r = v > 1.0 ? v : 1.0;
    for (int it = 0; it < 100; ++it) r = 0.5 * (r + v / r);
    return r;
}

struct Table {
    float v[256];
};

constexpr Table make_table()
{
    double x[128] = {};
    double ss = 0.0;
    for (int k = 0; k < 128; ++k) {  // upper half: codes 128 + k
        x[k] = c_quantile((128 + k + 0.5) / 256.0);
        ss += x[k] * x[k];
    }
    const double r = c_sqrt(2.0 * ss / 256.0);
    Table t = {};
    for (int k = 0; k < 128; ++k) {
        const float v = (float)(x[k] / r);
        t.v[128 + k] = v;
        t.v[127 - k] = -v;  // Phi^-1(1 - p) = -Phi^-1(p)
    }
    return t;
}

constexpr Table kTable = make_table();
static_assert(kTable.v[0] == -kTable.v[255] && kTable.v[127] < 0.0f && kTable.v[128] > 0.0f, "q8 table");
// device copy, in the code object's constant data
__constant__ const Table kTableDev = make_table();

// The four Philox words of block q (16 codes) of direction `probe`.
__device__ __forceinline__ uint4 block(Key key, uint32_t probe, uint64_t q)
{
    uint32_t c0 = (uint32_t)q, c1 = (uint32_t)(q >> 32), c2 = probe, c3 = 1u;
    philox4x32_10(c0, c1, c2, c3, key);
    return uint4{c0, c1, c2, c3};
}

// Table into LDS; call with every thread of the block, then __syncthreads().
__device__ __forceinline__ void load_table(float* lds)
{
    for (int k = threadIdx.x; k < 256; k += blockDim.x) lds[k] = kTableDev.v[k];
}

__device__ __forceinline__ float code(const float* lds, uint32_t word, int b)
{
    return lds[(word >> (8 * b)) & 0xFFu];
}

// Value of element j alone (slow path for ragged tails).
__device__ __forceinline__ float value1(const float* lds, Key key, uint32_t probe, uint64_t j)
{
    const uint4 w = block(key, probe, j >> 4);
    const uint32_t sel = (uint32_t)(j >> 2) & 3u;
    const uint32_t word = sel == 0 ? w.x : sel == 1 ? w.y : sel == 2 ? w.z : w.w;
    return code(lds, word, (int)(j & 3u));
}

}  // namespace dirs8
}  // namespace zo
