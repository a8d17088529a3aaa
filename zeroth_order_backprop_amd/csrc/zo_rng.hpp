// Direction generator for the SPSA step, device side (gfx950).
//
// Directions are never stored: element j of direction i under step seed s is
// recomputed wherever it is needed (perturb, fused GEMM prologue, update) from
// (s, i, j) alone, which is what lets the perturbation be rebuilt from a seed
// plus scalars ("0 차 최적화는 미탐구된 것이지, 저전력이 아니다", P5; FedSPZO
// summary, section 2, "통신 프로토콜").  The directions are Gaussian (same
// position paper, P1).
//
// Counter-based stream: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// Random Numbers: As Easy as 1, 2, 3", SC'11) with key = (s lo, s hi) and
// counter = (q lo, q hi, i, 0), q = j / 4; word j % 4 belongs to element j.
// Words (x0, x1) feed elements 4q, 4q+1 and (x2, x3) feed 4q+2, 4q+3 through
// Box-Muller: u_r = ((x_even >> 8) + 1) 2^-24, u_t = (x_odd >> 8) 2^-24,
// r = sqrt(-2 ln u_r), (z_even, z_odd) = r (cos 2 pi u_t, sin 2 pi u_t).
//
// The fp32 evaluation: ln u_r from the hardware log2 with the scaling carried
// exactly, sin/cos of a quarter turn via their Taylor series on [-pi/4, pi/4]
// after an exact integer quadrant reduction, and sqrt carried as a value plus
// its residual so the final product is rounded once.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zo {

struct Key {
    uint32_t k0, k1;
};

__device__ __forceinline__ Key make_key(uint64_t seed)
{
    return Key{(uint32_t)seed, (uint32_t)(seed >> 32)};
}

// One Philox4x32-10 block for counter (c0, c1, c2, c3).
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                              Key key)
{
    constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
    constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
    uint32_t k0 = key.k0, k1 = key.k1;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t pa = (uint64_t)c0 * kMulA;
        const uint64_t pb = (uint64_t)c2 * kMulB;
        // three-way xor in one v_bitop3_b32 (truth table 0x96 = a ^ b ^ c)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(pb >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(pa >> 32), c3, k1, 0x96);
        c1 = (uint32_t)pb;
        c3 = (uint32_t)pa;
        c0 = n0;
        c2 = n2;
        k0 += kWeylA;
        k1 += kWeylB;
    }
}

// ---- constants from the series definitions (evaluated at compile time) ----
constexpr double kPi = 3.14159265358979323846264338327950288;
constexpr double kHalfPi = kPi / 2.0;

constexpr double cpow(double x, int n) { return n == 0 ? 1.0 : x * cpow(x, n - 1); }
constexpr double cfact(int n) { return n <= 1 ? 1.0 : n * cfact(n - 1); }
// sin(pi t / 2) = sum_k (-1)^k (pi/2)^(2k+1) t^(2k+1) / (2k+1)!
constexpr double sin_coef(int k) { return (k % 2 ? -1.0 : 1.0) * cpow(kHalfPi, 2 * k + 1) / cfact(2 * k + 1); }
// cos(pi t / 2) = sum_k (-1)^k (pi/2)^(2k) t^(2k) / (2k)!
constexpr double cos_coef(int k) { return (k % 2 ? -1.0 : 1.0) * cpow(kHalfPi, 2 * k) / cfact(2 * k); }
constexpr float kS1 = (float)sin_coef(0), kS3 = (float)sin_coef(1), kS5 = (float)sin_coef(2),
                kS7 = (float)sin_coef(3), kS9 = (float)sin_coef(4);
constexpr float kC2 = (float)cos_coef(1), kC4 = (float)cos_coef(2), kC6 = (float)cos_coef(3),
                kC8 = (float)cos_coef(4), kC10 = (float)cos_coef(5);
constexpr double kLn2 = 0.693147180559945309417232121458176568;

// -2 ln(u_r) for u_r = (a + 1) 2^-24, a = x >> 8, as L + L_lo.  u_r is exact
// in fp32; the hardware log2 (v_log_f32) is within one ulp on every one of
// these 2^24 inputs, and the factor -2 ln 2 is applied in two parts so that
// L + L_lo carries no further rounding.
constexpr float kM2Ln2Hi = (float)(-2.0 * kLn2);
constexpr float kM2Ln2Lo = (float)(-2.0 * kLn2 - (double)kM2Ln2Hi);
__device__ __forceinline__ void minus_two_log_radius(uint32_t x, float& L, float& L_lo)
{
    const float u = (float)((x >> 8) + 1u) * 0x1p-24f;
    const float l2 = __builtin_amdgcn_logf(u);
    L = l2 * kM2Ln2Hi;
    L_lo = fmaf(l2, kM2Ln2Lo, fmaf(l2, kM2Ln2Hi, -L));
}

// (cos, sin) of 2 pi u_t for u_t = (x >> 8) 2^-24.
__device__ __forceinline__ void unit_circle(uint32_t x, float& c, float& s)
{
    const uint32_t b = x >> 8;                           // 24-bit angle
    const uint32_t k = (b + (1u << 21)) >> 22;           // nearest quarter turn, 0..4
    const int ti = (int)b - (int)(k << 22);              // in [-2^21, 2^21)
    const float t = (float)ti * 0x1p-22f;                // exact, in [-1/2, 1/2)
    const float t2 = t * t;
    float ps = kS9;
    ps = fmaf(ps, t2, kS7);
    ps = fmaf(ps, t2, kS5);
    ps = fmaf(ps, t2, kS3);
    ps = fmaf(ps, t2, kS1);
    const float st = ps * t;                             // sin(pi t / 2)
    float pc = kC10;
    pc = fmaf(pc, t2, kC8);
    pc = fmaf(pc, t2, kC6);
    pc = fmaf(pc, t2, kC4);
    pc = fmaf(pc, t2, kC2);
    const float ct = fmaf(pc, t2, 1.0f);                 // cos(pi t / 2)
    // rotate by k quarter turns: (cos, sin)(theta + k pi/2)
    const uint32_t q = k & 3u;
    const float a0 = (q & 1u) ? st : ct;
    const float a1 = (q & 1u) ? ct : st;
    c = ((q + 1u) & 2u) ? -a0 : a0;                      // q = 1, 2 negate cos part
    s = (q & 2u) ? -a1 : a1;                             // q = 2, 3 negate sin part
}

// Box-Muller pair from two words.
__device__ __forceinline__ void box_muller(uint32_t x_even, uint32_t x_odd, float& z_even, float& z_odd)
{
    float L, L_lo;
    minus_two_log_radius(x_even, L, L_lo);               // L >= 0
    const float r = __builtin_amdgcn_sqrtf(L);
    // r + r_lo = sqrt(L + L_lo) to well below fp32 rounding; r_lo = (L + L_lo - r^2) / (2 r)
    const float res = fmaf(-r, r, L) + L_lo;
    const float r_lo = (L > 0.0f) ? res * (0.5f * __builtin_amdgcn_rcpf(r)) : 0.0f;
    float c, s;
    unit_circle(x_odd, c, s);
    z_even = fmaf(c, r, c * r_lo);
    z_odd = fmaf(s, r, s * r_lo);
}

// Four Gaussians for elements 4q .. 4q+3 of counter stream `stream` of
// direction `probe` (stream 0: the weight directions; the Dust estimator's
// activation noise uses streams 2 and 3).
__device__ __forceinline__ float4 gauss4s(Key key, uint32_t probe, uint32_t stream, uint64_t q)
{
    uint32_t c0 = (uint32_t)q, c1 = (uint32_t)(q >> 32), c2 = probe, c3 = stream;
    philox4x32_10(c0, c1, c2, c3, key);
    float4 z;
    box_muller(c0, c1, z.x, z.y);
    box_muller(c2, c3, z.z, z.w);
    return z;
}

// Four Gaussians for elements 4q .. 4q+3 of direction `probe`.
__device__ __forceinline__ float4 gauss4(Key key, uint32_t probe, uint64_t q)
{
    uint32_t c0 = (uint32_t)q, c1 = (uint32_t)(q >> 32), c2 = probe, c3 = 0u;
    philox4x32_10(c0, c1, c2, c3, key);
    float4 z;
    box_muller(c0, c1, z.x, z.y);
    box_muller(c2, c3, z.z, z.w);
    return z;
}

}  // namespace zo
