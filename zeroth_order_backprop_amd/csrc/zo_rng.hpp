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
// The fp32 evaluation works in base-2 logarithms: sqrt(-log2 u_r) from the
// hardware log2 and rsq with one Newton correction carried as a residual, the
// constant sqrt(2 ln 2) folded into minimax sin/cos polynomials of a quarter
// turn after an exact integer quadrant reduction, and one rounding of the
// final product.
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

// ---- Box-Muller in base-2 logarithms ----
// With m = -log2 u_r the radius is sqrt(-2 ln u_r) = K sqrt(m), K = sqrt(2 ln 2).
// K is carried by the quarter-turn polynomials below, so the radius needs only
// sqrt(m), and m itself is the hardware log2 negated (no rounded -2 ln 2 factor).
//
// K sin(pi t / 2) = t (kS1 + kS3 t^2 + kS5 t^4 + kS7 t^6) and
// K cos(pi t / 2) = kC0 + kC2 t^2 + ... + kC8 t^8 on t in [-1/2, 1/2]: minimax
// fits (Remez exchange, absolute error) with fp32 coefficients chosen for the
// smallest error of the fp32 Horner evaluation over every reduced angle
// t = i 2^-22; derived by gen_trig_coefs.py beside this header.  Evaluated in
// fp32 they stay within 6.5e-8 (sin) and 7.7e-8 (cos) of the exact values;
// kC0 is the fp32 value nearest K (0.13 of its last place off).
constexpr float kS1 = 0x1.d976f4p+0f;    // 1.84947133
constexpr float kS3 = -0x1.85688ep-1f;   // -0.760563314
constexpr float kS5 = 0x1.80402cp-4f;    // 0.0938111991
constexpr float kS7 = -0x1.625a8cp-8f;   // -0.00540700834
constexpr float kC0 = 0x1.2d6abep+0f;    // 1.17741001
constexpr float kC2 = -0x1.73dbb6p+0f;   // -1.45257127
constexpr float kC4 = 0x1.31d74p-2f;     // 0.298672676
constexpr float kC6 = -0x1.9267b8p-6f;   // -0.0245608613
constexpr float kC8 = 0x1.16e82p-10f;    // 0.00106394477

// v_mul_legacy_f32: a product in which a zero operand gives 0 even against an
// infinity (the LLVM intrinsic, reached through its symbol name).
__device__ float fmul_zero_safe(float a, float b) __asm("llvm.amdgcn.fmul.legacy");

// sqrt(-log2 u_r) for u_r = (a + 1) 2^-24, a = x >> 8, as R + R_lo.  u_r is
// exact in fp32 and the hardware log2 (v_log_f32) is within one ulp on every
// one of these 2^24 inputs.  R = m rsq(m) and R_lo = (m - R^2) rsq(m) / 2 is
// one Newton correction, so R + R_lo is sqrt(m) to well below fp32 rounding.
// The zero-safe multiply (0 times anything is 0) makes u_r = 1, m = 0, give
// R = R_lo = 0 although rsq(0) is infinite.
__device__ __forceinline__ void log2_radius(uint32_t x, float& R, float& R_lo)
{
    const float u = fmaf((float)(x >> 8), 0x1p-24f, 0x1p-24f);
    const float m = -__builtin_amdgcn_logf(u);           // >= 0
    const float y = __builtin_amdgcn_rsqf(m);
    R = fmul_zero_safe(m, y);
    const float res = fmaf(-R, R, m);
    R_lo = fmul_zero_safe(res, 0.5f * y);
}

// K (cos, sin) of 2 pi u_t for u_t = (x >> 8) 2^-24.  The angle's 24 bits are
// b = x >> 8; the nearest quarter turn is k = (b + 2^21) >> 22 and the rest
// t = (b - k 2^22) 2^-22 is the sign-extended low 22 bits of b, read straight
// from x.  Rotating (cos, sin)(pi t / 2) by k quarter turns swaps the pair for
// odd k and negates: the cos part for k = 1, 2 and the sin part for k = 2, 3
// (k mod 4).  With y = x + 2^29 (mod 2^32), bit 30 of y is k's low bit, bit 31
// its high bit, and bit 31 of y + 2^30 is set exactly for k = 1, 2.
__device__ __forceinline__ void unit_circle_k(uint32_t x, float& c, float& s)
{
    const int ti = (int)(x << 2) >> 10;                  // bits 8..29 of x, sign-extended
    const float t = (float)ti * 0x1p-22f;                // exact, in [-1/2, 1/2)
    const float t2 = t * t;
    float ps = fmaf(kS7, t2, kS5);
    ps = fmaf(ps, t2, kS3);
    ps = fmaf(ps, t2, kS1);
    const float st = ps * t;                             // K sin(pi t / 2)
    float ct = fmaf(kC8, t2, kC6);
    ct = fmaf(ct, t2, kC4);
    ct = fmaf(ct, t2, kC2);
    ct = fmaf(ct, t2, kC0);                              // K cos(pi t / 2)
    const uint32_t y = x + (1u << 29), y2 = x + (3u << 29);
    const uint32_t odd = (uint32_t)((int)(y << 1) >> 31); // all ones for odd k
    const uint32_t sb = __float_as_uint(st), cb = __float_as_uint(ct);
    const uint32_t a0 = (odd & sb) | (~odd & cb);
    const uint32_t a1 = (odd & cb) | (~odd & sb);
    c = __uint_as_float(a0 ^ (y2 & 0x80000000u));
    s = __uint_as_float(a1 ^ (y & 0x80000000u));
}

// Box-Muller pair from two words.
__device__ __forceinline__ void box_muller(uint32_t x_even, uint32_t x_odd, float& z_even, float& z_odd)
{
    float R, R_lo, c, s;
    log2_radius(x_even, R, R_lo);
    unit_circle_k(x_odd, c, s);
    z_even = fmaf(c, R, c * R_lo);
    z_odd = fmaf(s, R, s * R_lo);
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
