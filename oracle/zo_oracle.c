/*
 * CPU oracle for the multi-probe SPSA step: direction generator, perturbation
 * and update.  TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this library; the product path
 * never does.  It shares no code, header, table or constant generator with the
 * HIP kernels.
 *
 * Plain, single-threaded, written for clarity: one element at a time, in the
 * order the method states.  Built with -O2 -ffp-contract=off so that no
 * multiply-add is fused unless written as fma() below.
 *
 * What the method computes (sources):
 *  - "Backprop 없이 Transformer를 학습시킨다" (thakicloud ZOO blog), section
 *    "zero-order optimization이란": SPSA takes two forwards per probe, at +1
 *    and -1 times a random perturbation.
 *  - same page, section "backprop의 메모리 세금", loop flowchart: draw N random
 *    directions, perturb W by +-delta*Delta_i, evaluate the loss only, form
 *    the SPSA estimate, update W <- W - eta*g_hat.
 *  - "0 차 최적화는 미탐구된 것이지, 저전력이 아니다" (gist.science 2605.15622),
 *    P1 (Gaussian directions) and P5 (directions rebuilt from a shared seed).
 *  - FedSPZO summary (gist.science 2502.10239), section 2 "통신 프로토콜":
 *    perturbation vectors are regenerated from seeds, so the exact model is
 *    rebuilt from scalars plus seeds.
 * The pages give no generator, no counter layout and no Gaussian map; the
 * readings taken here are:
 *  - Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 *    Easy as 1, 2, 3", SC'11): 10 rounds of the 4x32 Philox S-box with
 *    multipliers 0xD2511F53 / 0xCD9E8D57 and Weyl key increments
 *    0x9E3779B9 / 0xBB67AE85.
 *  - Direction element j of probe i under seed s: key = (s lo, s hi),
 *    counter = (q lo, q hi, i, 0) with q = j / 4, word j mod 4 of the output.
 *  - Words (x0, x1) give elements 4q, 4q+1 and (x2, x3) give 4q+2, 4q+3 by
 *    Box-Muller: u_r = ((x_even >> 8) + 1) * 2^-24 in (0, 1],
 *    u_t = (x_odd >> 8) * 2^-24 in [0, 1), r = sqrt(-2 ln u_r),
 *    z_even = r cos(2 pi u_t), z_odd = r sin(2 pi u_t); evaluated in fp64 and
 *    rounded once to fp32.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

/* One Philox4x32-10 block: ten rounds, key bumped between rounds. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)c[0];
        uint64_t p1 = (uint64_t)PHILOX_M1 * (uint64_t)c[2];
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c[1] ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c[3] ^ k1;
        uint32_t n3 = lo0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* The four words that cover element j of stream `stream` of direction
   `probe` under `seed` (stream 0: weight directions). */
static void stream_block(uint64_t seed, uint32_t probe, uint32_t stream, uint64_t j, uint32_t w[4])
{
    uint64_t q = j >> 2;
    uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), probe, stream};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    oracle_philox4x32_10(ctr, key, w);
}

static void direction_block(uint64_t seed, uint32_t probe, uint64_t j, uint32_t w[4])
{
    stream_block(seed, probe, 0u, j, w);
}

/* Raw words for elements j0 .. j0+n-1 (word j mod 4 of block j/4). */
void oracle_rng_words(uint64_t seed, uint32_t probe, uint64_t j0, uint64_t n, uint32_t* out)
{
    for (uint64_t t = 0; t < n; ++t) {
        uint64_t j = j0 + t;
        uint32_t w[4];
        direction_block(seed, probe, j, w);
        out[t] = w[j & 3u];
    }
}

/* Box-Muller on one word pair, in fp64.  Returns z_even, writes z_odd. */
double oracle_box_muller_f64(uint32_t x_even, uint32_t x_odd, double* z_odd)
{
    const double two_pi = 6.283185307179586476925286766559;
    double u_r = ((double)(x_even >> 8) + 1.0) * 0x1p-24;
    double u_t = (double)(x_odd >> 8) * 0x1p-24;
    double r = sqrt(-2.0 * log(u_r));
    *z_odd = r * sin(two_pi * u_t);
    return r * cos(two_pi * u_t);
}

/* ---- 8-bit packed directions -------------------------------------------
 * Reading of the ZOO blog's 1.5-SPSA section (an 8-bit packing random
 * generator with a fused unpack/apply kernel; no format given): element j of
 * direction `probe` is byte j mod 4 (least significant first) of word
 * (j / 4) mod 4 of the Philox block with counter (q lo, q hi, probe, 1),
 * q = j / 16, and byte value k stands for table[k], the k-th of 256
 * equal-probability Gaussian quantiles scaled to unit variance.  The table is
 * supplied by the caller (oracle.py builds it from the normal quantile
 * function); every routine below takes it as `q8`, NULL meaning Gaussian
 * directions. */
static float q8_value(uint64_t seed, uint32_t probe, uint64_t j, const float* q8)
{
    uint64_t q = j >> 4;
    uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), probe, 1u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oracle_philox4x32_10(ctr, key, w);
    uint32_t word = w[(j >> 2) & 3u];
    unsigned byte = (word >> (8u * (unsigned)(j & 3u))) & 0xFFu;
    return q8[byte];
}

/* Gaussian direction value of element j, fp64 definition rounded once to fp32. */
static float gauss_value(uint64_t seed, uint32_t probe, uint64_t j)
{
    uint32_t w[4];
    direction_block(seed, probe, j, w);
    unsigned pair = (unsigned)(j & 3u) >> 1; /* 0: words 0,1   1: words 2,3 */
    double zo;
    double ze = oracle_box_muller_f64(w[2 * pair], w[2 * pair + 1], &zo);
    return (float)((j & 1u) ? zo : ze);
}

/* Gaussian values of another counter stream (same Box-Muller map): the
   activation noise of the Dust estimator uses streams 2 (hidden layer) and
   3 (logits), element j = row * width + column. */
void oracle_gauss_stream(uint64_t seed, uint32_t probe, uint32_t stream, uint64_t j0, uint64_t n, float* z)
{
    for (uint64_t t = 0; t < n; ++t) {
        uint64_t j = j0 + t;
        uint32_t w[4];
        stream_block(seed, probe, stream, j, w);
        unsigned pair = (unsigned)(j & 3u) >> 1;
        double zo;
        double ze = oracle_box_muller_f64(w[2 * pair], w[2 * pair + 1], &zo);
        z[t] = (float)((j & 1u) ? zo : ze);
    }
}

static float dir_value(uint64_t seed, uint32_t probe, uint64_t j, const float* q8)
{
    return q8 ? q8_value(seed, probe, j, q8) : gauss_value(seed, probe, j);
}

static void gauss_impl(uint64_t seed, uint32_t probe, uint64_t j0, uint64_t n, float* z, const float* q8)
{
    for (uint64_t t = 0; t < n; ++t)
        z[t] = dir_value(seed, probe, j0 + t, q8);
}

/* Same, at strided element indices idx[0..n). */
static void gauss_at_impl(uint64_t seed, uint32_t probe, const uint64_t* idx, uint64_t n, float* z, const float* q8)
{
    for (uint64_t t = 0; t < n; ++t)
        z[t] = dir_value(seed, probe, idx[t], q8);
}

/* ---- bfloat16: round to nearest, ties to even ---------------------------- */

/* fp32 -> bf16 bits.  NaN stays NaN (quiet), infinities and overflow as IEEE. */
uint16_t oracle_bf16_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xFFFFu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u; /* carries into the exponent correctly, up to infinity */
    return (uint16_t)upper;
}

float oracle_f32_from_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp64 -> bf16, one rounding from the fp64 value (normal and subnormal). */
uint16_t oracle_bf16_from_f64(double x)
{
    if (isnan(x)) return 0x7FC0u;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (a == 0.0) return sign;
    /* bf16 keeps 8 significant bits; spacing at a is 2^(e-8) for a in
       [2^(e-1), 2^e), never below the subnormal spacing 2^-133. */
    int e;
    frexp(a, &e);
    int ex = e - 8;
    if (ex < -133) ex = -133;
    double q = ldexp(a, -ex);          /* exact: a power-of-two scaling */
    double qr = nearbyint(q);          /* current mode: ties to even */
    double v = ldexp(qr, ex);
    if (v > 3.3895313892515355e+38) return sign | 0x7F80u; /* beyond max: inf */
    float vf = (float)v;               /* exact: v has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &vf, 4);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

/* ---- perturbation: w <- round_storage(w + sigma * z_j) ------------------- */

static void perturb_f32_impl(float* w, uint64_t n, uint64_t j0, uint64_t seed, uint32_t probe, float sigma, const float* q8)
{
    for (uint64_t t = 0; t < n; ++t) {
        float z = dir_value(seed, probe, j0 + t, q8);
        w[t] = fmaf(sigma, z, w[t]); /* exact sigma*z + w, rounded once */
    }
}

static void perturb_bf16_impl(uint16_t* w, uint64_t n, uint64_t j0, uint64_t seed, uint32_t probe, float sigma, const float* q8)
{
    for (uint64_t t = 0; t < n; ++t) {
        float z = dir_value(seed, probe, j0 + t, q8);
        double v = (double)oracle_f32_from_bf16(w[t]) + (double)sigma * (double)z;
        w[t] = oracle_bf16_from_f64(v);
    }
}

/* ---- update: w <- round_storage(w + sum_i c_i z_i[j]) --------------------- */

static void update_f32_impl(float* w, uint64_t n, uint64_t j0, uint64_t seed,
                       uint32_t n_probes, const double* c, const float* q8)
{
    for (uint64_t t = 0; t < n; ++t) {
        double acc = 0.0;
        for (uint32_t i = 0; i < n_probes; ++i)
            acc += c[i] * (double)dir_value(seed, i, j0 + t, q8);
        w[t] = (float)((double)w[t] + acc);
    }
}

static void update_bf16_impl(uint16_t* w, uint64_t n, uint64_t j0, uint64_t seed,
                        uint32_t n_probes, const double* c, const float* q8)
{
    for (uint64_t t = 0; t < n; ++t) {
        double acc = 0.0;
        for (uint32_t i = 0; i < n_probes; ++i)
            acc += c[i] * (double)dir_value(seed, i, j0 + t, q8);
        w[t] = oracle_bf16_from_f64((double)oracle_f32_from_bf16(w[t]) + acc);
    }
}

/* Same updates at strided element indices (for sampled checks on large
   parameter vectors): w[t] is element idx[t]. */
static void update_f32_at_impl(float* w, const uint64_t* idx, uint64_t n, uint64_t seed,
                          uint32_t n_probes, const double* c, const float* q8)
{
    for (uint64_t t = 0; t < n; ++t) {
        double acc = 0.0;
        for (uint32_t i = 0; i < n_probes; ++i)
            acc += c[i] * (double)dir_value(seed, i, idx[t], q8);
        w[t] = (float)((double)w[t] + acc);
    }
}

static void update_bf16_at_impl(uint16_t* w, const uint64_t* idx, uint64_t n, uint64_t seed,
                           uint32_t n_probes, const double* c, const float* q8)
{
    for (uint64_t t = 0; t < n; ++t) {
        double acc = 0.0;
        for (uint32_t i = 0; i < n_probes; ++i)
            acc += c[i] * (double)dir_value(seed, i, idx[t], q8);
        w[t] = oracle_bf16_from_f64((double)oracle_f32_from_bf16(w[t]) + acc);
    }
}

static void perturb_f32_at_impl(float* w, const uint64_t* idx, uint64_t n, uint64_t seed,
                           uint32_t probe, float sigma, const float* q8)
{
    for (uint64_t t = 0; t < n; ++t)
        w[t] = fmaf(sigma, dir_value(seed, probe, idx[t], q8), w[t]);
}

static void perturb_bf16_at_impl(uint16_t* w, const uint64_t* idx, uint64_t n, uint64_t seed,
                            uint32_t probe, float sigma, const float* q8)
{
    for (uint64_t t = 0; t < n; ++t) {
        float z = dir_value(seed, probe, idx[t], q8);
        double v = (double)oracle_f32_from_bf16(w[t]) + (double)sigma * (double)z;
        w[t] = oracle_bf16_from_f64(v);
    }
}

/* Exhaustive fp32 -> bf16 over a range of bit patterns; writes mismatches
   against a caller-provided bf16 table (used to check this rounding against an
   independent library in bulk).  Returns the number of mismatches. */
uint64_t oracle_bf16_compare_range(uint32_t start, uint32_t count, const uint16_t* expect)
{
    uint64_t bad = 0;
    for (uint32_t t = 0; t < count; ++t) {
        uint32_t u = start + t;
        float f;
        memcpy(&f, &u, 4);
        uint16_t h = oracle_bf16_from_f32(f);
        uint16_t e = expect[t];
        int fnan = ((u & 0x7F800000u) == 0x7F800000u) && (u & 0x007FFFFFu);
        if (fnan) {
            if ((e & 0x7F80u) != 0x7F80u || (e & 0x7Fu) == 0) ++bad; /* both NaN */
        } else if (h != e) {
            ++bad;
        }
    }
    return bad;
}

/* In-place fp64 -> nearest bf16 value (kept as fp64), for the model forwards'
   declared bf16 rounding points. */
void oracle_round_bf16_array(double* x, uint64_t n)
{
    for (uint64_t t = 0; t < n; ++t)
        x[t] = (double)oracle_f32_from_bf16(oracle_bf16_from_f64(x[t]));
}

/* In-place fp64 -> nearest fp32 value (kept as fp64). */
void oracle_round_f32_array(double* x, uint64_t n)
{
    for (uint64_t t = 0; t < n; ++t)
        x[t] = (double)(float)x[t];
}

/* Box-Muller over an array of word pairs: out[2t], out[2t+1] in fp64. */
void oracle_box_muller_f64_array(const uint32_t* pairs, uint64_t n_pairs, double* out)
{
    for (uint64_t t = 0; t < n_pairs; ++t) {
        double zo;
        out[2 * t] = oracle_box_muller_f64(pairs[2 * t], pairs[2 * t + 1], &zo);
        out[2 * t + 1] = zo;
    }
}

/* ---- public entry points: Gaussian directions, and the same routines with

 * 8-bit directions from the 256-value table `q8` ------------------------- */

void oracle_gauss(uint64_t seed, uint32_t probe, uint64_t j0, uint64_t n, float* z)
{
    gauss_impl(seed, probe, j0, n, z, NULL);
}

void oracle_q8_values(uint64_t seed, uint32_t probe, uint64_t j0, uint64_t n, float* z, const float* q8)
{
    gauss_impl(seed, probe, j0, n, z, q8);
}

void oracle_gauss_at(uint64_t seed, uint32_t probe, const uint64_t* idx, uint64_t n, float* z)
{
    gauss_at_impl(seed, probe, idx, n, z, NULL);
}

void oracle_q8_values_at(uint64_t seed, uint32_t probe, const uint64_t* idx, uint64_t n, float* z, const float* q8)
{
    gauss_at_impl(seed, probe, idx, n, z, q8);
}

void oracle_perturb_f32(float* w, uint64_t n, uint64_t j0, uint64_t seed, uint32_t probe, float sigma)
{
    perturb_f32_impl(w, n, j0, seed, probe, sigma, NULL);
}

void oracle_q8_perturb_f32(float* w, uint64_t n, uint64_t j0, uint64_t seed, uint32_t probe, float sigma, const float* q8)
{
    perturb_f32_impl(w, n, j0, seed, probe, sigma, q8);
}

void oracle_perturb_bf16(uint16_t* w, uint64_t n, uint64_t j0, uint64_t seed, uint32_t probe, float sigma)
{
    perturb_bf16_impl(w, n, j0, seed, probe, sigma, NULL);
}

void oracle_q8_perturb_bf16(uint16_t* w, uint64_t n, uint64_t j0, uint64_t seed, uint32_t probe, float sigma, const float* q8)
{
    perturb_bf16_impl(w, n, j0, seed, probe, sigma, q8);
}

void oracle_update_f32(float* w, uint64_t n, uint64_t j0, uint64_t seed,
                       uint32_t n_probes, const double* c)
{
    update_f32_impl(w, n, j0, seed, n_probes, c, NULL);
}

void oracle_q8_update_f32(float* w, uint64_t n, uint64_t j0, uint64_t seed,
                       uint32_t n_probes, const double* c, const float* q8)
{
    update_f32_impl(w, n, j0, seed, n_probes, c, q8);
}

void oracle_update_bf16(uint16_t* w, uint64_t n, uint64_t j0, uint64_t seed,
                        uint32_t n_probes, const double* c)
{
    update_bf16_impl(w, n, j0, seed, n_probes, c, NULL);
}

void oracle_q8_update_bf16(uint16_t* w, uint64_t n, uint64_t j0, uint64_t seed,
                        uint32_t n_probes, const double* c, const float* q8)
{
    update_bf16_impl(w, n, j0, seed, n_probes, c, q8);
}

void oracle_update_f32_at(float* w, const uint64_t* idx, uint64_t n, uint64_t seed,
                          uint32_t n_probes, const double* c)
{
    update_f32_at_impl(w, idx, n, seed, n_probes, c, NULL);
}

void oracle_q8_update_f32_at(float* w, const uint64_t* idx, uint64_t n, uint64_t seed,
                          uint32_t n_probes, const double* c, const float* q8)
{
    update_f32_at_impl(w, idx, n, seed, n_probes, c, q8);
}

void oracle_update_bf16_at(uint16_t* w, const uint64_t* idx, uint64_t n, uint64_t seed,
                           uint32_t n_probes, const double* c)
{
    update_bf16_at_impl(w, idx, n, seed, n_probes, c, NULL);
}

void oracle_q8_update_bf16_at(uint16_t* w, const uint64_t* idx, uint64_t n, uint64_t seed,
                           uint32_t n_probes, const double* c, const float* q8)
{
    update_bf16_at_impl(w, idx, n, seed, n_probes, c, q8);
}

void oracle_perturb_f32_at(float* w, const uint64_t* idx, uint64_t n, uint64_t seed,
                           uint32_t probe, float sigma)
{
    perturb_f32_at_impl(w, idx, n, seed, probe, sigma, NULL);
}

void oracle_q8_perturb_f32_at(float* w, const uint64_t* idx, uint64_t n, uint64_t seed,
                           uint32_t probe, float sigma, const float* q8)
{
    perturb_f32_at_impl(w, idx, n, seed, probe, sigma, q8);
}

void oracle_perturb_bf16_at(uint16_t* w, const uint64_t* idx, uint64_t n, uint64_t seed,
                            uint32_t probe, float sigma)
{
    perturb_bf16_at_impl(w, idx, n, seed, probe, sigma, NULL);
}

void oracle_q8_perturb_bf16_at(uint16_t* w, const uint64_t* idx, uint64_t n, uint64_t seed,
                            uint32_t probe, float sigma, const float* q8)
{
    perturb_bf16_at_impl(w, idx, n, seed, probe, sigma, q8);
}
