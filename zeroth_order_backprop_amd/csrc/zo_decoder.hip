// Forward-only loss of the bf16 pre-LN decoder (GPT-small and OPT shapes) for
// the SPSA step: token + learned-position embedding, L blocks of
// h += W_o Attn(LN1 h), h += W_down act(W_up LN2 h), final LN, LM head tied to
// the token embedding, mean next-token cross-entropy over batch*(seq-1)
// positions.  The loss is a forward-only evaluation of the SPSA loop (ZOO blog
// "Backprop 없이 Transformer를 학습시킨다", section "backprop의 메모리 세금":
// loss only, no backprop, no stored activations beyond the current layer).
//
// Precision: bf16 weights and activations, fp32 MFMA accumulation, rounding to
// bf16 at: embedding sum, LN outputs, every GEMM output (after the
// activation), both residual sums, attention output.  LN statistics and
// softmax are fp32; the LM-head logits never leave fp32 and the loss is fp64.
//
// Every kernel can apply a perturbation on the fly (weights seen =
// bf16(fma(sigma, z, w)) with z regenerated for the element's arena index),
// which is how the perturbed-tile (fused) mode evaluates W +- eps z without
// writing W; with sigma = 0 and no direction the stored weights are used.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <math.h>
#include <string.h>

#include "zo_internal.hpp"
#include "zo_math.hpp"
#include "zo_models.hpp"
#include "zo_rng.hpp"

namespace zo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;

constexpr int kThreads = 256;
constexpr int kDmaThreads = 512, kDmaWavesM = 4;  // 256 x 256 stored-weight GEMM

// A perturbation applied while reading weights.
struct Pert {
    Key key;
    uint32_t probe;
    float sigma;
    int on;  // 0: stored weights as they are
};

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ bf16_t f2bf(float x) { return (bf16_t)(pack2(x, 0.0f) & 0xFFFFu); }

__device__ __forceinline__ float round_bf(float x) { return bf2f(f2bf(x)); }

// 8 consecutive bf16 weights starting at arena index j (j % 8 == 0 not
// required, j % 4 == 0 required), perturbed in place in the uint4.
__device__ __forceinline__ uint4 perturb8(uint4 v, uint64_t j, const Pert& p)
{
    const float4 za = gauss4(p.key, p.probe, j >> 2);
    const float4 zb = gauss4(p.key, p.probe, (j >> 2) + 1);
    float f[8] = {bf2f(v.x & 0xFFFF), bf2f(v.x >> 16), bf2f(v.y & 0xFFFF), bf2f(v.y >> 16),
                  bf2f(v.z & 0xFFFF), bf2f(v.z >> 16), bf2f(v.w & 0xFFFF), bf2f(v.w >> 16)};
    const float z[8] = {za.x, za.y, za.z, za.w, zb.x, zb.y, zb.z, zb.w};
#pragma unroll
    for (int t = 0; t < 8; ++t) f[t] = fmaf(p.sigma, z[t], f[t]);
    return uint4{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
}

// One perturbed weight (slow path: LN parameters, ragged ends).
__device__ __forceinline__ float weight1(const bf16_t* w, uint64_t i, uint64_t dir, const Pert& p)
{
    float v = bf2f(w[i]);
    if (p.on) {
        const uint64_t j = dir + i;
        const float4 z = gauss4(p.key, p.probe, j >> 2);
        const uint32_t s = (uint32_t)(j & 3u);
        const float zz = s == 0 ? z.x : s == 1 ? z.y : s == 2 ? z.z : z.w;
        v = round_bf(fmaf(p.sigma, zz, v));
    }
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sumf(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ double wave_sumd(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// ============================================================ embedding
// h[t][c] = bf16(tok_emb[tok[t]][c] + pos_emb[t % S][c]); one block per token.
__global__ __launch_bounds__(kThreads) void embed_kernel(const int32_t* __restrict__ tokens, int S, int d,
                                                          const bf16_t* __restrict__ tok_emb, uint64_t tok_dir,
                                                          const bf16_t* __restrict__ pos_emb, uint64_t pos_dir,
                                                          Pert p, bf16_t* __restrict__ h)
{
    const int t = blockIdx.x;
    const int tok = tokens[t];
    const int s = t % S;
    const uint64_t te = (uint64_t)tok * d, pe = (uint64_t)s * d;
    for (int c = threadIdx.x; c < d; c += kThreads) {
        const float a = weight1(tok_emb, te + c, tok_dir, p);
        const float b = weight1(pos_emb, pe + c, pos_dir, p);
        h[(size_t)t * d + c] = f2bf(a + b);
    }
}

// ============================================================ LayerNorm
// x[t] = bf16((h[t] - mean) / sqrt(var + 1e-5) * g + b), fp32 statistics.
// One wave per row (4 rows per block, no LDS): lane l holds the 4-element
// groups l, l + 64, ... of the row in registers (8-byte loads), the mean and
// the variance come from wave reductions.
constexpr int kLnMaxQuads = 32;  // d <= 64 lanes * 32 groups * 4 = 8192
template <int NQ>
__global__ __launch_bounds__(kThreads) void layernorm_kernel(const bf16_t* __restrict__ h, int rows, int d,
                                                              const bf16_t* __restrict__ g, uint64_t g_dir,
                                                              const bf16_t* __restrict__ b, uint64_t b_dir, Pert p,
                                                              bf16_t* __restrict__ x)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= rows) return;
    const int nq = d >> 2;
    const uint2* row = reinterpret_cast<const uint2*>(h + (size_t)t * d);
    float v[NQ][4];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        const int q = lane + 64 * k;
        if (q < nq) {
            const uint2 u = row[q];
            v[k][0] = bf2f(u.x & 0xFFFF); v[k][1] = bf2f(u.x >> 16);
            v[k][2] = bf2f(u.y & 0xFFFF); v[k][3] = bf2f(u.y >> 16);
        } else {
            v[k][0] = v[k][1] = v[k][2] = v[k][3] = 0.f;
        }
        s += (v[k][0] + v[k][1]) + (v[k][2] + v[k][3]);
    }
    const float mean = wave_sumf(s) / (float)d;
    float q2 = 0.f;
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        if (lane + 64 * k < nq) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float dv = v[k][e] - mean;
                q2 = fmaf(dv, dv, q2);
            }
        }
    }
    const float var = wave_sumf(q2) / (float)d;
    const float rstd = 1.0f / sqrtf(var + 1e-5f);
    uint2* out = reinterpret_cast<uint2*>(x + (size_t)t * d);
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        const int q = lane + 64 * k;
        if (q >= nq) continue;
        float o[4];
        if (p.on) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 4 * q + e;
                o[e] = fmaf((v[k][e] - mean) * rstd, weight1(g, c, g_dir, p), weight1(b, c, b_dir, p));
            }
        } else {
            const uint2 gg = reinterpret_cast<const uint2*>(g)[q];
            const uint2 bb = reinterpret_cast<const uint2*>(b)[q];
            const float gv[4] = {bf2f(gg.x & 0xFFFF), bf2f(gg.x >> 16), bf2f(gg.y & 0xFFFF), bf2f(gg.y >> 16)};
            const float bv[4] = {bf2f(bb.x & 0xFFFF), bf2f(bb.x >> 16), bf2f(bb.y & 0xFFFF), bf2f(bb.y >> 16)};
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = fmaf((v[k][e] - mean) * rstd, gv[e], bv[e]);
        }
        out[q] = uint2{pack2(o[0], o[1]), pack2(o[2], o[3])};
    }
}

// Wide rows (d > 2048): one 256-thread block per row, NQ groups of 4 per
// thread (group q = tid + 256 k); the sums are combined across the 4 waves
// through LDS in a fixed order.
template <int NQ>
__global__ __launch_bounds__(kThreads) void layernorm_wide_kernel(const bf16_t* __restrict__ h, int d,
                                                                   const bf16_t* __restrict__ g, uint64_t g_dir,
                                                                   const bf16_t* __restrict__ b, uint64_t b_dir, Pert p,
                                                                   bf16_t* __restrict__ x)
{
    __shared__ float part[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t t = blockIdx.x;
    const int nq = d >> 2;
    const uint2* row = reinterpret_cast<const uint2*>(h + t * d);
    float v[NQ][4];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        const int q = tid + kThreads * k;
        if (q < nq) {
            const uint2 u = row[q];
            v[k][0] = bf2f(u.x & 0xFFFF); v[k][1] = bf2f(u.x >> 16);
            v[k][2] = bf2f(u.y & 0xFFFF); v[k][3] = bf2f(u.y >> 16);
        } else {
            v[k][0] = v[k][1] = v[k][2] = v[k][3] = 0.f;
        }
        s += (v[k][0] + v[k][1]) + (v[k][2] + v[k][3]);
    }
    s = wave_sumf(s);
    if (lane == 0) part[0][wave] = s;
    __syncthreads();
    const float mean = (((part[0][0] + part[0][1]) + part[0][2]) + part[0][3]) / (float)d;
    float q2 = 0.f;
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        if (tid + kThreads * k < nq) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float dv = v[k][e] - mean;
                q2 = fmaf(dv, dv, q2);
            }
        }
    }
    q2 = wave_sumf(q2);
    if (lane == 0) part[1][wave] = q2;
    __syncthreads();
    const float var = (((part[1][0] + part[1][1]) + part[1][2]) + part[1][3]) / (float)d;
    const float rstd = 1.0f / sqrtf(var + 1e-5f);
    uint2* out = reinterpret_cast<uint2*>(x + t * d);
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        const int q = tid + kThreads * k;
        if (q >= nq) continue;
        float o[4];
        if (p.on) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 4 * q + e;
                o[e] = fmaf((v[k][e] - mean) * rstd, weight1(g, c, g_dir, p), weight1(b, c, b_dir, p));
            }
        } else {
            const uint2 gg = reinterpret_cast<const uint2*>(g)[q];
            const uint2 bb = reinterpret_cast<const uint2*>(b)[q];
            const float gv[4] = {bf2f(gg.x & 0xFFFF), bf2f(gg.x >> 16), bf2f(gg.y & 0xFFFF), bf2f(gg.y >> 16)};
            const float bv[4] = {bf2f(bb.x & 0xFFFF), bf2f(bb.x >> 16), bf2f(bb.y & 0xFFFF), bf2f(bb.y >> 16)};
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = fmaf((v[k][e] - mean) * rstd, gv[e], bv[e]);
        }
        out[q] = uint2{pack2(o[0], o[1]), pack2(o[2], o[3])};
    }
}

// LayerNorm of `rows` rows of width d (d % 4 == 0, d <= 8192): one wave per
// row with the smallest register footprint that holds it (NQ groups of 4 per
// lane) up to d = 2048, one block per row beyond.
void launch_layernorm(const bf16_t* h, int rows, int d, const bf16_t* g, uint64_t g_dir, const bf16_t* b,
                      uint64_t b_dir, const Pert& p, bf16_t* x, hipStream_t s)
{
    const int nq = (d / 4 + 63) / 64;
    const dim3 grid((rows + 3) / 4);
    if (nq <= 1) layernorm_kernel<1><<<grid, kThreads, 0, s>>>(h, rows, d, g, g_dir, b, b_dir, p, x);
    else if (nq <= 3) layernorm_kernel<3><<<grid, kThreads, 0, s>>>(h, rows, d, g, g_dir, b, b_dir, p, x);
    else if (nq <= 8) layernorm_kernel<8><<<grid, kThreads, 0, s>>>(h, rows, d, g, g_dir, b, b_dir, p, x);
    else layernorm_wide_kernel<kLnMaxQuads / 4><<<rows, kThreads, 0, s>>>(h, d, g, g_dir, b, b_dir, p, x);
}

// ============================================================ bf16 GEMM
// C[M][N] = A[M][K] * W[N][K]^T, bf16 in, fp32 accumulate (MFMA 32x32x16).
// 256 threads = 2x2 waves; each wave owns a (BM/2) x (BN/2) tile of 32x32
// MFMA blocks.  LDS holds two stages of A and B with rows padded by 8 bf16
// (16 B) so the b128 fragment reads of 32 consecutive rows spread over all
// banks.  Global loads for stage k+1 are in flight during stage k's MFMAs.
enum { EPI_STORE = 0, EPI_GELU = 1, EPI_RELU = 2, EPI_RESID = 3, EPI_LMHEAD = 4 };

struct GemmParams {
    const bf16_t* A;  // [M][K]
    const bf16_t* W;  // [N][K]
    uint64_t w_dir;   // arena index of W[0][0]
    bf16_t* C;        // [M][N] (EPI_STORE / GELU / RELU) or the residual h (EPI_RESID, [M][N])
    int M, N, K;
    // LM head: per (n_tile, row) running max / sum of exp, and the target logit
    float* lm_max;
    float* lm_sum;
    float* lm_pick;
    const int32_t* tokens;  // targets: row r's target is tokens[r + 1] (same sequence)
    int S;
};


// Linear tile index -> (tm, tn): consecutive workgroups land on consecutive
// XCDs, so give each XCD a contiguous range of tiles, and walk tiles in
// groups of G M-tiles so neighbours share A rows and W columns in L2.
template <int G = 8>
__device__ __forceinline__ void tile_of(int b, int nbm, int nbn, int& tm, int& tn)
{
    const int total = nbm * nbn;
    int t = b;
    if (total % 8 == 0) t = (b % 8) * (total / 8) + b / 8;
    const int group = t / (G * nbn);
    const int first = group * G;
    const int gsize = min(nbm - first, G);
    const int r = t % (G * nbn);
    tm = first + r % gsize;
    tn = r / gsize;
}

// Writes one block tile's accumulators (see the GEMM kernels below).
// Accumulator element r of a 32x32 block: row 8 (r/4) + 4 lh + r%4, col lr.
// Stores go through LDS: the activated, bf16-rounded tile is written to
// `smem` (rows padded by 8 bf16, so the two row groups of one write land on
// different banks), then every thread moves 16-byte row chunks, for the
// residual path reading the matching 16 bytes of h first: all global traffic
// of the epilogue is coalesced 16-byte accesses.  Needs N % 8 == 0, C 16-byte
// aligned and BM * (BN + 8) bf16 of LDS that no wave still reads.
template <int BM, int BN>
constexpr size_t epilogue_lds_bytes() { return (size_t)BM * (BN + 8) * sizeof(bf16_t); }

template <int BM, int BN, int EPI, int RB, int CB, int NT, int WGM>
__device__ __forceinline__ void gemm_epilogue_impl(const GemmParams& g, f32x16 (&acc)[RB][CB], int m0, int n0, int tn,
                                                   bf16_t* smem)
{
    // NT threads as a WGM x WGN grid of waves, each owning WM x WN
    constexpr int WGN = NT / 64 / WGM, WM = BM / WGM, WN = BN / WGN;
    static_assert(WM == RB * 32 && WN == CB * 32, "wave tile mismatch");
    const int M = g.M, N = g.N;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WGN, wn = wave % WGN;
    const int lr = lane & 31, lh = lane >> 5;
    if constexpr (EPI != EPI_LMHEAD) {
        constexpr int LDC = BN + 8;
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wm * WM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                    const int col = wn * WN + j * 32 + lr;
                    float v = acc[i][j][r];
                    if constexpr (EPI == EPI_GELU) v = gelu_erf(v);
                    if constexpr (EPI == EPI_RELU) v = fmaxf(v, 0.0f);
                    smem[row * LDC + col] = f2bf(v);
                }
        __syncthreads();
        constexpr int CPR = BN / 8;  // 16-byte chunks per row
#pragma unroll 4
        for (int p = tid; p < BM * CPR; p += NT) {
            const int row = p / CPR, cc = p % CPR;
            const int gr = m0 + row, gc = n0 + 8 * cc;
            if (gr >= M || gc >= N) continue;
            uint4 v = *reinterpret_cast<const uint4*>(smem + row * LDC + 8 * cc);
            uint4* dst = reinterpret_cast<uint4*>(g.C + (size_t)gr * N + gc);
            if constexpr (EPI == EPI_RESID) {
                // h + bf16(product), rounded once more to bf16
                const uint4 h = *dst;
                auto add2 = [](uint32_t hw, uint32_t pw) {
                    return pack2(bf2f(hw & 0xFFFF) + bf2f(pw & 0xFFFF), bf2f(hw >> 16) + bf2f(pw >> 16));
                };
                v = uint4{add2(h.x, v.x), add2(h.y, v.y), add2(h.z, v.z), add2(h.w, v.w)};
            }
            *dst = v;
        }
    } else {
        static_assert(WGN == 2, "LM-head partials assume two wave columns");
        // Fused cross-entropy partials over this tile's BN vocabulary columns:
        // per row the max and the sum of exp(logit - max), plus the target
        // logit when the target column lies in this tile.
        __shared__ float part_m[2][BM], part_s[2][BM];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lrow = wm * WM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                const int row = m0 + lrow;
                float mx = -INFINITY;
#pragma unroll
                for (int j = 0; j < CB; ++j) {
                    const int col = n0 + wn * WN + j * 32 + lr;
                    if (col < N) mx = fmaxf(mx, acc[i][j][r]);
                }
#pragma unroll
                for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
                float se = 0.f;
#pragma unroll
                for (int j = 0; j < CB; ++j) {
                    const int col = n0 + wn * WN + j * 32 + lr;
                    if (col < N) se += __expf(acc[i][j][r] - mx);
                }
#pragma unroll
                for (int o = 16; o > 0; o >>= 1) se += __shfl_xor(se, o, 64);
                if (lr == 0) {
                    part_m[wn][lrow] = mx;
                    part_s[wn][lrow] = se;
                }
                if (row < M && (row % g.S) != g.S - 1) {
                    const int target = g.tokens[row + 1];
#pragma unroll
                    for (int j = 0; j < CB; ++j) {
                        const int col = n0 + wn * WN + j * 32 + lr;
                        if (col == target) g.lm_pick[row] = acc[i][j][r];
                    }
                }
            }
        __syncthreads();
        for (int lrow = tid; lrow < BM; lrow += NT) {
            const int row = m0 + lrow;
            if (row >= M) continue;
            const float m1 = part_m[0][lrow], m2 = part_m[1][lrow];
            const float mx = fmaxf(m1, m2);
            float se = 0.f;
            if (m1 > -INFINITY) se += part_s[0][lrow] * __expf(m1 - mx);
            if (m2 > -INFINITY) se += part_s[1][lrow] * __expf(m2 - mx);
            g.lm_max[(size_t)tn * M + row] = mx;
            g.lm_sum[(size_t)tn * M + row] = se;
        }
    }
}

template <int BM, int BN, int EPI, int NT = kThreads, int WGM = 2, int RB, int CB>
__device__ __forceinline__ void gemm_epilogue(const GemmParams& g, f32x16 (&acc)[RB][CB], int m0, int n0, int tn,
                                              bf16_t* smem)
{
    gemm_epilogue_impl<BM, BN, EPI, RB, CB, NT, WGM>(g, acc, m0, n0, tn, smem);
}

template <int BM, int BN, int EPI, bool PERT>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmParams g, Pert p)
{
    constexpr int BK = 64;
    constexpr int LDK = BK + 8;  // padded row (bf16)
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int RB = WM / 32, CB = WN / 32;
    constexpr int A_CH = BM * BK / 8, B_CH = BN * BK / 8;  // 16-byte chunks per stage
    constexpr int A_PER = A_CH / kThreads, B_PER = B_CH / kThreads;
    static_assert(A_CH % kThreads == 0 && B_CH % kThreads == 0, "tile / thread mismatch");
    extern __shared__ __align__(16) bf16_t lds[];
    // stage st: A tile at lds + st * BM * LDK, B tile at lds + 2 BM LDK + st * BN * LDK
    auto As = [&](int st) { return lds + st * (BM * LDK); };
    auto Bs = [&](int st) { return lds + 2 * (BM * LDK) + st * (BN * LDK); };

    const int M = g.M, N = g.N, K = g.K;
    const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    int tm, tn;
    tile_of(blockIdx.x, nbm, nbn, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, lh = lane >> 5;

    f32x16 acc[RB][CB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) acc[i][j] = f32x16{};

    uint4 ra[A_PER], rb[B_PER];
    auto load = [&](int k0) {
#pragma unroll
        for (int t = 0; t < A_PER; ++t) {
            const int c = tid + t * kThreads;
            const int r = c / (BK / 8), kc = 8 * (c % (BK / 8));
            const int gm = m0 + r, gk = k0 + kc;
            ra[t] = (gm < M && gk < K) ? *reinterpret_cast<const uint4*>(g.A + (size_t)gm * K + gk)
                                       : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int t = 0; t < B_PER; ++t) {
            const int c = tid + t * kThreads;
            const int r = c / (BK / 8), kc = 8 * (c % (BK / 8));
            const int gn = n0 + r, gk = k0 + kc;
            rb[t] = (gn < N && gk < K) ? *reinterpret_cast<const uint4*>(g.W + (size_t)gn * K + gk)
                                       : uint4{0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](int stage, int k0) {
#pragma unroll
        for (int t = 0; t < A_PER; ++t) {
            const int c = tid + t * kThreads;
            const int r = c / (BK / 8), kc = 8 * (c % (BK / 8));
            *reinterpret_cast<uint4*>(As(stage) + r * LDK + kc) = ra[t];
        }
#pragma unroll
        for (int t = 0; t < B_PER; ++t) {
            const int c = tid + t * kThreads;
            const int r = c / (BK / 8), kc = 8 * (c % (BK / 8));
            uint4 v = rb[t];
            if constexpr (PERT) {
                const int gn = n0 + r, gk = k0 + kc;
                if (gn < N && gk < K) v = perturb8(v, g.w_dir + (uint64_t)gn * K + gk, p);
            }
            *reinterpret_cast<uint4*>(Bs(stage) + r * LDK + kc) = v;
        }
    };

    const int KT = (K + BK - 1) / BK;
    load(0);
    store(0, 0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK; ks += 16) {
            bf16x8 af[RB], bfr[CB];
#pragma unroll
            for (int i = 0; i < RB; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(As(cur) + (wm * WM + i * 32 + lr) * LDK + ks + 8 * lh);
#pragma unroll
            for (int j = 0; j < CB; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(Bs(cur) + (wn * WN + j * 32 + lr) * LDK + ks + 8 * lh);
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int j = 0; j < CB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) store(cur ^ 1, (kt + 1) * BK);
        __syncthreads();
    }

    gemm_epilogue<BM, BN, EPI>(g, acc, m0, n0, tn, lds);
}

// The same product with the stage tiles written to LDS directly by the loads
// (global_load_lds, 16 B per lane) for the stored-weight path: no register
// staging.  Rows past M or N load a clamped (valid) row and are never stored.
// Barriers are bare s_barrier after each wave has waited (vmcnt) for its own
// share of a stage, so that later stages stay in flight across them.

// vmcnt(n) with expcnt / lgkmcnt left at their maxima (gfx9 encoding)
#define ZO_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
#define ZO_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4))

// Large tiles: 8 waves (two per SIMD, so one wave's MFMAs cover the other's
// LDS and barrier waits) in a 4 x 2 grid of 64 x 128 wave tiles; a ring of 5
// BK = 32 stages (all 160 KB of LDS), prefetch distance 4: the loads' latency
// is what the waves wait on (measured 2-10% faster than a ring of 4).  The LM
// head keeps a ring of 4: its epilogue's cross-entropy partials take 4 KB of
// static LDS besides.  LDS rows are 64 B (4 chunks of 16 B), chunk c of row r
// at position c ^ ((r >> 2) & 3), so the 32 rows a fragment read touches
// spread over all banks.  The two k-halves of a stage are read into
// alternating register sets: the second half's reads and the next stage's
// first half are issued while the MFMAs of the previous half run.
template <int EPI>
constexpr int dma_stages() { return EPI == EPI_LMHEAD ? 4 : 5; }

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(kDmaThreads) void gemm_bf16_dma_kernel(GemmParams g)
{
    constexpr int BK = 32, STAGES = dma_stages<EPI>();
    constexpr int NT = kDmaThreads, WGM = kDmaWavesM, WGN = NT / 64 / WGM;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int RB = WM / 32, CB = WN / 32;
    constexpr int A_INS = BM * 4 / NT, B_INS = BN * 4 / NT;
    constexpr int INS = A_INS + B_INS;  // load instructions per thread per stage
    constexpr int STAGE = (BM + BN) * BK;
    static_assert(A_INS * NT == BM * 4 && B_INS * NT == BN * 4, "tile / thread mismatch");
    static_assert((STAGES - 2) * INS < 64, "vmcnt range");
    extern __shared__ __align__(16) bf16_t lds[];

    const int M = g.M, N = g.N, K = g.K;
    const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    int tm, tn;
    tile_of<4>(blockIdx.x, nbm, nbn, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WGN, wn = wave % WGN;
    const int lr = lane & 31, lh = lane >> 5;

    f32x16 acc[RB][CB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) acc[i][j] = f32x16{};

    const int KT = K / BK;
    auto issue = [&](int kt) {
        bf16_t* sa = lds + (kt % STAGES) * STAGE;
        bf16_t* sb = sa + BM * BK;
        const int k0 = kt * BK;
#pragma unroll
        for (int j = 0; j < A_INS; ++j) {
            const int p = j * NT + tid, row = p >> 2, lc = (p & 3) ^ ((row >> 2) & 3);
            const bf16_t* src = g.A + (size_t)min(m0 + row, M - 1) * K + k0 + 8 * lc;
            bf16_t* dst = sa + (j * NT + wave * 64) * 8;  // wave-uniform: lane l lands at +16 l bytes
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < B_INS; ++j) {
            const int p = j * NT + tid, row = p >> 2, lc = (p & 3) ^ ((row >> 2) & 3);
            const bf16_t* src = g.W + (size_t)min(n0 + row, N - 1) * K + k0 + 8 * lc;
            bf16_t* dst = sb + (j * NT + wave * 64) * 8;
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
    };
    static_assert(STAGES >= 3 && STAGES <= 5, "wait_vm covers up to three stages in flight");
    auto wait_vm = [](int stages_in_flight) {
        if (stages_in_flight >= 3) ZO_WAIT_VM(3 * INS);
        else if (stages_in_flight >= 2) ZO_WAIT_VM(2 * INS);
        else if (stages_in_flight == 1) ZO_WAIT_VM(INS);
        else ZO_WAIT_VM(0);
    };
    // fragment offsets (elements) of this lane for k-half ks of a stage
    int aoff[2][RB], boff[2][CB];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int lc = 2 * ks + lh;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int row = wm * WM + i * 32 + lr;
            aoff[ks][i] = (row * 4 + (lc ^ ((row >> 2) & 3))) * 8;
        }
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            const int row = wn * WN + j * 32 + lr;
            boff[ks][j] = BM * BK + (row * 4 + (lc ^ ((row >> 2) & 3))) * 8;
        }
    }
    bf16x8 fa[2][RB], fb[2][CB];
    auto read = [&](int kt, int ks, int slot) {
        const bf16_t* st = lds + (kt % STAGES) * STAGE;
#pragma unroll
        for (int j = 0; j < CB; ++j) fb[slot][j] = *reinterpret_cast<const bf16x8*>(st + boff[ks][j]);
#pragma unroll
        for (int i = 0; i < RB; ++i) fa[slot][i] = *reinterpret_cast<const bf16x8*>(st + aoff[ks][i]);
    };
    auto mma = [&](int slot) {
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
    };

    for (int st = 0; st < STAGES - 1 && st < KT; ++st) issue(st);
    wait_vm(min(STAGES - 2, KT - 1));  // stage 0 landed; the next ones may be in flight
    asm volatile("s_barrier" ::: "memory");
    read(0, 0, 0);
    for (int kt = 0; kt < KT; ++kt) {
        read(kt, 1, 1);
        mma(0);
        if (kt + 1 < KT) {
            // stage kt+1 landed (kt+2 .. kt+STAGES-2 may remain in flight)
            // and this wave's reads of stage kt are in registers; after the
            // barrier every wave is done with stage kt-1's buffer, which is
            // refilled
            wait_vm(min(STAGES - 3, KT - 2 - kt));
            ZO_WAIT_LGKM0();
            asm volatile("s_barrier" ::: "memory");
            if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1);
            read(kt + 1, 0, 0);
        }
        mma(1);
    }
    __syncthreads();  // every wave is done with the stage buffers
    gemm_epilogue<BM, BN, EPI, NT, WGM>(g, acc, m0, n0, tn, lds);
}

// Small tiles (128 x 128 or 128 x 64): two BK = 64 stages, NT/64 waves in a
// WGM x (NT/64/WGM) grid.  LDS rows are 128 B (8 chunks of 16 B),
// chunk c of row r at position c ^ ((r >> 1) & 7): the 32 rows of a fragment
// read (16 B each, half the wave on one chunk column) cover every bank
// evenly.  Stage k+1 loads while stage k's MFMAs run.
template <int BM, int BN, int EPI, int NT, int WGM>
__global__ __launch_bounds__(NT) void gemm_bf16_k64_kernel(GemmParams g)
{
    constexpr int BK = 64;
    constexpr int WGN = NT / 64 / WGM, WM = BM / WGM, WN = BN / WGN;
    constexpr int RB = WM / 32, CB = WN / 32;
    constexpr int A_INS = BM * 8 / NT, B_INS = BN * 8 / NT;
    constexpr int STAGE = (BM + BN) * BK;
    static_assert(A_INS * NT == BM * 8 && B_INS * NT == BN * 8, "tile / thread mismatch");
    extern __shared__ __align__(16) bf16_t lds[];

    const int M = g.M, N = g.N, K = g.K;
    const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    int tm, tn;
    tile_of<8>(blockIdx.x, nbm, nbn, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WGN, wn = wave % WGN;
    const int lr = lane & 31, lh = lane >> 5;

    f32x16 acc[RB][CB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) acc[i][j] = f32x16{};

    const int KT = K / BK;
    auto issue = [&](int kt) {
        bf16_t* sa = lds + (kt & 1) * STAGE;
        bf16_t* sb = sa + BM * BK;
        const int k0 = kt * BK;
#pragma unroll
        for (int j = 0; j < A_INS; ++j) {
            const int p = j * NT + tid, row = p >> 3, lc = (p & 7) ^ ((row >> 1) & 7);
            const bf16_t* src = g.A + (size_t)min(m0 + row, M - 1) * K + k0 + 8 * lc;
            bf16_t* dst = sa + (j * NT + wave * 64) * 8;
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < B_INS; ++j) {
            const int p = j * NT + tid, row = p >> 3, lc = (p & 7) ^ ((row >> 1) & 7);
            const bf16_t* src = g.W + (size_t)min(n0 + row, N - 1) * K + k0 + 8 * lc;
            bf16_t* dst = sb + (j * NT + wave * 64) * 8;
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
    };

    issue(0);
    for (int kt = 0; kt < KT; ++kt) {
        ZO_WAIT_VM(0);
        asm volatile("s_barrier" ::: "memory");
        if (kt + 1 < KT) issue(kt + 1);
        const bf16_t* sa = lds + (kt & 1) * STAGE;
        const bf16_t* sb = sa + BM * BK;
        // Fragments of the four 16-deep steps.  With a fused epilogue (GELU,
        // residual) all of them are read first and the MFMAs follow, the
        // scheduling barriers keeping the compiler from moving each read down
        // next to its MFMA (where it waits before every MFMA); with the plain
        // store epilogue the reads stay per step, which measured faster there.
        constexpr bool HOIST = EPI != EPI_STORE;
        constexpr int NF = HOIST ? 4 : 1;
        bf16x8 af[NF][RB], bfr[NF][CB];
        auto read_step = [&](int ks, int f) {
            const int lc = 2 * ks + lh;
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const int row = wm * WM + i * 32 + lr;
                af[f][i] = *reinterpret_cast<const bf16x8*>(sa + (row * 8 + (lc ^ ((row >> 1) & 7))) * 8);
            }
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const int row = wn * WN + j * 32 + lr;
                bfr[f][j] = *reinterpret_cast<const bf16x8*>(sb + (row * 8 + (lc ^ ((row >> 1) & 7))) * 8);
            }
        };
        auto mma_step = [&](int f) {
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int j = 0; j < CB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[f][i], bfr[f][j], acc[i][j], 0, 0, 0);
        };
        if constexpr (HOIST) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) read_step(ks, ks);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) mma_step(ks);
            __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                read_step(ks, 0);
                mma_step(0);
            }
        }
        // every wave is done reading this stage before the next issue refills it
        asm volatile("s_barrier" ::: "memory");
    }
    gemm_epilogue<BM, BN, EPI, NT, WGM>(g, acc, m0, n0, tn, lds);
}

// Per-row cross-entropy (logsumexp_r - pick_r) for rows r with r % S != S-1.
// A block covers 64 rows; its 4 waves take every 4th vocabulary tile and merge
// (max, sum of exp) online in fp64, then the 4 partial results are merged in
// fixed order; each block writes the fp64 sum of its rows' losses.
__global__ __launch_bounds__(kThreads) void ce_rows_kernel(const float* __restrict__ lm_max,
                                                            const float* __restrict__ lm_sum,
                                                            const float* __restrict__ lm_pick, int n_tiles, int M,
                                                            int S, double* __restrict__ block_sum)
{
    __shared__ double pm[4][64], ps[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * 64 + lane;
    double m = -INFINITY, se = 0.0;
    if (row < M) {
        for (int t = wave; t < n_tiles; t += 4) {
            const double tm = (double)lm_max[(size_t)t * M + row];
            if (tm == -INFINITY) continue;
            const double ts = (double)lm_sum[(size_t)t * M + row];
            if (tm > m) {
                se = se * exp(m - tm) + ts;
                m = tm;
            } else {
                se += ts * exp(tm - m);
            }
        }
    }
    pm[wave][lane] = m;
    ps[wave][lane] = se;
    __syncthreads();
    if (wave != 0) return;
    double v = 0.0;
    if (row < M && row % S != S - 1) {
        double mx = pm[0][lane];
        for (int w = 1; w < 4; ++w) mx = fmax(mx, pm[w][lane]);
        double tot = 0.0;
        for (int w = 0; w < 4; ++w)
            if (pm[w][lane] > -INFINITY) tot += ps[w][lane] * exp(pm[w][lane] - mx);
        v = (mx + log(tot)) - (double)lm_pick[row];
    }
    v = wave_sumd(v);
    if (lane == 0) block_sum[blockIdx.x] = v;
}

// loss = (sum of block sums, fixed order) / (B (S-1))
__global__ __launch_bounds__(kThreads) void ce_final_kernel(const double* __restrict__ block_sum, int n_blocks,
                                                             int M, int S, double* __restrict__ loss)
{
    __shared__ double red[4];
    double v = 0.0;
    for (int i = threadIdx.x; i < n_blocks; i += kThreads) v += block_sum[i];
    v = wave_sumd(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) *loss = (((red[0] + red[1]) + red[2]) + red[3]) / (double)((M / S) * (S - 1));
}

// ============================================================ attention
// Causal softmax(Q K^T / sqrt(dh)) V per (sequence, head), flash style.  The
// wave computes S^T = K Q^T for 32 queries (one per lane column) so the
// running max / sum of each query live in one lane; P^T goes straight from
// the accumulators into the B operand of O^T = V^T P^T (the contraction
// order over keys is the same permutation on both operands).  P is rounded to
// bf16 for the MFMA; max, sums and rescaling are fp32, exponentials are exp2
// of scores pre-scaled by log2(e) / sqrt(dh).
// Block: 4 waves x 32 queries = 128 queries; keys in tiles of 64.
template <int DH>
__global__ __launch_bounds__(kThreads) void attention_kernel(const bf16_t* __restrict__ qkv, int S, int d, int H,
                                                              bf16_t* __restrict__ out)
{
    constexpr int BQ = 128, BKV = DH == 64 ? 64 : 32;
    constexpr int NB = BKV / 32;  // 32-key blocks per tile
    constexpr int KS = DH / 16;   // MFMA k-steps over the head dim for S^T
    constexpr int OT = DH / 32;   // 32-row blocks of O^T
    constexpr int LDK = DH + 8;   // K tile row (bf16), padded
    constexpr int LDV = BKV + 4;  // V^T tile row (bf16): 8 rows apart = 16 banks apart
    __shared__ __align__(16) bf16_t Ks[BKV * LDK];
    __shared__ __align__(16) bf16_t Vt[DH * LDV];

    const int qblocks = (S + BQ - 1) / BQ;
    // heaviest (latest) query blocks first
    const int qb = qblocks - 1 - (blockIdx.x % qblocks);
    const int bh = blockIdx.x / qblocks;
    const int b = bh / H, hd = bh % H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 31, lh = lane >> 5;
    const int q0 = qb * BQ;
    const int qw = q0 + wave * 32;  // this wave's first query
    const int myq = qw + lr;        // this lane's query (S^T column)
    const size_t row_stride = 3 * (size_t)d;
    const bf16_t* base = qkv + (size_t)b * S * row_stride;
    const int qoff = hd * DH, koff = d + hd * DH, voff = 2 * d + hd * DH;
    const float c = 1.4426950408889634f / sqrtf((float)DH);  // log2(e) / sqrt(dh)

    // Q^T as the B operand: lane (lr = query, lh) holds dh 8 lh + 16 ks .. +7
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (myq < S)
            qf[ks] = *reinterpret_cast<const bf16x8*>(base + (size_t)myq * row_stride + qoff + 16 * ks + 8 * lh);
        else
            qf[ks] = bf16x8{};
    }
    f32x16 o[OT];
#pragma unroll
    for (int t = 0; t < OT; ++t) o[t] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;  // in log2 units

    const int kv_end = min(S, q0 + BQ);  // causal: keys < last query of the block
    // Each thread stages CH (key pair, 8-column) chunks of K and V per tile:
    // keys 2 kp and 2 kp + 1, head-dim columns dc .. dc + 7.  The next tile's
    // chunks are loaded into registers while the current tile is computed.
    // K chunks go to LDS as 16-byte row pieces, so dc runs fastest across the
    // lanes (one row's bytes contiguous); V goes in transposed as 4-byte key
    // pairs, so there kp runs fastest (consecutive lanes, consecutive words:
    // with dc fastest the lanes of one key pair hit one bank).
    constexpr int CH = (BKV / 2) * (DH / 8) / kThreads;
    static_assert(CH * kThreads == (BKV / 2) * (DH / 8), "tile / thread mismatch");
    uint4 rk[CH][2], rv[CH][2];
    auto load_kv = [&](int k0) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int cc = tid + j * kThreads;
            const int kp = cc / (DH / 8), dc = 8 * (cc % (DH / 8));
            const int kpv = cc % (BKV / 2), dcv = 8 * (cc / (BKV / 2));
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int key = k0 + 2 * kp + e, keyv = k0 + 2 * kpv + e;
                rk[j][e] = rv[j][e] = uint4{0u, 0u, 0u, 0u};
                if (key < S) rk[j][e] = *reinterpret_cast<const uint4*>(base + (size_t)key * row_stride + koff + dc);
                if (keyv < S) rv[j][e] = *reinterpret_cast<const uint4*>(base + (size_t)keyv * row_stride + voff + dcv);
            }
        }
    };
    auto store_kv = [&]() {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int cc = tid + j * kThreads;
            const int kp = cc / (DH / 8), dc = 8 * (cc % (DH / 8));
            const int kpv = cc % (BKV / 2), dcv = 8 * (cc / (BKV / 2));
            *reinterpret_cast<uint4*>(Ks + (2 * kp) * LDK + dc) = rk[j][0];
            *reinterpret_cast<uint4*>(Ks + (2 * kp + 1) * LDK + dc) = rk[j][1];
            // V^T: column pair (2 kpv, 2 kpv + 1) of row dcv + e, one 4-byte write each
            const uint32_t a[4] = {rv[j][0].x, rv[j][0].y, rv[j][0].z, rv[j][0].w};
            const uint32_t b4[4] = {rv[j][1].x, rv[j][1].y, rv[j][1].z, rv[j][1].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                *reinterpret_cast<uint32_t*>(Vt + (dcv + 2 * e) * LDV + 2 * kpv) = (a[e] & 0xFFFFu) | (b4[e] << 16);
                *reinterpret_cast<uint32_t*>(Vt + (dcv + 2 * e + 1) * LDV + 2 * kpv) =
                    (a[e] >> 16) | (b4[e] & 0xFFFF0000u);
            }
        }
    };
    load_kv(0);
    for (int k0 = 0; k0 < kv_end; k0 += BKV) {
        __syncthreads();  // every wave is done with the previous tile
        store_kv();
        __syncthreads();
        if (k0 + BKV < kv_end) load_kv(k0 + BKV);  // in flight during this tile's MFMAs
        if (k0 > qw + 31) continue;  // every key of this tile is after all of this wave's queries
        // S^T [BKV keys][32 queries] as NB 32x32 blocks
        f32x16 st[NB];
#pragma unroll
        for (int hblk = 0; hblk < NB; ++hblk) {
            st[hblk] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 kf =
                    *reinterpret_cast<const bf16x8*>(Ks + (32 * hblk + lr) * LDK + 16 * ks + 8 * lh);
                st[hblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], st[hblk], 0, 0, 0);
            }
        }
        // element r of block hblk: key k0 + 32 hblk + 8 (r/4) + 4 lh + r%4, query myq
        if (k0 + BKV - 1 > qw) {  // diagonal tile: some key may follow some query of the wave
            const int last = min(myq, S - 1);
#pragma unroll
            for (int hblk = 0; hblk < NB; ++hblk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * hblk + 8 * (r >> 2) + 4 * lh + (r & 3);
                    st[hblk][r] = key <= last ? st[hblk][r] : -INFINITY;
                }
        }
        // running max in log2 units: max(s c) = c max(s) for c > 0
        float tmax = -INFINITY;
#pragma unroll
        for (int hblk = 0; hblk < NB; ++hblk)
#pragma unroll
            for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, st[hblk][r]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * c;
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        float psum = 0.f;
        bf16x8 pb[NB][2];
#pragma unroll
        for (int hblk = 0; hblk < NB; ++hblk)
#pragma unroll
            for (int sblk = 0; sblk < 2; ++sblk) {
                uint32_t w4[4];
#pragma unroll
                for (int t = 0; t < 8; t += 2) {
                    // exp2(s c - m): one fma per score; exp2(-inf) = 0 for masked keys
                    const float e0 = __builtin_amdgcn_exp2f(fmaf(st[hblk][8 * sblk + t], c, -m_new));
                    const float e1 = __builtin_amdgcn_exp2f(fmaf(st[hblk][8 * sblk + t + 1], c, -m_new));
                    psum += e0 + e1;
                    w4[t >> 1] = pack2(e0, e1);
                }
                const uint4 u = {w4[0], w4[1], w4[2], w4[3]};
                pb[hblk][sblk] = __builtin_bit_cast(bf16x8, u);
            }
        psum += __shfl_xor(psum, 32, 64);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        // rescale only when some query of the wave raised its max
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int t = 0; t < OT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
        }
        // O^T += V^T P^T over the BKV keys in 2 NB MFMA k-steps; step (hblk, sblk)
        // uses accumulator elements 8 sblk .. 8 sblk + 7 of block hblk, i.e.
        // keys 32 hblk + 16 sblk + 8 (t/4) + 4 lh + t%4
#pragma unroll
        for (int hblk = 0; hblk < NB; ++hblk)
#pragma unroll
            for (int sblk = 0; sblk < 2; ++sblk)
#pragma unroll
                for (int t = 0; t < OT; ++t) {
                    // A = V^T rows dh = 32 t + lr, the same 8 keys in the same order
                    const bf16_t* vr = Vt + (32 * t + lr) * LDV + 32 * hblk + 16 * sblk + 4 * lh;
                    const uint2 lo = *reinterpret_cast<const uint2*>(vr);
                    const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
                    const uint4 packed = {lo.x, lo.y, hi.x, hi.y};
                    const bf16x8 va = __builtin_bit_cast(bf16x8, packed);
                    o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[hblk][sblk], o[t], 0, 0, 0);
                }
    }
    if (myq >= S) return;
    const float inv = 1.0f / l_run;
    // O^T element r of block t: dh 32 t + 8 (r/4) + 4 lh + r%4, query myq
    bf16_t* dst = out + ((size_t)b * S + myq) * d + hd * DH;
#pragma unroll
    for (int t = 0; t < OT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[32 * t + 8 * (r >> 2) + 4 * lh + (r & 3)] = f2bf(o[t][r] * inv);
}

// ============================================================ host side
int cdiv(int a, int b) { return (a + b - 1) / b; }

template <int BM, int BN, int EPI, bool PERT>
zo_status launch_gemm(const GemmParams& gp, const Pert& p, hipStream_t s, const char* fam)
{
    const int blocks = cdiv(gp.M, BM) * cdiv(gp.N, BN);
    if constexpr (PERT) {
        // perturbed tiles pass through registers: z is applied before the LDS store
        constexpr int LDK = 64 + 8;
        const size_t lds = std::max((size_t)(2 * BM * LDK + 2 * BN * LDK) * sizeof(bf16_t),
                                    epilogue_lds_bytes<BM, BN>());
        auto kern = gemm_bf16_kernel<BM, BN, EPI, true>;
        static bool attr = false;
        if (!attr) {
            if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
                hipSuccess)
                return fail(ZO_ERR_HIP, "cannot reserve %zu bytes of LDS", lds);
            attr = true;
        }
        KernelTimer timer(fam, s);
        kern<<<blocks, kThreads, lds, s>>>(gp, p);
    } else {
        // 256-wide tiles: a ring of dma_stages<EPI>() BK = 32 stages; 128-wide: 2-stage BK = 64
        constexpr bool big = BM == 256;
        // the LM head's cross-entropy epilogue needs two wave columns of 4 waves
        constexpr bool eight = !big && EPI != EPI_LMHEAD;
        constexpr size_t stages = big ? (size_t)dma_stages<EPI>() * (BM + BN) * 32 * sizeof(bf16_t)
                                      : (size_t)2 * (BM + BN) * 64 * sizeof(bf16_t);
        constexpr size_t lds = std::max(stages, epilogue_lds_bytes<BM, BN>());
        void (*kern)(GemmParams);
        if constexpr (big)
            kern = gemm_bf16_dma_kernel<BM, BN, EPI>;
        else if constexpr (eight)
            kern = gemm_bf16_k64_kernel<BM, BN, EPI, 512, 4>;
        else
            kern = gemm_bf16_k64_kernel<BM, BN, EPI, kThreads, 2>;
        static bool attr = false;
        if (!attr) {
            if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
                hipSuccess)
                return fail(ZO_ERR_HIP, "cannot reserve %zu bytes of LDS", lds);
            attr = true;
        }
        KernelTimer timer(fam, s);
        kern<<<blocks, (big || eight) ? kDmaThreads : kThreads, lds, s>>>(gp);
    }
    return check_launch("bf16 GEMM");
}

// Tile choice: 256x256 when the grid still fills the 256 CUs, else 128x128.
// The register-staged perturbed kernel keeps the LM head at 128x128 (its
// 256-wide cross-entropy epilogue would not fit the registers).
template <int EPI, bool PERT>
constexpr bool may_use_big_tiles() { return !(PERT && EPI == EPI_LMHEAD); }

int gemm_tile_n(int M, int N, bool pert, int epi)
{
    const long big = (long)cdiv(M, 256) * cdiv(N, 256);
    return (big >= 256 && !(pert && epi == EPI_LMHEAD)) ? 256 : 128;
}

template <int EPI, bool PERT>
zo_status gemm(const GemmParams& gp, const Pert& p, hipStream_t s, const char* fam)
{
    if constexpr (may_use_big_tiles<EPI, PERT>()) {
        if (gemm_tile_n(gp.M, gp.N, PERT, EPI) == 256) return launch_gemm<256, 256, EPI, PERT>(gp, p, s, fam);
    }
    if constexpr (!PERT && EPI != EPI_LMHEAD) {
        // narrow outputs: 128 x 64 tiles when 128 x 128 would leave CUs idle
        if ((long)cdiv(gp.M, 128) * cdiv(gp.N, 128) < 256) return launch_gemm<128, 64, EPI, PERT>(gp, p, s, fam);
    }
    return launch_gemm<128, 128, EPI, PERT>(gp, p, s, fam);
}

template <int EPI>
zo_status gemm_any(const GemmParams& gp, const Pert& p, hipStream_t s, const char* fam)
{
    return p.on ? gemm<EPI, true>(gp, p, s, fam) : gemm<EPI, false>(gp, p, s, fam);
}

struct DecoderWs {
    bf16_t *h, *x, *qkv, *att, *u;
    float *lm_max, *lm_sum, *lm_pick;
    double* ce_part;
    size_t bytes;
};

constexpr int kLmTile = 128;  // narrowest LM-head tile: sizes the per-tile partials

DecoderWs carve(const zo_model_desc& d, void* base)
{
    const size_t M = (size_t)d.batch * d.seq;
    const size_t D = d.d_model, F = d.ffn;
    const size_t tiles = cdiv((int)d.vocab, kLmTile);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) / 256 * 256;
        return (char*)base + o;
    };
    DecoderWs w;
    w.h = (bf16_t*)take(M * D * 2);
    w.x = (bf16_t*)take(M * D * 2);
    w.qkv = (bf16_t*)take(M * 3 * D * 2);
    w.att = (bf16_t*)take(M * D * 2);
    w.u = (bf16_t*)take(M * F * 2);
    w.lm_max = (float*)take(tiles * M * 4);
    w.lm_sum = (float*)take(tiles * M * 4);
    w.lm_pick = (float*)take(M * 4);
    w.ce_part = (double*)take((M + 63) / 64 * 8);
    w.bytes = off;
    return w;
}

}  // namespace

zo_status decoder_check(const zo_model_desc& d)
{
    const int64_t dh = d.d_model / d.heads;
    if (dh != 64 && dh != 128) return fail(ZO_ERR_UNSUPPORTED, "head dim must be 64 or 128");
    if (d.d_model % 64 || d.ffn % 64) return fail(ZO_ERR_UNSUPPORTED, "d_model and ffn must be multiples of 64");
    if (d.d_model > 64 * 4 * kLnMaxQuads) return fail(ZO_ERR_UNSUPPORTED, "d_model too large for LayerNorm");
    if (d.batch * d.seq > (1 << 24) || d.vocab > (1 << 24)) return fail(ZO_ERR_UNSUPPORTED, "shape too large");
    return ZO_OK;
}

size_t decoder_workspace(const zo_model_desc& d) { return carve(d, nullptr).bytes; }

zo_status decoder_forward(const ModelView& m, const zo_batch& b, const zo_pert* perts, int n, double* loss,
                          hipStream_t s)
{
    const zo_model_desc& d = m.desc;
    const int B = (int)b.batch, S = (int)b.seq, D = (int)d.d_model, F = (int)d.ffn, V = (int)d.vocab;
    const int H = (int)d.heads, dh = D / H, L = (int)d.layers;
    const int M = B * S;
    DecoderWs w = carve(d, m.workspace);
    const bf16_t* P = (const bf16_t*)m.params;
    // tensor order: tok_emb, pos_emb, per layer (ln1_g, ln1_b, w_qkv, w_o, ln2_g, ln2_b, w_up, w_down), lnf_g, lnf_b
    auto off = [&](int idx) { return m.offsets[idx]; };
    const int n_evals = n == 0 ? 1 : n;
    for (int e = 0; e < n_evals; ++e) {
        Pert p = {};
        if (n) {
            p.key = Key{(uint32_t)perts[e].seed, (uint32_t)(perts[e].seed >> 32)};
            p.probe = perts[e].probe;
            p.sigma = perts[e].sigma;
            p.on = 1;
        }
        {
            KernelTimer t("embed", s);
            embed_kernel<<<M, kThreads, 0, s>>>(b.tokens, S, D, P + off(0), off(0), P + off(1), off(1), p, w.h);
            if (zo_status st = check_launch("embed")) return st;
        }
        for (int l = 0; l < L; ++l) {
            const int t0 = 2 + 8 * l;
            {
                KernelTimer t("layernorm", s);
                launch_layernorm(w.h, M, D, P + off(t0), off(t0), P + off(t0 + 1), off(t0 + 1), p, w.x, s);
                if (zo_status st = check_launch("layernorm")) return st;
            }
            GemmParams gq = {};
            gq.A = w.x; gq.W = P + off(t0 + 2); gq.w_dir = off(t0 + 2); gq.C = w.qkv; gq.M = M; gq.N = 3 * D; gq.K = D;
            if (zo_status st = gemm_any<EPI_STORE>(gq, p, s, "gemm_bf16")) return st;
            {
                KernelTimer t("attention", s);
                const int blocks = B * H * cdiv(S, 128);
                if (dh == 64)
                    attention_kernel<64><<<blocks, kThreads, 0, s>>>(w.qkv, S, D, H, w.att);
                else
                    attention_kernel<128><<<blocks, kThreads, 0, s>>>(w.qkv, S, D, H, w.att);
                if (zo_status st = check_launch("attention")) return st;
            }
            GemmParams go = {};
            go.A = w.att; go.W = P + off(t0 + 3); go.w_dir = off(t0 + 3); go.C = w.h; go.M = M; go.N = D; go.K = D;
            if (zo_status st = gemm_any<EPI_RESID>(go, p, s, "gemm_bf16")) return st;
            {
                KernelTimer t("layernorm", s);
                launch_layernorm(w.h, M, D, P + off(t0 + 4), off(t0 + 4), P + off(t0 + 5), off(t0 + 5), p, w.x, s);
                if (zo_status st = check_launch("layernorm")) return st;
            }
            GemmParams gu = {};
            gu.A = w.x; gu.W = P + off(t0 + 6); gu.w_dir = off(t0 + 6); gu.C = w.u; gu.M = M; gu.N = F; gu.K = D;
            zo_status su = d.act == ZO_ACT_GELU ? gemm_any<EPI_GELU>(gu, p, s, "gemm_bf16")
                                                : gemm_any<EPI_RELU>(gu, p, s, "gemm_bf16");
            if (su) return su;
            GemmParams gd = {};
            gd.A = w.u; gd.W = P + off(t0 + 7); gd.w_dir = off(t0 + 7); gd.C = w.h; gd.M = M; gd.N = D; gd.K = F;
            if (zo_status st = gemm_any<EPI_RESID>(gd, p, s, "gemm_bf16")) return st;
        }
        const int tf = 2 + 8 * L;
        {
            KernelTimer t("layernorm", s);
            launch_layernorm(w.h, M, D, P + off(tf), off(tf), P + off(tf + 1), off(tf + 1), p, w.x, s);
            if (zo_status st = check_launch("layernorm")) return st;
        }
        GemmParams gl = {};
        gl.A = w.x; gl.W = P + off(0); gl.w_dir = off(0); gl.M = M; gl.N = V; gl.K = D;
        gl.lm_max = w.lm_max; gl.lm_sum = w.lm_sum; gl.lm_pick = w.lm_pick; gl.tokens = b.tokens; gl.S = S;
        if (zo_status st = gemm_any<EPI_LMHEAD>(gl, p, s, "lm_head")) return st;
        {
            KernelTimer t("reduce", s);
            const int nb = cdiv(M, 64);
            const int lm_tiles = cdiv(V, gemm_tile_n(M, V, p.on != 0, EPI_LMHEAD));
            ce_rows_kernel<<<nb, kThreads, 0, s>>>(w.lm_max, w.lm_sum, w.lm_pick, lm_tiles, M, S, w.ce_part);
            ce_final_kernel<<<1, kThreads, 0, s>>>(w.ce_part, nb, M, S, loss + e);
            if (zo_status st = check_launch("ce reduce")) return st;
        }
    }
    return ZO_OK;
}

// ------------------------------------------------------------ debug entries
zo_status debug_gemm_bf16(const void* A, const void* W, void* C, int M, int N, int K, int epi, hipStream_t s)
{
    if (!A || !W || !C || M <= 0 || N <= 0 || K <= 0) return fail(ZO_ERR_INVALID, "bad GEMM arguments");
    if (K % 64) return fail(ZO_ERR_UNSUPPORTED, "K must be a multiple of 64");
    if (N % 8) return fail(ZO_ERR_UNSUPPORTED, "N must be a multiple of 8");
    if (((uintptr_t)A | (uintptr_t)W | (uintptr_t)C) & 15) return fail(ZO_ERR_INVALID, "A, W, C must be 16-byte aligned");
    GemmParams g = {};
    g.A = (const bf16_t*)A; g.W = (const bf16_t*)W; g.C = (bf16_t*)C; g.M = M; g.N = N; g.K = K;
    Pert p = {};
    switch (epi) {
        case 0: return gemm_any<EPI_STORE>(g, p, s, "gemm_bf16");
        case 1: return gemm_any<EPI_GELU>(g, p, s, "gemm_bf16");
        case 2: return gemm_any<EPI_RELU>(g, p, s, "gemm_bf16");
        case 3: return gemm_any<EPI_RESID>(g, p, s, "gemm_bf16");
    }
    return fail(ZO_ERR_INVALID, "epilogue must be 0..3");
}

zo_status debug_attention(const void* qkv, void* out, int B, int S, int H, int dh, hipStream_t s)
{
    if (!qkv || !out || B <= 0 || S <= 0 || H <= 0) return fail(ZO_ERR_INVALID, "bad attention arguments");
    if (dh != 64 && dh != 128) return fail(ZO_ERR_UNSUPPORTED, "head dim must be 64 or 128");
    const int blocks = B * H * cdiv(S, 128);
    KernelTimer t("attention", s);
    if (dh == 64)
        attention_kernel<64><<<blocks, kThreads, 0, s>>>((const bf16_t*)qkv, S, H * dh, H, (bf16_t*)out);
    else
        attention_kernel<128><<<blocks, kThreads, 0, s>>>((const bf16_t*)qkv, S, H * dh, H, (bf16_t*)out);
    return check_launch("attention");
}

zo_status debug_layernorm(const void* h, const void* g, const void* b, void* x, int rows, int d, hipStream_t s)
{
    if (!h || !g || !b || !x || rows <= 0 || d <= 0) return fail(ZO_ERR_INVALID, "bad LayerNorm arguments");
    if (d > 64 * 4 * kLnMaxQuads || d % 4) return fail(ZO_ERR_UNSUPPORTED, "row length must be a multiple of 4, <= 8192");
    Pert p = {};
    KernelTimer t("layernorm", s);
    launch_layernorm((const bf16_t*)h, rows, d, (const bf16_t*)g, 0, (const bf16_t*)b, 0, p, (bf16_t*)x, s);
    return check_launch("layernorm");
}

}  // namespace zo
