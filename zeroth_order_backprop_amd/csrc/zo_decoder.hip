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
#include <new>
#include <vector>
#include <math.h>
#include <string.h>

#include "zo_internal.hpp"
#include "zo_math.hpp"
#include "zo_models.hpp"
#include "zo_rng.hpp"
#include "zo_dirs8.hpp"

// The buffer-resource direct-to-LDS load (llvm.amdgcn.raw.buffer.load.lds).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ void zo_raw_buffer_load_lds(i32x4_t rsrc, __attribute__((address_space(3))) void* lds, int size,
                                       int voffset, int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");
// 16-byte buffer load / store (an offset past the resource's size reads
// zeros, writes nothing).
__device__ void zo_raw_buffer_store_x4(i32x4_t data, i32x4_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.store.v4i32");
__device__ i32x4_t zo_raw_buffer_load_x4(i32x4_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");

namespace zo {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;

constexpr int kThreads = 256;
constexpr int kGemmThreads = 256, kGemmWavesM = 2;  // stored-weight GEMM tiles (256 or 128 wide)

// A perturbation applied while reading weights.
struct Pert {
    Key key;
    uint32_t probe;
    float sigma;
    int on;    // 0: stored weights as they are
    int dirs;  // ZO_DIRS_GAUSS, or ZO_DIRS_Q8: values T[code] from the code object's table (L1-resident)
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

// Word k of a Philox block.
__device__ __forceinline__ uint32_t word_of(uint4 c, uint32_t k)
{
    return k == 0 ? c.x : k == 1 ? c.y : k == 2 ? c.z : c.w;
}

// 8 consecutive bf16 weights starting at arena index j (j % 8 == 0 not
// required, j % 4 == 0 required), perturbed in place in the uint4; `tab`:
// the 8-bit table (an LDS copy where the caller has one).
__device__ __forceinline__ uint4 perturb8(uint4 v, uint64_t j, const Pert& p, const float* tab)
{
    float f[8] = {bf2f(v.x & 0xFFFF), bf2f(v.x >> 16), bf2f(v.y & 0xFFFF), bf2f(v.y >> 16),
                  bf2f(v.z & 0xFFFF), bf2f(v.z >> 16), bf2f(v.w & 0xFFFF), bf2f(v.w >> 16)};
    float z[8];
    if (p.dirs == ZO_DIRS_Q8) {
        // words j/4 and j/4 + 1 of the stream: one Philox block (two when
        // the pair straddles blocks)
        const uint64_t k0 = j >> 2;
        const uint4 c0 = dirs8::block(p.key, p.probe, k0 >> 2);
        const uint32_t w0 = (uint32_t)(k0 & 3u);
        const uint32_t lo = word_of(c0, w0);
        const uint32_t hi = w0 < 3 ? word_of(c0, w0 + 1) : dirs8::block(p.key, p.probe, (k0 >> 2) + 1).x;
#pragma unroll
        for (int t = 0; t < 8; ++t) z[t] = dirs8::code(tab, t < 4 ? lo : hi, t & 3);
    } else {
        const float4 za = gauss4(p.key, p.probe, j >> 2);
        const float4 zb = gauss4(p.key, p.probe, (j >> 2) + 1);
        z[0] = za.x; z[1] = za.y; z[2] = za.z; z[3] = za.w;
        z[4] = zb.x; z[5] = zb.y; z[6] = zb.z; z[7] = zb.w;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) f[t] = fmaf(p.sigma, z[t], f[t]);
    return uint4{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
}

// One perturbed weight (slow path: LN parameters, ragged ends).
// Row groups: rows [g R, (g + 1) R) of a launch belong to evaluation g, whose
// parameters sit g * stride elements after the first copy's (R = 0: one group).
struct RowGroups {
    int rows;
    uint64_t stride;
};

__device__ __forceinline__ float weight1(const bf16_t* w, uint64_t i, uint64_t dir, const Pert& p)
{
    float v = bf2f(w[i]);
    if (p.on) {
        const uint64_t j = dir + i;
        float zz;
        if (p.dirs == ZO_DIRS_Q8) {
            zz = dirs8::value1(dirs8::kTableDev.v, p.key, p.probe, j);
        } else {
            const float4 z = gauss4(p.key, p.probe, j >> 2);
            const uint32_t s = (uint32_t)(j & 3u);
            zz = s == 0 ? z.x : s == 1 ? z.y : s == 2 ? z.z : z.w;
        }
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
// A token id outside [0, V) reads nothing and gives its row NaN, so the loss
// of the evaluation comes out NaN (and a step skips its update).
__global__ __launch_bounds__(kThreads) void embed_kernel(const int32_t* __restrict__ tokens, int S, int d, int V,
                                                          const bf16_t* __restrict__ tok_emb, uint64_t tok_dir,
                                                          const bf16_t* __restrict__ pos_emb, uint64_t pos_dir,
                                                          Pert p, RowGroups gr, bf16_t* __restrict__ h)
{
    const int t = blockIdx.x;
    int tl = t;
    if (gr.rows) {
        const int gi = t / gr.rows;
        tl = t - gi * gr.rows;
        tok_emb += (uint64_t)gi * gr.stride;
        pos_emb += (uint64_t)gi * gr.stride;
    }
    const int tok = tokens[tl];
    const int s = t % S;
    if ((unsigned)tok >= (unsigned)V) {
        for (int c = threadIdx.x; c < d; c += kThreads) h[(size_t)t * d + c] = (bf16_t)0x7FC0u;
        return;
    }
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
                                                              RowGroups gr, bf16_t* __restrict__ x)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= rows) return;
    if (gr.rows) {
        const uint64_t go = (uint64_t)(t / gr.rows) * gr.stride;
        g += go;
        b += go;
    }
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

// Wide rows (d > 2048, d % 8 == 0): one 256-thread block per row, NO groups
// of 8 per thread (group q = tid + 256 k, one 16-byte load each); the sums
// are combined across the 4 waves through LDS in a fixed order.
template <int NO>
__global__ __launch_bounds__(kThreads) void layernorm_wide_kernel(const bf16_t* __restrict__ h, int d,
                                                                   const bf16_t* __restrict__ g, uint64_t g_dir,
                                                                   const bf16_t* __restrict__ b, uint64_t b_dir, Pert p,
                                                                   RowGroups gr, bf16_t* __restrict__ x)
{
    __shared__ float part[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t t = blockIdx.x;
    if (gr.rows) {
        const uint64_t go = (uint64_t)(blockIdx.x / gr.rows) * gr.stride;
        g += go;
        b += go;
    }
    const int no = d >> 3;
    const uint4* row = reinterpret_cast<const uint4*>(h + t * d);
    float v[NO][8];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NO; ++k) {
        const int q = tid + kThreads * k;
        if (q < no) {
            const uint4 u = row[q];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[k][2 * e] = bf2f(w[e] & 0xFFFF);
                v[k][2 * e + 1] = bf2f(w[e] >> 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[k][e] = 0.f;
        }
        s += ((v[k][0] + v[k][1]) + (v[k][2] + v[k][3])) + ((v[k][4] + v[k][5]) + (v[k][6] + v[k][7]));
    }
    s = wave_sumf(s);
    if (lane == 0) part[0][wave] = s;
    __syncthreads();
    const float mean = (((part[0][0] + part[0][1]) + part[0][2]) + part[0][3]) / (float)d;
    float q2 = 0.f;
#pragma unroll
    for (int k = 0; k < NO; ++k) {
        if (tid + kThreads * k < no) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
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
    uint4* out = reinterpret_cast<uint4*>(x + t * d);
#pragma unroll
    for (int k = 0; k < NO; ++k) {
        const int q = tid + kThreads * k;
        if (q >= no) continue;
        float o[8];
        if (p.on) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 8 * q + e;
                o[e] = fmaf((v[k][e] - mean) * rstd, weight1(g, c, g_dir, p), weight1(b, c, b_dir, p));
            }
        } else {
            const uint4 gg = reinterpret_cast<const uint4*>(g)[q];
            const uint4 bb = reinterpret_cast<const uint4*>(b)[q];
            const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w}, bw[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[2 * e] = fmaf((v[k][2 * e] - mean) * rstd, bf2f(gw[e] & 0xFFFF), bf2f(bw[e] & 0xFFFF));
                o[2 * e + 1] = fmaf((v[k][2 * e + 1] - mean) * rstd, bf2f(gw[e] >> 16), bf2f(bw[e] >> 16));
            }
        }
        out[q] = uint4{pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7])};
    }
}

// LayerNorm of `rows` rows of width d (d % 4 == 0, and d % 8 == 0 above 2048;
// d <= 8192): one wave per
// row with the smallest register footprint that holds it (NQ groups of 4 per
// lane) up to d = 2048, one block per row beyond.
void launch_layernorm(const bf16_t* h, int rows, int d, const bf16_t* g, uint64_t g_dir, const bf16_t* b,
                      uint64_t b_dir, const Pert& p, bf16_t* x, hipStream_t s, RowGroups gr = RowGroups{0, 0})
{
    const int nq = (d / 4 + 63) / 64;
    const dim3 grid((rows + 3) / 4);
    if (nq <= 1) layernorm_kernel<1><<<grid, kThreads, 0, s>>>(h, rows, d, g, g_dir, b, b_dir, p, gr, x);
    else if (nq <= 3) layernorm_kernel<3><<<grid, kThreads, 0, s>>>(h, rows, d, g, g_dir, b, b_dir, p, gr, x);
    else if (nq <= 8) layernorm_kernel<8><<<grid, kThreads, 0, s>>>(h, rows, d, g, g_dir, b, b_dir, p, gr, x);
    else layernorm_wide_kernel<kLnMaxQuads / 8><<<rows, kThreads, 0, s>>>(h, d, g, g_dir, b, b_dir, p, gr, x);
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
    const int32_t* tokens;  // targets: row r's target is tokens[r + 1] (same sequence;
    int S;                  // read by the perturbed-tile LM head only)
    // row groups (stored-weight kernels only): rows [g R, (g + 1) R) use the
    // weights grp_stride * g elements after W (R = grp_rows; 0: one group)
    int grp_rows;
    uint64_t grp_stride;
};


// Linear tile index -> (tm, tn): consecutive workgroups land on consecutive
// XCDs, so give each XCD a contiguous range of tiles, and walk tiles in
// groups of G M-tiles so neighbours share A rows and W columns in L2.
template <int G = 8>
__device__ __forceinline__ void tile_of(int b, int nbm, int nbn, int& tm, int& tn)
{
    const int total = nbm * nbn;
    // blocks go round-robin to the 8 XCDs: each XCD takes a contiguous range
    const int nx = total / 8, rx = total % 8, xcd = b % 8;
    const int t = xcd * nx + min(xcd, rx) + b / 8;
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
                    // a target outside the vocabulary gives the row a NaN loss
                    if ((unsigned)target >= (unsigned)N && tn == 0 && wn == 0 && lr == 0)
                        g.lm_pick[row] = __builtin_nanf("");
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
    // 8-bit directions: the code table in LDS (a dependent lookup per weight)
    __shared__ float q8tab[PERT ? 256 : 1];
    if constexpr (PERT) {
        if (p.dirs == ZO_DIRS_Q8) dirs8::load_table(q8tab);
        __syncthreads();
    }
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
                if (gn < N && gk < K) v = perturb8(v, g.w_dir + (uint64_t)gn * K + gk, p, q8tab);
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

// The perturbed-tile product with the block's weight panel resident in LDS:
// a block owns 64 output columns, writes D(W + sigma z) of those 64 rows over
// all of K into LDS once (rows padded by 8 bf16: the 16 rows of a fragment
// read then start 4 banks apart), and walks the 128-row tiles mt = ms,
// ms + msplit, ... of the activations, which stream through a two-stage
// register-staged ring.  Each weight's direction is thus generated once per
// block instead of once per 128-row tile; the products and their summation
// order are those of gemm_bf16_kernel<128, 64, EPI, true>.  Needs K % 64 == 0
// and 64 (K + 8) + 2 128 72 bf16 of LDS (K <= 960).
constexpr int kPanelBN = 64, kPanelBM = 128, kPanelMaxK = 960;
constexpr size_t panel_lds_bytes(int K) { return ((size_t)kPanelBN * (K + 8) + 2 * kPanelBM * 72) * sizeof(bf16_t); }

template <int EPI>
__global__ __launch_bounds__(kThreads) void gemm_pert_panel_kernel(GemmParams g, Pert p, int msplit)
{
    constexpr int BM = kPanelBM, BN = kPanelBN, BK = 64, LDK = BK + 8;
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int RB = WM / 32, CB = WN / 32;
    constexpr int A_CH = BM * BK / 8, A_PER = A_CH / kThreads;
    static_assert(A_CH % kThreads == 0 && EPI != EPI_LMHEAD, "tile / thread mismatch");
    extern __shared__ __align__(16) bf16_t lds[];
    __shared__ float q8tab[256];
    if (p.dirs == ZO_DIRS_Q8) dirs8::load_table(q8tab);
    __syncthreads();

    const int M = g.M, N = g.N, K = g.K, LDW = K + 8;
    bf16_t* wp = lds;  // [BN][LDW]
    auto As = [&](int st) { return lds + BN * LDW + st * (BM * LDK); };
    const int npanels = (N + BN - 1) / BN;
    const int pn = blockIdx.x % npanels, ms = blockIdx.x / npanels;
    const int n0 = pn * BN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, lh = lane >> 5;

    // the perturbed panel
    const int cpr = K / 8;
    for (int c = tid; c < BN * cpr; c += kThreads) {
        const int r = c / cpr, kc = 8 * (c % cpr);
        const int gn = n0 + r;
        uint4 v = uint4{0u, 0u, 0u, 0u};
        if (gn < N) {
            v = *reinterpret_cast<const uint4*>(g.W + (size_t)gn * K + kc);
            v = perturb8(v, g.w_dir + (uint64_t)gn * K + kc, p, q8tab);
        }
        *reinterpret_cast<uint4*>(wp + r * LDW + kc) = v;
    }

    uint4 ra[A_PER];
    auto load = [&](int m0, int k0) {
#pragma unroll
        for (int t = 0; t < A_PER; ++t) {
            const int c = tid + t * kThreads;
            const int r = c / (BK / 8), kc = 8 * (c % (BK / 8));
            const int gm = m0 + r, gk = k0 + kc;
            ra[t] = gm < M ? *reinterpret_cast<const uint4*>(g.A + (size_t)gm * K + gk) : uint4{0u, 0u, 0u, 0u};
        }
    };
    auto store = [&](int stage) {
#pragma unroll
        for (int t = 0; t < A_PER; ++t) {
            const int c = tid + t * kThreads;
            const int r = c / (BK / 8), kc = 8 * (c % (BK / 8));
            *reinterpret_cast<uint4*>(As(stage) + r * LDK + kc) = ra[t];
        }
    };
    const int KT = K / BK, nmt = (M + BM - 1) / BM;
    for (int mt = ms; mt < nmt; mt += msplit) {
        const int m0 = mt * BM;
        f32x16 acc[RB][CB];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j) acc[i][j] = f32x16{};
        load(m0, 0);
        store(0);
        __syncthreads();  // (the first trip: the panel is complete too)
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < KT) load(m0, (kt + 1) * BK);
#pragma unroll
            for (int ks = 0; ks < BK; ks += 16) {
                bf16x8 af[RB], bfr[CB];
#pragma unroll
                for (int i = 0; i < RB; ++i)
                    af[i] = *reinterpret_cast<const bf16x8*>(As(cur) + (wm * WM + i * 32 + lr) * LDK + ks + 8 * lh);
#pragma unroll
                for (int j = 0; j < CB; ++j)
                    bfr[j] = *reinterpret_cast<const bf16x8*>(wp + (wn * WN + j * 32 + lr) * LDW + kt * BK + ks +
                                                              8 * lh);
#pragma unroll
                for (int i = 0; i < RB; ++i)
#pragma unroll
                    for (int j = 0; j < CB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
            if (kt + 1 < KT) store(cur ^ 1);
            __syncthreads();
        }
        // the epilogue stages the tile in the ring's LDS (every wave is done
        // with it), then the next tile refills the ring
        gemm_epilogue<BM, BN, EPI>(g, acc, m0, n0, pn, As(0));
        __syncthreads();
    }
}

// The same product with the stage tiles written to LDS directly by the loads
// (global_load_lds, 16 B per lane) for the stored-weight path: no register
// staging.  Rows past M or N load a clamped (valid) row and are never stored.
// Barriers are bare s_barrier after each wave has waited (vmcnt) for its own
// share of a stage, so that later stages stay in flight across them.

// Direct-to-LDS loads through a buffer resource (MUBUF "buffer_load ... lds"):
// 16 bytes per lane land at the wave-uniform LDS address + 16 x lane.  Unlike
// the flat-encoded global_load_lds, the compiler counts these on vmcnt alone,
// so its waits for LDS fragment reads (lgkmcnt) can stay partial.  The
// resource covers `bytes` bytes from `base` (no stride; loads beyond return
// zeros) with the raw-buffer configuration word of the gfx9 family.

__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    i32x4_t r;
    r.x = (int)(uint32_t)a;
    r.y = (int)(uint32_t)(a >> 32);  // stride 0
    r.z = (int)bytes;
    r.w = 0x00020000;
    return r;
}

// vmcnt(n) with expcnt / lgkmcnt left at their maxima (gfx9 encoding)
#define ZO_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
#define ZO_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4))

// The activated, bf16-rounded tile of 16x16 accumulators into `smem`, rows
// padded by 8 bf16 (element r of a 16x16 block: row 4 (lane / 16) + r, column
// lane % 16).
template <int BM, int BN, int EPI, int NT, int WGM, int RB, int CB>
__device__ __forceinline__ void epilogue16_stage(f32x4 (&acc)[RB][CB], bf16_t* smem)
{
    constexpr int WGN = NT / 64 / WGM, WM = BM / WGM, WN = BN / WGN, LDC = BN + 8;
    static_assert(WM == RB * 16 && WN == CB * 16, "wave tile mismatch");
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WGN, wn = wave % WGN;
    const int l16 = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * WM + i * 16 + 4 * lq + r;
                const int col = wn * WN + j * 16 + l16;
                float v = acc[i][j][r];
                if constexpr (EPI == EPI_GELU) v = gelu_erf(v);
                if constexpr (EPI == EPI_RELU) v = fmaxf(v, 0.0f);
                smem[row * LDC + col] = f2bf(v);
            }
}

// The LM head's fused cross-entropy partials from a block tile of 16x16
// accumulators (element r of a 16x16 block: row 4 (lane / 16) + r, column
// lane % 16): per row the max and the sum of exp(logit - max) over the tile's
// columns, reduced over the 16 lanes of a row group and the two wave columns.
// (The target logits come from lm_pick_kernel.)  Full tiles skip the column
// bound checks; exp(x - m) is evaluated as 2^(x log2 e - m log2 e) with one fma.
template <int BM, int BN, int NT, int WGM, int RB, int CB>
__device__ __forceinline__ void lmhead_epilogue16(const GemmParams& g, f32x4 (&acc)[RB][CB], int m0, int n0, int tn)
{
    constexpr int WGN = NT / 64 / WGM, WM = BM / WGM, WN = BN / WGN;
    static_assert(WM == RB * 16 && WN == CB * 16, "wave tile mismatch");
    constexpr float kLog2e = 1.44269504088896341f;
    const int M = g.M, N = g.N;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WGN, wn = wave % WGN;
    const int l16 = lane & 15, lq = lane >> 4;
    const int cbase = n0 + wn * WN + l16;  // this lane's column of j = 0
    const bool full = n0 + BN <= N;        // uniform
    {
        static_assert(WGN == 2, "LM-head partials assume two wave columns");
        __shared__ float part_m[2][BM], part_s[2][BM];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int lrow = wm * WM + i * 16 + 4 * lq + r;
                float mx = -INFINITY;
                if (full) {
#pragma unroll
                    for (int j = 0; j < CB; ++j) mx = fmaxf(mx, acc[i][j][r]);
                } else {
#pragma unroll
                    for (int j = 0; j < CB; ++j)
                        if (cbase + 16 * j < N) mx = fmaxf(mx, acc[i][j][r]);
                }
#pragma unroll
                for (int o = 8; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
                const float mxl = mx * kLog2e;
                float se = 0.f;
                if (full) {
#pragma unroll
                    for (int j = 0; j < CB; ++j) se += __builtin_amdgcn_exp2f(fmaf(acc[i][j][r], kLog2e, -mxl));
                } else {
#pragma unroll
                    for (int j = 0; j < CB; ++j)
                        if (cbase + 16 * j < N) se += __builtin_amdgcn_exp2f(fmaf(acc[i][j][r], kLog2e, -mxl));
                }
#pragma unroll
                for (int o = 8; o > 0; o >>= 1) se += __shfl_xor(se, o, 64);
                if (l16 == 0) {
                    part_m[wn][lrow] = mx;
                    part_s[wn][lrow] = se;
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

// Scheduling groups spreading NR fragment reads (and after the barrier NR
// stage loads) evenly over NM MFMAs: read i follows MFMA (i + 1) NM / NR.
template <int I, int NR, int NM>
__device__ __forceinline__ void spread_pre()
{
    if constexpr (I < NR) {
        constexpr int c = (I + 1) * NM / NR - I * NM / NR;
        __builtin_amdgcn_sched_group_barrier(0x008, c, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        spread_pre<I + 1, NR, NM>();
    }
}
template <int I, int NR, int NM>
__device__ __forceinline__ void spread_post()
{
    if constexpr (I < NR) {
        constexpr int c = (I + 1) * NM / NR - I * NM / NR, c1 = c / 2;
        if constexpr (c1 > 0) __builtin_amdgcn_sched_group_barrier(0x008, c1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, c - c1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        spread_post<I + 1, NR, NM>();
    }
}

// Stored-weight GEMM tiles, 4 waves of 16x16x32 MFMAs in a 2 x 2 grid.
// 256 x 256 tiles: one wave per SIMD with a 128 x 128 wave tile (64
// accumulators of 4 in AGPRs), 128 KB of stages.  128 x 128 and 128 x 64 tiles
// (outputs too small to fill the CUs with 256-wide ones): 64 x 64 and 64 x 32
// wave tiles, 64 or 48 KB of stages, two or three blocks per CU.
// Two BK = 64 stages of (BM + BN) x 64 bf16; every row of a stage is one whole
// 128-byte line of A or W, so each direct-to-LDS load brings in full lines.
// Rows are 8 chunks of 16 B, chunk c of row r at position c ^ ((r >> 1) & 7):
// the 16 rows a fragment read touches (one chunk each) spread over all banks.
// A stage is two 32-deep k-steps read into alternating register sets.  With
// one wave per SIMD nothing covers a stall, so the wave's instruction stream
// is spread evenly: the k-step's fragment reads over its MFMAs (one per four
// on 256-wide tiles), and after the barrier one read and one stage load per
// such group (scheduling groups 0x008 MFMA, 0x100 LDS read, 0x020 global
// read; read and load alternate in the source, since the compiler keeps LDS
// reads ahead of the loads that write LDS).  On 256-wide tiles the same
// kernel with the reads clustered (one per MFMA over the first sixteen)
// measured 9% slower, eight waves of 64 x 128 with 32x32x16 MFMAs 9-12%
// slower; on the 128-wide tiles this kernel is 4-11% faster than eight waves
// of 32x32x16 MFMAs.
// Stage kt+2 is loaded into stage kt's buffer right after the barrier that
// ends every wave's reads of stage kt, so it has one stage of MFMAs to land.
// 256-wide tiles run a persistent grid (one block per CU walking its tiles in
// the order of tile_of).  With the stored epilogues the next tile's first two
// stages are issued before this tile's output stores: the stores, which all
// CUs issue at about the same time and which the chip's write bandwidth then
// paces, drain under the next tile's first k-step instead of before its first
// wait (vmcnt counts loads and stores in issue order, so any later wait
// covers them).
template <int BM, int BN, int EPI, int NT, int WGM>
__device__ __forceinline__ void gemm_dma_body(const GemmParams& g)
{
    constexpr int BK = 64;
    constexpr int WGN = NT / 64 / WGM;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int RB = WM / 16, CB = WN / 16;
    constexpr int A_INS = BM * 8 / NT, B_INS = BN * 8 / NT;
    constexpr int INS = A_INS + B_INS;
    constexpr int STAGE = (BM + BN) * BK;
    static_assert(A_INS * NT == BM * 8 && B_INS * NT == BN * 8, "tile / thread mismatch");
    // Stored epilogues overlap the next tile's first loads; the LM head's
    // partials finish before the next tile starts.
    constexpr bool OVERLAP = EPI != EPI_LMHEAD;
    // output chunks (16 B) per row and per thread
    constexpr int CPR = BN / 8, NST = BM * CPR / NT, LDC = BN + 8;
    static_assert(NST * NT == BM * CPR, "tile / thread mismatch");
    static_assert(INS + NST < 64, "vmcnt range");
    extern __shared__ __align__(16) bf16_t lds[];

    const int M = g.M, N = g.N, K = g.K;
    asm volatile("" ::"s"(g.C), "s"(g.lm_max), "s"(g.lm_sum), "s"(g.lm_pick), "s"(g.tokens), "s"(g.S));
    const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN, ntiles = nbm * nbn;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WGN, wn = wave % WGN;
    const int KT = K / BK;
    const i32x4_t ra = buffer_rsrc(g.A, (uint32_t)((size_t)M * K * 2));
    i32x4_t rw = buffer_rsrc(g.W, (uint32_t)((size_t)N * K * 2));

    // the output (stored epilogues; the host keeps M N 2 under 2 GiB)
    const i32x4_t rc = buffer_rsrc(g.C, OVERLAP ? (uint32_t)((size_t)M * N * 2) : 0u);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // the block's current tile and this thread's source offsets in it
    int tile = blockIdx.x, m0 = 0, n0 = 0, tn = 0;
    int voa[A_INS], vob[B_INS];
    auto set_tile = [&](int t) {
        int tm;
        tile_of<4>(t, nbm, nbn, tm, tn);
        m0 = tm * BM;
        n0 = tn * BN;
        if (g.grp_rows) {  // tiles never straddle groups (grp_rows % BM == 0)
            const int gi = __builtin_amdgcn_readfirstlane(m0 / g.grp_rows);
            rw = buffer_rsrc(g.W + (size_t)gi * g.grp_stride, (uint32_t)((size_t)N * K * 2));
        }
#pragma unroll
        for (int j = 0; j < A_INS; ++j) {
            const int p = j * NT + tid, row = p >> 3, lc = (p & 7) ^ ((row >> 1) & 7);
            voa[j] = (min(m0 + row, M - 1) * K + 8 * lc) * 2;
        }
#pragma unroll
        for (int j = 0; j < B_INS; ++j) {
            const int p = j * NT + tid, row = p >> 3, lc = (p & 7) ^ ((row >> 1) & 7);
            vob[j] = (min(n0 + row, N - 1) * K + 8 * lc) * 2;
        }
    };
    f32x4 acc[RB][CB];
    auto issue = [&](int kt) {
        bf16_t* sa = lds + (kt & 1) * STAGE;
        bf16_t* sb = sa + BM * BK;
        const int koff = min(kt, KT - 1) * BK * 2;
#pragma unroll
        for (int j = 0; j < A_INS; ++j) {
            bf16_t* dst = sa + (j * NT + wave_u * 64) * 8;
            zo_raw_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)dst, 16, voa[j], koff, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < B_INS; ++j) {
            bf16_t* dst = sb + (j * NT + wave_u * 64) * 8;
            zo_raw_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)dst, 16, vob[j], koff, 0, 0);
        }
    };
    // 16x16x32 operands: lane l holds row (l & 15) of its block, k-chunk l >> 4
    // of the 32-deep step; rows >> 1 & 7 of the swizzle come from l & 15 alone
    const int r16 = lane & 15, kq = lane >> 4, sw = (r16 >> 1) & 7;
    int aoff[2], boff[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        aoff[s] = (wm * WM + r16) * BK + (((4 * s + kq) ^ sw) * 8);
        boff[s] = BM * BK + (wn * WN + r16) * BK + (((4 * s + kq) ^ sw) * 8);
    }
    bf16x8 fa[2][RB], fb[2][CB];
    auto read = [&](int kt, int s, int slot) {
        const bf16_t* st = lds + (kt & 1) * STAGE;
#pragma unroll
        for (int j = 0; j < CB; ++j) fb[slot][j] = *reinterpret_cast<const bf16x8*>(st + boff[s] + j * 16 * BK);
#pragma unroll
        for (int i = 0; i < RB; ++i) fa[slot][i] = *reinterpret_cast<const bf16x8*>(st + aoff[s] + i * 16 * BK);
    };
    auto mma = [&](int slot) {
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
    };
    constexpr int NR = RB + CB, NM = RB * CB;  // fragment reads, MFMAs per k-step
    // one fragment read / one stage load by index (reads: B fragments first)
    auto read1 = [&](int kt, int s, int slot, int idx) {
        const bf16_t* st = lds + (kt & 1) * STAGE;
        if (idx < CB) fb[slot][idx] = *reinterpret_cast<const bf16x8*>(st + boff[s] + idx * 16 * BK);
        else fa[slot][idx - CB] = *reinterpret_cast<const bf16x8*>(st + aoff[s] + (idx - CB) * 16 * BK);
    };
    auto issue1 = [&](int kt, int idx) {
        bf16_t* sa = lds + (kt & 1) * STAGE;
        bf16_t* sb = sa + BM * BK;
        const int koff = min(kt, KT - 1) * BK * 2;
        if (idx < A_INS) {
            bf16_t* dst = sa + (idx * NT + wave_u * 64) * 8;
            zo_raw_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)dst, 16, voa[idx], koff, 0, 0);
        } else {
            bf16_t* dst = sb + ((idx - A_INS) * NT + wave_u * 64) * 8;
            zo_raw_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)dst, 16, vob[idx - A_INS], koff, 0, 0);
        }
    };
    static_assert(NR == INS, "spread pattern assumes as many reads as loads");

    set_tile(tile);
    issue(0);
    issue(1);
    bool stores_pending = false;  // the previous tile's output stores may be in flight
    for (;;) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) acc[i][j] = f32x4{};
    // stage 0 landed (stage 1 and the previous tile's stores may remain)
    if (stores_pending)
        ZO_WAIT_VM(INS + NST);
    else
        ZO_WAIT_VM(INS);
    asm volatile("s_barrier" ::: "memory");
    read(0, 0, 0);
    ZO_WAIT_LGKM0();
    for (int kt = 0; kt < KT - 1; ++kt) {
        __builtin_amdgcn_sched_barrier(0);
        read(kt, 1, 1);
        mma(0);
        spread_pre<0, NR, NM>();
        __builtin_amdgcn_sched_barrier(0);
        ZO_WAIT_VM(0);
        ZO_WAIT_LGKM0();
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int idx = 0; idx < NR; ++idx) {
            read1(kt + 1, 0, 0, idx);
            issue1(kt + 2, idx);
        }
        mma(1);
        spread_post<0, NR, NM>();
        __builtin_amdgcn_sched_barrier(0);
    }
    read(KT - 1, 1, 1);
    mma(0);
    mma(1);
    ZO_WAIT_VM(0);    // the trailing reloads have landed before the buffers are reused
    __syncthreads();  // every wave is done with the stage buffers
    const int next = tile + (int)gridDim.x;
    const bool more = next < ntiles;
    if constexpr (!OVERLAP) {
        lmhead_epilogue16<BM, BN, NT, WGM>(g, acc, m0, n0, tn);
        // (its stores then complete before the next tile's first wait ends)
        if (!more) break;
        __syncthreads();  // the epilogue's LDS use is over
        tile = next;
        set_tile(tile);
        issue(0);
        issue(1);
    } else {
        // The tile goes through LDS (rows padded by 8 bf16) into registers
        // (with the residual, h added there); once every wave has its chunks
        // the next tile's first two stages are issued, and only then this
        // tile's stores: the next tile's first wait then covers its own
        // loads, not these stores.
        epilogue16_stage<BM, BN, EPI, NT, WGM>(acc, lds);
        __syncthreads();
        // output chunk k of this thread: tile row p / CPR, 16-byte column p % CPR
        const int cm0 = m0, cn0 = n0;
        auto offs = [&](int k) {
            const int p = k * NT + tid, gr = cm0 + p / CPR, gc = cn0 + 8 * (p % CPR);
            return (gr < M && gc < N) ? (gr * N + gc) * 2 : (int)0x80000000u;  // past the end: dropped
        };
        if constexpr (EPI == EPI_RESID) {
            // h + bf16(product), rounded once more to bf16, back into this
            // thread's staged chunks; h read in batches of 8 chunks (every
            // load of a batch in flight at once)
            constexpr int HB = NST < 8 ? NST : 8;
            static_assert(NST % HB == 0, "whole batches");
            auto add2 = [](uint32_t hw, uint32_t pw) {
                return pack2(bf2f(hw & 0xFFFF) + bf2f(pw & 0xFFFF), bf2f(hw >> 16) + bf2f(pw >> 16));
            };
#pragma unroll
            for (int hb = 0; hb < NST / HB; ++hb) {
                i32x4_t hv[HB];
#pragma unroll
                // non-temporal (aux bit 1, nt): each h line is read once, so it
                // should not displace the operand panels the XCD's other tiles
                // are still reading from L2
                for (int k = 0; k < HB; ++k) hv[k] = zo_raw_buffer_load_x4(rc, offs(hb * HB + k), 0, 2);
#pragma unroll
                for (int k = 0; k < HB; ++k) {
                    const int p = (hb * HB + k) * NT + tid;
                    uint4* sp = reinterpret_cast<uint4*>(lds + (p / CPR) * LDC + 8 * (p % CPR));
                    const uint4 h = __builtin_bit_cast(uint4, hv[k]), v = *sp;
                    *sp = uint4{add2(h.x, v.x), add2(h.y, v.y), add2(h.z, v.z), add2(h.w, v.w)};
                }
            }
        }
        uint4 vals[NST];
#pragma unroll
        for (int k = 0; k < NST; ++k) {
            const int p = k * NT + tid;
            vals[k] = *reinterpret_cast<const uint4*>(lds + (p / CPR) * LDC + 8 * (p % CPR));
        }
        ZO_WAIT_LGKM0();
        asm volatile("s_barrier" ::: "memory");  // every wave has read its chunks
        if (more) {
            tile = next;
            set_tile(tile);
            issue(0);
            issue(1);
        }
#pragma unroll
        // non-temporal stores, for the same reason as the residual's reads
        // (O / down GEMMs 3-4% faster, OPT-1.3B-shaped QKV 2.5%)
        for (int k = 0; k < NST; ++k) zo_raw_buffer_store_x4(__builtin_bit_cast(i32x4_t, vals[k]), rc, offs(k), 0, 2);
        if (!more) break;
        stores_pending = true;
    }
    }
}

template <int BM, int BN, int EPI, int NT, int WGM>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(BM == 256 ? 1 : 2))) void gemm_bf16_dma_kernel(GemmParams g)
{
    gemm_dma_body<BM, BN, EPI, NT, WGM>(g);
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

// Target logits of the stored-weight LM head: pick[r] = x[r] . E[t] with
// t = tokens[r + 1], the next token of the same sequence (rows at a sequence
// end have none), E the token embedding (the tied head), fp32 accumulation of
// the bf16 products.  The GEMM's cross-entropy partials then need no
// per-element target test.  One wave per row, 16-byte loads (K % 8 == 0);
// row groups read their own copy of E.  An id outside the vocabulary gives
// the row a NaN loss.
__global__ __launch_bounds__(kThreads) void lm_pick_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ emb,
                                                            int K, const int32_t* __restrict__ tokens, int M, int S,
                                                            int V, RowGroups gr, float* __restrict__ pick)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= M || row % S == S - 1) return;
    int rl = row;
    if (gr.rows) {
        const int gi = row / gr.rows;
        rl = row - gi * gr.rows;
        emb += (uint64_t)gi * gr.stride;
    }
    const int t = tokens[rl + 1];
    if ((unsigned)t >= (unsigned)V) {
        if (lane == 0) pick[row] = __builtin_nanf("");
        return;
    }
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)row * K);
    const uint4* er = reinterpret_cast<const uint4*>(emb + (size_t)t * K);
    float acc = 0.f;
    for (int c = lane; c < K / 8; c += 64) {
        const uint4 a = xr[c], b = er[c];
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fmaf(bf2f(aw[e] & 0xFFFF), bf2f(bw[e] & 0xFFFF), acc);
            acc = fmaf(bf2f(aw[e] >> 16), bf2f(bw[e] >> 16), acc);
        }
    }
    acc = wave_sumf(acc);
    if (lane == 0) pick[row] = acc;
}

// loss = (sum of block sums, fixed order) / (B (S-1)), one block per row group
__global__ __launch_bounds__(kThreads) void ce_final_kernel(const double* __restrict__ block_sum, int n_blocks,
                                                             int M, int S, double* __restrict__ loss)
{
    // block g: row group g's loss from its n_blocks partial sums
    block_sum += (size_t)blockIdx.x * n_blocks;
    loss += blockIdx.x;
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
// Block: 4 waves x 32 queries = 128 queries; keys in tiles of BKV.  K and V
// tiles go straight from global memory into a ring of NSLOT LDS slots
// (buffer-resource direct-to-LDS loads, NSLOT - 1 tiles ahead, one barrier
// per tile), both key-major as in qkv; the V^T operand is read with the
// transposing LDS read ds_read_b64_tr_b16: within each 16-lane group, lane
// 4 q + r receives element r of the 8 bytes read by lanes q, 4 + q, 8 + q and
// 12 + q (lane 4 e + q reads key e, head-dim columns 4 q .. 4 q + 3, so lane
// 4 q + r gets keys 0..3 of column 4 q + r).  Rows are 16-byte chunks, chunk
// c of row r at position c ^ s(r).  The LDS serves 256 bytes (64 banks) a
// cycle: 16 lanes of a 16-byte read, 32 of an 8-byte one.  With 256-byte rows
// (d_h 128) every row starts on bank 0: s(r) = 4 (r & 3) + ((r >> 2) & 3)
// spreads the 16 rows of a K fragment read over the 16 bank groups and gives
// the 4 rows of a V^T read (4 chunks each) disjoint groups.  With 128-byte rows
// (d_h 64) odd rows start half-way: s(r) = 4 ((r >> 1) & 1) + ((r >> 2) & 3)
// does the same within each half.  (An earlier swizzle laid out for 32 banks
// left 2-way conflicts on K and 4-way on V^T: 6e7 conflict cycles a call.)
template <int DH>
__device__ __forceinline__ int att_swz(int row)
{
    return DH == 128 ? 4 * (row & 3) + ((row >> 2) & 3) : 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}

// Eight transposing LDS reads at per-lane addresses a[] plus a common
// immediate offset OFF (the 16-bit offset field, so that a ring slot known at
// compile time costs no address arithmetic), and the wait for them, in one
// asm statement: no register they write is reused before its data lands.
// (Through the builtin, the compiler waits for every direct-to-LDS load in
// flight, the next tiles' included, before each such read.)
template <int OFF>
__device__ __forceinline__ void ds_read_tr8_off(uint2 (&v)[8], const uint32_t (&a)[8])
{
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
        "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// Lane l and lane l ^ 32 combined through v_permlane32_swap (a VALU exchange
// of the two half-waves, no LDS round trip).  Both results of the swap hold
// one value of each half, so max and the sum come out the same in both lanes
// (the sum in the same operand order: low half first).
__device__ __forceinline__ float halves_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int V>
struct IntC {
    static constexpr int value = V;
};

template <int DH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(DH == 64 ? 3 : 2)))
void attention_kernel(const bf16_t* __restrict__ qkv, int S, int d, int H, bf16_t* __restrict__ out)
{
    constexpr int BQ = 128, BKV = DH == 64 ? 64 : 32;
    constexpr int NB = BKV / 32;  // 32-key blocks per tile
    constexpr int KS = DH / 16;   // MFMA k-steps over the head dim for S^T
    constexpr int OT = DH / 32;   // 32-row blocks of O^T
    constexpr int ROWB = DH * 2;  // bytes of a K or V row
    // ring depth: d_h 128 takes 4 slots (64 KB, 2 blocks per CU as its registers
    // allow anyway), d_h 64 keeps 3 (48 KB: 3 blocks per CU)
    constexpr int TILEB = BKV * ROWB, SLOTB = 2 * TILEB, NSLOT = DH == 128 ? 4 : 3;
    constexpr int LOADS = TILEB / 1024 / 4;  // 1 KB wave loads per wave per tile, each of K and V
    constexpr int STEPS = 8 / (2 * OT);      // P V^T k-steps per group of eight transposing reads
    static_assert(LOADS * 4 * 1024 == TILEB, "tile / wave mismatch");
    __shared__ __align__(16) unsigned char lds[NSLOT * SLOTB];

    const int qblocks = (S + BQ - 1) / BQ;
    // Blocks go round-robin to the 8 XCDs; renumbered so that each XCD runs a
    // contiguous range, every query block of a (sequence, head) shares one
    // L2 for its K and V (about a quarter faster than spreading them).
    const int nx = gridDim.x / 8, rx = gridDim.x % 8, xcd = blockIdx.x % 8;
    const int lb = xcd * nx + min(xcd, rx) + blockIdx.x / 8;
    // heaviest (latest) query blocks first
    const int qb = qblocks - 1 - (lb % qblocks);
    const int bh = lb / qblocks;
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
    const int ntiles = (kv_end + BKV - 1) / BKV;
    // Wave load j fills 1 KB block wave * LOADS + j of the K (V) tile, lane l
    // its bytes 16 l .. 16 l + 15.  The resource ends at the sequence's last
    // row: rows past S read as zeros (masked keys, multiplied by P = 0).
    const i32x4_t rs = buffer_rsrc(base, (uint32_t)((size_t)S * row_stride * 2));
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int lrow[LOADS], lcol[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int byte = (wave * LOADS + j) * 1024 + 16 * lane;
        const int row = byte / ROWB, pos = (byte % ROWB) / 16;
        lrow[j] = row;
        lcol[j] = 16 * (pos ^ att_swz<DH>(row));
    }
    // Tiles past the last reload rows no wave reads, so that every iteration
    // issues the same loads and waits for the same count.
    auto issue = [&](int t) {
        unsigned char* sk = lds + (t % NSLOT) * SLOTB;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const uint32_t ro = (uint32_t)(t * BKV + lrow[j]) * (uint32_t)(row_stride * 2) + lcol[j];
            unsigned char* dk = sk + (wave_u * LOADS + j) * 1024;
            zo_raw_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dk, 16, ro + 2 * koff, 0, 0, 0);
            zo_raw_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dk + TILEB), 16, ro + 2 * voff, 0,
                                   0, 0);
        }
    };
    // this lane's read offsets in a slot: K rows 32 hblk + lr, chunk 2 ks + lh;
    // V^T: key row (lane & 15) >> 2 of its group's four, columns 4 (lane & 3)
    const int ksw = att_swz<DH>(lr);
    const int g = lane >> 4, ve = (lane & 15) >> 2, vq = lane & 3;
    const int vrow = 4 * (g >> 1) + ve;
    const int vhalf = 8 * (vq & 1);
    // the swizzle of V^T rows vrow + 16 m + 8 h depends on h only
    int vcol[OT][2];
#pragma unroll
    for (int t = 0; t < OT; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            vcol[t][h] = 16 * ((4 * t + 2 * (g & 1) + (vq >> 1)) ^ att_swz<DH>(8 * h + vrow)) + vhalf;

    // d_h 128 has the registers for two tiles' K fragment sets: the next
    // tile's are read while this tile's scores are formed and its softmax
    // runs, which takes the LDS round trip off the critical path; the
    // cross-half reductions go through v_permlane32_swap.  (d_h 64, at three
    // waves per SIMD, has no such room: it reads each tile's fragments right
    // before its MFMAs.)
    // K fragments: d_h 128 has the registers for two tiles' sets, so the next
    // tile's are read while this tile's scores are formed and its softmax
    // runs (the LDS round trip leaves the critical path); d_h 64, at three
    // waves per SIMD, reads each tile's right before its MFMAs.
    constexpr bool PREK = DH == 128;
    static_assert(2 * NB % STEPS == 0, "whole V^T read groups");
    bf16x8 kf[PREK ? 2 : 1][NB][KS];
    // ring slot T: its K tile at a compile-time LDS offset
    auto read_k = [&](auto T, bf16x8 (&dst)[NB][KS]) {
        const unsigned char* sk = lds + decltype(T)::value * SLOTB;
#pragma unroll
        for (int hblk = 0; hblk < NB; ++hblk)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                dst[hblk][ks] =
                    *reinterpret_cast<const bf16x8*>(sk + (32 * hblk + lr) * ROWB + 16 * ((2 * ks + lh) ^ ksw));
    };
    // this lane's V^T read addresses for one group of eight reads in slot 0
    // (the slot and the group's first key row go into the offset field)
    uint32_t va[8];
#pragma unroll
    for (int u = 0; u < STEPS; ++u)
#pragma unroll
        for (int t = 0; t < OT; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                va[(u * OT + t) * 2 + h] = lds_addr(lds + TILEB + (16 * u + 8 * h + vrow) * ROWB + vcol[t][h]);

    for (int t = 0; t < NSLOT - 1; ++t) issue(t);
    // Q in registers before the loop: a wait for it there is partial (the
    // tiles' loads were issued after it), at the loop's entry it would be total
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
    if constexpr (PREK) {
        // tile 0 landed for every wave: its K fragments into set 0
        ZO_WAIT_VM(2 * LOADS * (NSLOT - 2));
        asm volatile("s_barrier" ::: "memory");
        read_k(IntC<0>{}, kf[0]);
    }
    // One key tile: it, its ring slot SL = it % NSLOT and (PREK) the K
    // fragment set KC = it % 2 holding it.
    auto step = [&](int it, auto KC, auto SL) {
        constexpr int kc = decltype(KC)::value, sl = decltype(SL)::value;
        const int k0 = it * BKV;
        // This wave's part of tile it (PREK: of tile it + 1, whose K
        // fragments this iteration reads) landed, later tiles may be in
        // flight; after the barrier every part has, and no wave still reads
        // the slot of tile it - 1 (PREK: its K fragments were read two
        // iterations ago), which is refilled.
        ZO_WAIT_VM(2 * LOADS * (NSLOT - (PREK ? 3 : 2)));
        ZO_WAIT_LGKM0();
        asm volatile("s_barrier" ::: "memory");
        issue(it + NSLOT - 1);
        // every key of this tile (and of all later ones) is after all of this
        // wave's queries
        if (k0 > qw + 31) return;
        // all of the tile's K fragments are read before the first MFMA (one
        // LDS round trip instead of one per MFMA: left alone, the compiler
        // waits before each)
        if constexpr (!PREK) read_k(SL, kf[0]);
        __builtin_amdgcn_sched_barrier(0);
        // S^T [BKV keys][32 queries] as NB 32x32 blocks, each one chain of
        // MFMAs over the head dim (a dependent MFMA issues back to back).
        f32x16 st[NB];
#pragma unroll
        for (int hblk = 0; hblk < NB; ++hblk) st[hblk] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int hblk = 0; hblk < NB; ++hblk)
                st[hblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kc][hblk][ks], qf[ks], st[hblk], 0, 0, 0);
        if constexpr (PREK) {
            // the next tile's K fragments, under these MFMAs and the softmax
            // (a tile past the last one is read into registers no result uses)
            __builtin_amdgcn_sched_barrier(0);
            read_k(IntC<(sl + 1) % NSLOT>{}, kf[1 - kc]);
            __builtin_amdgcn_sched_barrier(0);
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
        tmax = halves_max(tmax) * c;
        // Lazy rescaling: the reference max m_run is kept until some query of
        // the wave exceeds it by more than 8 (log2 units), so the weights
        // 2^(s c - m) stay at most 256 (fp32 sums and bf16 P carry them at the
        // same relative precision) and most tiles skip the rescale of O.
        const bool raise = __any(tmax > m_run + 8.0f);
        const float m_new = raise ? fmaxf(m_run, tmax) : m_run;
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
        psum = halves_sum(psum);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        // rescale only when some query of the wave raised its max
        if (raise) {
#pragma unroll
            for (int t = 0; t < OT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
        }
        // O^T += V^T P^T over the BKV keys in 2 NB MFMA k-steps; step (hblk, sblk)
        // uses accumulator elements 8 sblk .. 8 sblk + 7 of block hblk, i.e.
        // keys 32 hblk + 16 sblk + 8 (t/4) + 4 lh + t%4: the A operand (V^T rows
        // dh = 32 t + lr) takes the same keys in the same order, from two
        // transposing reads of four keys each (keys +0..3 and +8..11).  Groups
        // of eight reads cover STEPS such steps, at the slot's and the
        // group's offset.  While a wave issues these MFMA runs it takes issue
        // priority over the SIMD's other waves, whose score and softmax work
        // fills the MFMA pipe's shadow (about 2% at d_h 128; raising it for
        // the S^T runs too gains nothing).
        auto pv = [&](auto S0) {
            constexpr int s0 = decltype(S0)::value;
            uint2 v[8];
            ds_read_tr8_off<sl * SLOTB + 16 * s0 * ROWB>(v, va);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int u = 0; u < STEPS; ++u) {
                const int hblk = (s0 + u) >> 1, sblk = (s0 + u) & 1;
#pragma unroll
                for (int t = 0; t < OT; ++t) {
                    const uint2 lo = v[(u * OT + t) * 2], hi = v[(u * OT + t) * 2 + 1];
                    const uint4 packed = {lo.x, lo.y, hi.x, hi.y};
                    o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, packed), pb[hblk][sblk],
                                                                  o[t], 0, 0, 0);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        };
        pv(IntC<0>{});
        if constexpr (2 * NB > STEPS) pv(IntC<STEPS>{});
        static_assert(2 * NB <= 2 * STEPS, "at most two V^T read groups");
    };
    // NSLOT tiles per trip: every ring slot (and K fragment set) is a
    // compile-time choice; the trips end on a multiple of NSLOT, so the
    // tail's slots are known too
    static_assert(NSLOT == 3 || NSLOT == 4, "unrolled ring");
    static_assert(!PREK || NSLOT % 2 == 0, "K fragment sets alternate within a trip");
    int it = 0;
#pragma unroll 1
    for (; it + NSLOT - 1 < ntiles; it += NSLOT) {
        step(it, IntC<0>{}, IntC<0>{});
        step(it + 1, IntC<PREK ? 1 : 0>{}, IntC<1>{});
        step(it + 2, IntC<0>{}, IntC<2>{});
        if constexpr (NSLOT == 4) step(it + 3, IntC<PREK ? 1 : 0>{}, IntC<3>{});
    }
    if (it < ntiles) step(it, IntC<0>{}, IntC<0>{});
    if (it + 1 < ntiles) step(it + 1, IntC<PREK ? 1 : 0>{}, IntC<1>{});
    if constexpr (NSLOT == 4)
        if (it + 2 < ntiles) step(it + 2, IntC<0>{}, IntC<2>{});
    ZO_WAIT_VM(0);  // no load may land in LDS after the block ends
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

void launch_attention(const bf16_t* qkv, int B, int S, int d, int H, int dh, bf16_t* out, hipStream_t s)
{
    const int blocks = B * H * cdiv(S, 128);
    if (dh == 64)
        attention_kernel<64><<<blocks, kThreads, 0, s>>>(qkv, S, d, H, out);
    else
        attention_kernel<128><<<blocks, kThreads, 0, s>>>(qkv, S, d, H, out);
}

// Compute units of the current device (cached per device).
int device_cus()
{
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

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
        // every tile: 4 waves of 16x16x32 MFMAs, two BK = 64 stages
        constexpr bool big = BM == 256;
        constexpr size_t stages = (size_t)2 * (BM + BN) * 64 * sizeof(bf16_t);
        constexpr size_t lds = std::max(stages, epilogue_lds_bytes<BM, BN>());
        void (*kern)(GemmParams) = gemm_bf16_dma_kernel<BM, BN, EPI, kGemmThreads, kGemmWavesM>;
        const int threads = kGemmThreads;
        static bool attr = false;
        if (!attr) {
            if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
                hipSuccess)
                return fail(ZO_ERR_HIP, "cannot reserve %zu bytes of LDS", lds);
            attr = true;
        }
        KernelTimer timer(fam, s);
        // 256-wide tiles: a persistent grid of one block per CU walking its tiles
        kern<<<big ? std::min(blocks, device_cus()) : blocks, threads, lds, s>>>(gp);
    }
    return check_launch("bf16 GEMM");
}

// Tile choice: 256x256 when the grid still fills the 256 CUs, else 128x128.
// The register-staged perturbed kernel keeps the LM head at 128x128 (its
// 256-wide cross-entropy epilogue would not fit the registers).
template <int EPI, bool PERT>
constexpr bool may_use_big_tiles() { return !(PERT && EPI == EPI_LMHEAD); }

// 256x256 tiles (one block per CU, persistent) when they keep the CUs busy:
// at least one tile per CU and the last round of tiles at least 85% full
// (384 tiles on 256 CUs leave a third of the second round idle, where 128x128
// tiles at two or three blocks per CU spread evenly).  The GELU epilogue at
// 256x256 spills registers and costs as much as the MFMAs at K = 768, so
// short-K GELU products stay at 128x128.
int gemm_tile_n(int M, int N, int K, bool pert, int epi)
{
    if (pert && epi == EPI_LMHEAD) return 128;
    const long big = (long)cdiv(M, 256) * cdiv(N, 256);
    const long cus = device_cus();
    if (big < cus) return 128;
    if (epi == EPI_GELU && K < 2048) return 128;
    const long rounds = (big + cus - 1) / cus;
    return big * 100 >= rounds * cus * 85 ? 256 : 128;
}

// The panel-resident perturbed-tile product (see gemm_pert_panel_kernel):
// about one block per CU, each panel's 128-row tiles split among msplit blocks.
template <int EPI>
zo_status launch_gemm_panel(const GemmParams& gp, const Pert& p, hipStream_t s, const char* fam)
{
    const int npanels = cdiv(gp.N, kPanelBN), nmt = cdiv(gp.M, kPanelBM);
    const int msplit = std::max(1, std::min(nmt, (device_cus() + npanels / 2) / npanels));
    const size_t lds = panel_lds_bytes(gp.K);
    auto kern = gemm_pert_panel_kernel<EPI>;
    static bool attr = false;
    if (!attr) {
        if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)panel_lds_bytes(kPanelMaxK)) != hipSuccess)
            return fail(ZO_ERR_HIP, "cannot reserve %zu bytes of LDS", panel_lds_bytes(kPanelMaxK));
        attr = true;
    }
    KernelTimer timer(fam, s);
    kern<<<npanels * msplit, kThreads, lds, s>>>(gp, p, msplit);
    return check_launch("bf16 GEMM (weight panel)");
}

template <int EPI, bool PERT>
zo_status gemm(const GemmParams& gp, const Pert& p, hipStream_t s, const char* fam)
{
    if constexpr (PERT && EPI != EPI_LMHEAD) {
        // short K: the perturbed weight panel stays in LDS, each direction
        // generated once per block
        if (gp.K <= kPanelMaxK && gp.K % 64 == 0) return launch_gemm_panel<EPI>(gp, p, s, fam);
    }
    if constexpr (may_use_big_tiles<EPI, PERT>()) {
        if (gemm_tile_n(gp.M, gp.N, gp.K, PERT, EPI) == 256) return launch_gemm<256, 256, EPI, PERT>(gp, p, s, fam);
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

// Workspace for `groups` evaluations side by side (rows of every group).
DecoderWs carve(const zo_model_desc& d, void* base, int groups = 1)
{
    const size_t M = (size_t)groups * d.batch * d.seq;
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
    // GEMM operands are addressed with 31-bit byte offsets: activations
    // [M][D], [M][3D], [M][F]; weights [3D][D], [F][D], [D][F], [V][D]
    const int64_t M = d.batch * d.seq, D = d.d_model, F = d.ffn;
    const int64_t widest = std::max(std::max(3 * D, F), (int64_t)d.vocab);
    if (M * std::max(3 * D, F) * 2 >= (1ll << 31) || widest * D * 2 >= (1ll << 31))
        return fail(ZO_ERR_UNSUPPORTED, "a GEMM operand exceeds 2 GiB");
    return ZO_OK;
}

size_t decoder_workspace(const zo_model_desc& d) { return carve(d, nullptr).bytes; }
size_t decoder_group_workspace(const zo_model_desc& d, int groups) { return carve(d, nullptr, groups).bytes; }

// ---- captured forwards ----
// A forward at the stored weights is the same ~90 launches for every
// evaluation of a step; captured once into a HIP graph and replayed, the
// launches reach the GPU together instead of one by one (between small
// kernels the GPU otherwise idles several microseconds per launch).  One
// entry per (tokens, batch, seq, weights, row groups): the graph reads the
// weights, workspace and tokens through the pointers it was captured with.
// The first evaluation of a key runs eagerly (every one-time set-up done), the
// second captures.
namespace {
struct FwdGraph {
    const int32_t* tokens;
    int64_t batch, seq;
    const void* params;
    const void* ws;
    int groups;
    hipGraphExec_t exec;  // null: seen once, not captured yet
};
struct GraphCache {
    std::vector<FwdGraph> entries;
    hipStream_t capture = nullptr;
};
constexpr size_t kMaxGraphs = 8;

}  // namespace

void decoder_graphs_free(void* cache)
{
    auto* gc = static_cast<GraphCache*>(cache);
    if (!gc) return;
    for (auto& f : gc->entries)
        if (f.exec) (void)hipGraphExecDestroy(f.exec);
    if (gc->capture) (void)hipStreamDestroy(gc->capture);
    delete gc;
}

namespace {

// The launches of one evaluation up to the per-row cross-entropy partials.
// `groups` > 1: that many evaluations side by side, group g reading the
// parameter arena copy at P + g * gstride (stored-weight kernels only; the
// host keeps B S a multiple of 256 so that no GEMM tile straddles two groups).
zo_status decoder_eval_launches(const ModelView& m, const zo_batch& b, const Pert& p, const DecoderWs& w,
                                hipStream_t s, const bf16_t* P, int groups = 1, uint64_t gstride = 0)
{
    const zo_model_desc& d = m.desc;
    const int B = (int)b.batch, S = (int)b.seq, D = (int)d.d_model, F = (int)d.ffn, V = (int)d.vocab;
    const int H = (int)d.heads, dh = D / H, L = (int)d.layers;
    const int M = groups * B * S;
    const RowGroups gr = groups > 1 ? RowGroups{B * S, gstride} : RowGroups{0, 0};
    const int grp_rows = gr.rows;
    // tensor order: tok_emb, pos_emb, per layer (ln1_g, ln1_b, w_qkv, w_o, ln2_g, ln2_b, w_up, w_down), lnf_g, lnf_b
    auto off = [&](int idx) { return m.offsets[idx]; };
    {
        KernelTimer t("embed", s);
        embed_kernel<<<M, kThreads, 0, s>>>(b.tokens, S, D, V, P + off(0), off(0), P + off(1), off(1), p, gr, w.h);
        if (zo_status st = check_launch("embed")) return st;
    }
    for (int l = 0; l < L; ++l) {
        const int t0 = 2 + 8 * l;
        {
            KernelTimer t("layernorm", s);
            launch_layernorm(w.h, M, D, P + off(t0), off(t0), P + off(t0 + 1), off(t0 + 1), p, w.x, s, gr);
            if (zo_status st = check_launch("layernorm")) return st;
        }
        GemmParams gq = {};
        gq.A = w.x; gq.W = P + off(t0 + 2); gq.w_dir = off(t0 + 2); gq.C = w.qkv; gq.M = M; gq.N = 3 * D; gq.K = D;
        gq.grp_rows = grp_rows; gq.grp_stride = gstride;
        if (zo_status st = gemm_any<EPI_STORE>(gq, p, s, "gemm_bf16.qkv")) return st;
        {
            KernelTimer t("attention", s);
            launch_attention(w.qkv, groups * B, S, D, H, dh, w.att, s);
            if (zo_status st = check_launch("attention")) return st;
        }
        GemmParams go = {};
        go.A = w.att; go.W = P + off(t0 + 3); go.w_dir = off(t0 + 3); go.C = w.h; go.M = M; go.N = D; go.K = D;
        go.grp_rows = grp_rows; go.grp_stride = gstride;
        if (zo_status st = gemm_any<EPI_RESID>(go, p, s, "gemm_bf16.o")) return st;
        {
            KernelTimer t("layernorm", s);
            launch_layernorm(w.h, M, D, P + off(t0 + 4), off(t0 + 4), P + off(t0 + 5), off(t0 + 5), p, w.x, s, gr);
            if (zo_status st = check_launch("layernorm")) return st;
        }
        GemmParams gu = {};
        gu.A = w.x; gu.W = P + off(t0 + 6); gu.w_dir = off(t0 + 6); gu.C = w.u; gu.M = M; gu.N = F; gu.K = D;
        gu.grp_rows = grp_rows; gu.grp_stride = gstride;
        zo_status su = d.act == ZO_ACT_GELU ? gemm_any<EPI_GELU>(gu, p, s, "gemm_bf16.up")
                                            : gemm_any<EPI_RELU>(gu, p, s, "gemm_bf16.up");
        if (su) return su;
        GemmParams gd = {};
        gd.A = w.u; gd.W = P + off(t0 + 7); gd.w_dir = off(t0 + 7); gd.C = w.h; gd.M = M; gd.N = D; gd.K = F;
        gd.grp_rows = grp_rows; gd.grp_stride = gstride;
        if (zo_status st = gemm_any<EPI_RESID>(gd, p, s, "gemm_bf16.down")) return st;
    }
    const int tf = 2 + 8 * L;
    {
        KernelTimer t("layernorm", s);
        launch_layernorm(w.h, M, D, P + off(tf), off(tf), P + off(tf + 1), off(tf + 1), p, w.x, s, gr);
        if (zo_status st = check_launch("layernorm")) return st;
    }
    GemmParams gl = {};
    gl.A = w.x; gl.W = P + off(0); gl.w_dir = off(0); gl.M = M; gl.N = V; gl.K = D;
    gl.lm_max = w.lm_max; gl.lm_sum = w.lm_sum; gl.lm_pick = w.lm_pick; gl.tokens = b.tokens; gl.S = S;
    gl.grp_rows = grp_rows; gl.grp_stride = gstride;
    if (zo_status st = gemm_any<EPI_LMHEAD>(gl, p, s, "lm_head")) return st;
    if (!p.on) {
        // the stored-weight head's target logits (the perturbed-tile head picks
        // them in its epilogue)
        KernelTimer t("lm_head", s);
        lm_pick_kernel<<<cdiv(M, 4), kThreads, 0, s>>>(w.x, P + off(0), D, b.tokens, M, S, V, gr, w.lm_pick);
        if (zo_status st = check_launch("lm pick")) return st;
    }
    {
        KernelTimer t("reduce", s);
        const int lm_tiles = cdiv(V, gemm_tile_n(M, V, D, p.on != 0, EPI_LMHEAD));
        ce_rows_kernel<<<cdiv(M, 64), kThreads, 0, s>>>(w.lm_max, w.lm_sum, w.lm_pick, lm_tiles, M, S, w.ce_part);
        if (zo_status st = check_launch("ce rows")) return st;
    }
    return ZO_OK;
}

// The captured forward for this batch, or null when the evaluation should
// run eagerly (first sight of the batch).
zo_status forward_graph(const ModelView& m, const zo_batch& b, const DecoderWs& w, hipGraphExec_t* out,
                        const bf16_t* P, int groups, uint64_t gstride)
{
    *out = nullptr;
    auto*& gc = reinterpret_cast<GraphCache*&>(*m.graphs);
    if (!gc) {
        gc = new (std::nothrow) GraphCache;
        if (!gc) return fail(ZO_ERR_INVALID, "out of host memory");
    }
    for (auto& f : gc->entries)
        if (f.tokens == b.tokens && f.batch == (int64_t)b.batch && f.seq == (int64_t)b.seq && f.params == P &&
            f.ws == (const void*)w.h && f.groups == groups) {
            if (f.exec) {
                *out = f.exec;
                return ZO_OK;
            }
            // seen once: capture now
            if (!gc->capture && hipStreamCreateWithFlags(&gc->capture, hipStreamNonBlocking) != hipSuccess)
                return fail(ZO_ERR_HIP, "cannot create the capture stream");
            if (hipStreamBeginCapture(gc->capture, hipStreamCaptureModeThreadLocal) != hipSuccess)
                return fail(ZO_ERR_HIP, "cannot begin a graph capture");
            const zo_status st = decoder_eval_launches(m, b, Pert{}, w, gc->capture, P, groups, gstride);
            hipGraph_t graph = nullptr;
            const hipError_t e = hipStreamEndCapture(gc->capture, &graph);
            if (st || e != hipSuccess || !graph) {
                if (graph) (void)hipGraphDestroy(graph);
                return st ? st : fail(ZO_ERR_HIP, "graph capture failed: %s", hipGetErrorString(e));
            }
            hipGraphExec_t ex = nullptr;
            const hipError_t ei = hipGraphInstantiate(&ex, graph, nullptr, nullptr, 0);
            (void)hipGraphDestroy(graph);
            if (ei != hipSuccess || !ex) return fail(ZO_ERR_HIP, "graph instantiation failed: %s", hipGetErrorString(ei));
            f.exec = ex;
            *out = ex;
            return ZO_OK;
        }
    if (gc->entries.size() >= kMaxGraphs) {
        if (gc->entries.front().exec) (void)hipGraphExecDestroy(gc->entries.front().exec);
        gc->entries.erase(gc->entries.begin());
    }
    gc->entries.push_back(FwdGraph{b.tokens, (int64_t)b.batch, (int64_t)b.seq, P, w.h, groups, nullptr});
    return ZO_OK;
}

}  // namespace

zo_status decoder_forward(const ModelView& m, const zo_batch& b, const zo_pert* perts, int n, double* loss,
                          hipStream_t s)
{
    const zo_model_desc& d = m.desc;
    const int M = (int)(b.batch * b.seq), S = (int)b.seq;
    DecoderWs w = carve(d, m.workspace);
    const int n_evals = n == 0 ? 1 : n;
    for (int e = 0; e < n_evals; ++e) {
        Pert p = {};
        if (n) {
            p.key = Key{(uint32_t)perts[e].seed, (uint32_t)(perts[e].seed >> 32)};
            p.probe = perts[e].probe;
            p.sigma = perts[e].sigma;
            p.on = 1;
            p.dirs = d.dirs;
        }
        hipGraphExec_t ex = nullptr;
        if (!n && m.graphs && !timing_active())
            if (zo_status st = forward_graph(m, b, w, &ex, (const bf16_t*)m.params, 1, 0)) return st;
        if (ex) {
            if (hipGraphLaunch(ex, s) != hipSuccess) return fail(ZO_ERR_HIP, "graph launch failed");
        } else if (zo_status st = decoder_eval_launches(m, b, p, w, s, (const bf16_t*)m.params)) {
            return st;
        }
        {
            KernelTimer t("reduce", s);
            ce_final_kernel<<<1, kThreads, 0, s>>>(w.ce_part, cdiv(M, 64), M, S, loss + e);
            if (zo_status st = check_launch("ce reduce")) return st;
        }
    }
    return ZO_OK;
}

zo_status decoder_forward_groups(const ModelView& m, const zo_batch& b, const void* params, int groups,
                                 uint64_t gstride, void* ws, double* loss, hipStream_t s)
{
    const int M = (int)(b.batch * b.seq), S = (int)b.seq;
    if (groups < 1 || (groups > 1 && M % 256)) return fail(ZO_ERR_INVALID, "bad row groups");
    const DecoderWs w = carve(m.desc, ws, groups);
    hipGraphExec_t ex = nullptr;
    if (m.graphs && !timing_active())
        if (zo_status st = forward_graph(m, b, w, &ex, (const bf16_t*)params, groups, gstride)) return st;
    if (ex) {
        if (hipGraphLaunch(ex, s) != hipSuccess) return fail(ZO_ERR_HIP, "graph launch failed");
    } else if (zo_status st = decoder_eval_launches(m, b, Pert{}, w, s, (const bf16_t*)params, groups, gstride)) {
        return st;
    }
    KernelTimer t("reduce", s);
    ce_final_kernel<<<groups, kThreads, 0, s>>>(w.ce_part, cdiv(M, 64), M, S, loss);
    return check_launch("ce reduce");
}

// ------------------------------------------------------------ debug entries
zo_status debug_gemm_bf16(const void* A, const void* W, void* C, int M, int N, int K, int epi, hipStream_t s)
{
    if (!A || !W || !C || M <= 0 || N <= 0 || K <= 0) return fail(ZO_ERR_INVALID, "bad GEMM arguments");
    if (K % 64) return fail(ZO_ERR_UNSUPPORTED, "K must be a multiple of 64");
    if (N % 8) return fail(ZO_ERR_UNSUPPORTED, "N must be a multiple of 8");
    if (((uintptr_t)A | (uintptr_t)W | (uintptr_t)C) & 15) return fail(ZO_ERR_INVALID, "A, W, C must be 16-byte aligned");
    if ((int64_t)M * K * 2 >= (1ll << 31) || (int64_t)N * K * 2 >= (1ll << 31) || (int64_t)M * N * 2 >= (1ll << 31))
        return fail(ZO_ERR_UNSUPPORTED, "A, W and C must each be under 2 GiB");
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
    if ((int64_t)B * S * 3 * H * dh * 2 >= (1ll << 31)) return fail(ZO_ERR_UNSUPPORTED, "qkv must be under 2 GiB");
    if (((uintptr_t)qkv | (uintptr_t)out) & 15) return fail(ZO_ERR_INVALID, "qkv and out must be 16-byte aligned");
    KernelTimer t("attention", s);
    launch_attention((const bf16_t*)qkv, B, S, H * dh, H, dh, (bf16_t*)out, s);
    return check_launch("attention");
}

zo_status debug_layernorm(const void* h, const void* g, const void* b, void* x, int rows, int d, hipStream_t s)
{
    if (!h || !g || !b || !x || rows <= 0 || d <= 0) return fail(ZO_ERR_INVALID, "bad LayerNorm arguments");
    if (d > 64 * 4 * kLnMaxQuads || d % 4 || (d > 2048 && d % 8))
        return fail(ZO_ERR_UNSUPPORTED, "row length must be a multiple of 4 (of 8 above 2048), <= 8192");
    if (((uintptr_t)h | (uintptr_t)g | (uintptr_t)b | (uintptr_t)x) & 15)
        return fail(ZO_ERR_INVALID, "LayerNorm buffers must be 16-byte aligned");
    Pert p = {};
    KernelTimer t("layernorm", s);
    launch_layernorm((const bf16_t*)h, rows, d, (const bf16_t*)g, 0, (const bf16_t*)b, 0, p, (bf16_t*)x, s);
    return check_launch("layernorm");
}

}  // namespace zo
