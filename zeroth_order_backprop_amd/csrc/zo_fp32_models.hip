// Forward-only losses of the fp32 model families (least squares, 2-layer MLP)
// with the perturbation applied inside the GEMM: each weight tile is loaded
// from HBM, its direction values are regenerated for the tile's global element
// indices, D(fma(sigma, z, w)) is written to LDS, and the tile feeds fp32 MFMA
// (v_mfma_f32_32x32x2_f32).  The weights in memory are never modified.  One
// launch covers a whole list of evaluations (grid z = evaluation group); the
// two evaluations of a probe (+eps, -eps) share one regeneration of z.
//
// This is the forward-loss step of the SPSA loop (ZOO blog "Backprop 없이
// Transformer를 학습시킨다", section "backprop의 메모리 세금": N forwards that
// measure only the loss, no backprop), with the perturbed-tile idea of the
// same page's 1.5-SPSA section (a fused unpack/apply kernel) redone for gfx950.
//
// Loss definitions:
//   least squares: L = ||X W - Y||_F^2 / (2 n), W [d_in][d_out]
//   MLP:           L = mean_b CE(GELU(X W1^T) W2^T, y_b), no biases
// Reductions are two-stage and fixed-order (fp64 partials), so results are
// bitwise reproducible.
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

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kMaxClasses = 16;

struct EvalList {
    uint32_t n_groups;
    uint32_t perturbed;  // 0: the stored weights, no direction
    uint64_t seed[kMaxEvalsPerCall];
    uint32_t probe[kMaxEvalsPerCall];
    float sigma[kMaxEvalsPerCall][2];
    int32_t out[kMaxEvalsPerCall][2];
};

struct GemmArgs {
    const float* X;   // [M][K]
    const float* W;   // B operand: [K][N] (B_KN) or [N][K]
    uint64_t w_dir;   // direction index of W[0]
    int M, N, K;
    // least squares
    const float* Y;   // [M][N]
    double* part;     // fp64 partial per (eval, block)
    // MLP second layer
    const float* W2;  // [C][N]
    uint64_t w2_dir;
    int C;
    float* logit_part;  // [eval][n_tile][C][M] (split mode: [branch][n_tile][(1 + ps) C][M])
    int ps;             // SG_PROBE_SPLIT: theta_2 directions per branch
    uint32_t z2_probe0; // SG_PROBE_SPLIT: direction index of theta_2 direction 0
    float lr;           // SG_UPDATE: H[m][n] -= lr * acc
    const int* skip;    // SG_UPDATE: nonzero -> write nothing
};

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// GELU with the exact (erf) form.

enum { EPI_LSQ = 0, EPI_MLP = 1 };

// C[M][N] = X * B, B_KN: B = W ([K][N]);  else B = W^T (W is [N][K]).
// NT threads = NT/64 waves in a (NT/128) x 2 grid over the BM x BN block
// tile; each wave owns a WM x WN piece as 32x32 MFMA tiles, for NV weight
// variants at once.
template <int BM, int BN, int BK, bool B_KN, int NV, int EPI, int NT>
__global__ __launch_bounds__(NT) void fgemm_kernel(GemmArgs a, EvalList ev)
{
    constexpr int kThreads = NT;
    constexpr int WAVES_M = NT / 128;
    extern __shared__ __align__(16) float smem[];
    constexpr int SA = BK + 4;  // padded LDS row stride (floats)
    constexpr int WM = BM / WAVES_M, WN = BN / 2;
    constexpr int RB = WM / 32, CB = WN / 32;
    constexpr int A_VEC = BM * BK / 4;  // float4 per A tile
    constexpr int B_VEC = BN * BK / 4;  // quads per B tile
    constexpr int A_PER = (A_VEC + kThreads - 1) / kThreads;
    constexpr int B_PER = (B_VEC + kThreads - 1) / kThreads;

    const int g = blockIdx.z;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int M = a.M, N = a.N, K = a.K;
    const Key key = make_key(ev.seed[g]);
    const uint32_t probe = ev.probe[g];
    const bool pert = ev.perturbed != 0;
    float sig[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) sig[v] = ev.sigma[g][v];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, lh = lane >> 5;
    static_assert(RB >= 1 && CB >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 blocks");

    f32x16 acc[NV][RB][CB];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j) acc[v][i][j] = f32x16{};

    static_assert(A_VEC % kThreads == 0 && B_VEC % kThreads == 0, "tile quads must divide evenly over the threads");
    float4 ra[A_PER], rb[B_PER], zb[B_PER];
    // LDS stage st: A tile at smem + st * STAGE, then NV B tiles
    constexpr int STAGE = BM * SA + NV * BN * SA;
    auto As = [&](int st) { return smem + st * STAGE; };
    auto Bs = [&](int st, int v) { return smem + st * STAGE + BM * SA + v * BN * SA; };
    // B quad i: four consecutive k of one column (W [N][K]) or four consecutive
    // columns at one k (W [K][N]).  The latter are stored transposed as single
    // floats, so there k runs fastest across the lanes: consecutive lanes write
    // consecutive words of an LDS row (columns fastest put the 16 lanes of one
    // k on two banks).  Their 16-byte global loads then come from different
    // rows of W, which stays in L2.
    auto b_coords = [&](int i, int k0, int& ln, int& lk, int& gn, int& gk) {
        if (!B_KN) { ln = i / (BK / 4); lk = 4 * (i % (BK / 4)); }
        else { lk = i % BK; ln = 4 * (i / BK); }
        gn = n0 + ln;
        gk = k0 + lk;
    };
    // Branch-free tile loads: out-of-range quads read element 0 and are
    // replaced by zeros, so a whole k-step stays one basic block and the
    // scheduler can place the direction arithmetic between the MFMAs.
    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int t = 0; t < A_PER; ++t) {
            const int i = tid + t * kThreads;
            const int r = i / (BK / 4), c4 = i % (BK / 4);
            const int gm = m0 + r, gk = k0 + 4 * c4;
            const bool ok = gm < M && gk < K;
            const float4 v = *reinterpret_cast<const float4*>(a.X + (ok ? (size_t)gm * K + gk : 0));
            ra[t] = ok ? v : float4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int t = 0; t < B_PER; ++t) {
            const int i = tid + t * kThreads;
            int ln, lk, gn, gk;
            b_coords(i, k0, ln, lk, gn, gk);
            const bool ok = gn < N && gk < K;
            const size_t idx = B_KN ? (size_t)gk * N + gn : (size_t)gn * K + gk;
            const float4 v = *reinterpret_cast<const float4*>(a.W + (ok ? idx : 0));
            rb[t] = ok ? v : float4{0.f, 0.f, 0.f, 0.f};
        }
    };
    // Direction values of B quad t of the tile at k0, as three pieces (the
    // Philox block, then each Box-Muller pair) that are spread over the
    // k-step's MFMA groups.  Zero outside the matrix and for the stored weights.
    uint32_t wd[B_PER][4];
    bool zok[B_PER];
    auto z_piece = [&](int piece, int k0) {
        const int t = piece / 3, part = piece % 3;
        if (part == 0) {
            const int i = tid + t * kThreads;
            int ln, lk, gn, gk;
            b_coords(i, k0, ln, lk, gn, gk);
            zok[t] = pert & (gn < N) & (gk < K);
            const size_t idx = B_KN ? (size_t)gk * N + gn : (size_t)gn * K + gk;
            const uint64_t q = (a.w_dir + (zok[t] ? idx : 0)) >> 2;
            uint32_t c0 = (uint32_t)q, c1 = (uint32_t)(q >> 32), c2 = probe, c3 = 0u;
            philox4x32_10(c0, c1, c2, c3, key);
            wd[t][0] = c0; wd[t][1] = c1; wd[t][2] = c2; wd[t][3] = c3;
        } else {
            float z0, z1;
            box_muller(wd[t][2 * part - 2], wd[t][2 * part - 1], z0, z1);
            if (part == 1) { zb[t].x = zok[t] ? z0 : 0.f; zb[t].y = zok[t] ? z1 : 0.f; }
            else { zb[t].z = zok[t] ? z0 : 0.f; zb[t].w = zok[t] ? z1 : 0.f; }
        }
    };
    auto store_tiles = [&](int st, int k0) {
#pragma unroll
        for (int t = 0; t < A_PER; ++t) {
            const int i = tid + t * kThreads;
            const int r = i / (BK / 4), c4 = i % (BK / 4);
            *reinterpret_cast<float4*>(As(st) + r * SA + 4 * c4) = ra[t];
        }
#pragma unroll
        for (int t = 0; t < B_PER; ++t) {
            const int i = tid + t * kThreads;
            int ln, lk, gn, gk;
            b_coords(i, k0, ln, lk, gn, gk);
            const float4 z = zb[t];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float4 w = rb[t];
                w.x = fmaf(sig[v], z.x, w.x); w.y = fmaf(sig[v], z.y, w.y);
                w.z = fmaf(sig[v], z.z, w.z); w.w = fmaf(sig[v], z.w, w.w);
                // outside the matrix the tile is zero: fma(sigma, 0, 0) = 0
                float* Bv = Bs(st, v);
                if (!B_KN) {
                    *reinterpret_cast<float4*>(Bv + ln * SA + lk) = w;
                } else {
                    Bv[(ln + 0) * SA + lk] = w.x; Bv[(ln + 1) * SA + lk] = w.y;
                    Bv[(ln + 2) * SA + lk] = w.z; Bv[(ln + 3) * SA + lk] = w.w;
                }
            }
        }
    };
    // one k-substep of 8: lane (lr, lh) supplies k = kk + 4 lh + s in MFMA
    // step s; the same permutation of k on both operands leaves the sum unchanged
    auto mma_step = [&](int st, int kk) {
        f32x4 af[RB], bf[NV][CB];
#pragma unroll
        for (int i = 0; i < RB; ++i)
            af[i] = *reinterpret_cast<const f32x4*>(As(st) + (wm * WM + i * 32 + lr) * SA + kk + 4 * lh);
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int j = 0; j < CB; ++j)
                bf[v][j] = *reinterpret_cast<const f32x4*>(Bs(st, v) + (wn * WN + j * 32 + lr) * SA + kk + 4 * lh);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int i = 0; i < RB; ++i)
#pragma unroll
                    for (int j = 0; j < CB; ++j)
                        acc[v][i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][s], bf[v][j][s], acc[v][i][j],
                                                                            0, 0, 0);
    };
    constexpr int NKK = BK / 8, NPIECE = 3 * B_PER;

    load_tiles(0);
#pragma unroll
    for (int pc = 0; pc < NPIECE; ++pc) z_piece(pc, 0);
    store_tiles(0, 0);
    __syncthreads();
    int cur = 0;
    const int KT = (K + BK - 1) / BK;
    for (int kt = 0; kt + 1 < KT; ++kt) {
        const int kn = (kt + 1) * BK;
        load_tiles(kn);  // in flight during the MFMAs
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            mma_step(cur, 8 * kk);
#pragma unroll
            for (int pc = 0; pc < NPIECE; ++pc)
                if ((pc * NKK) / NPIECE == kk) z_piece(pc, kn);
        }
        store_tiles(cur ^ 1, kn);
        __syncthreads();
        cur ^= 1;
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) mma_step(cur, 8 * kk);
    // every MFMA result lands before the epilogue's branches (as in sgemm_kernel)
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j) asm volatile("" : "+a"(acc[v][i][j]));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");

    // accumulator element r of a 32x32 tile: row 8 (r/4) + 4 lh + r%4, col lr
    if constexpr (EPI == EPI_LSQ) {
        constexpr int NW = NT / 64;
        __shared__ double wsum[NV][NW];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            double s = 0.0;
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int j = 0; j < CB; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                        const int col = n0 + wn * WN + j * 32 + lr;
                        if (row < M && col < N) {
                            const double d = (double)acc[v][i][j][r] - (double)a.Y[(size_t)row * N + col];
                            s = fma(d, d, s);
                        }
                    }
            s = wave_sum(s);
            if (lane == 0) wsum[v][wave] = s;
        }
        __syncthreads();
        if (tid < NV) {
            double t = 0.0;
            for (int w = 0; w < NW; ++w) t += wsum[tid][w];
            const int blk = blockIdx.y * gridDim.x + blockIdx.x;
            a.part[(size_t)ev.out[g][tid] * gridDim.x * gridDim.y + blk] = t;
        }
    } else {
        // GELU(H tile) -> LDS, then partial logits over this tile's BN hidden
        // units against the (perturbed) W2 columns n0 .. n0+BN.
        constexpr int SH = BN + 1;
        float* Hs = smem;              // BM x SH
        float* W2s = Hs + BM * SH;     // NV x C x BN
        const int C = a.C;
        __syncthreads();
        for (int q = tid; q < C * (BN / 4); q += kThreads) {
            const int c = q / (BN / 4), n4 = 4 * (q % (BN / 4));
            const int gn = n0 + n4;
            float4 w = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
            if (gn < N) {
                const size_t idx = (size_t)c * N + gn;
                w = *reinterpret_cast<const float4*>(a.W2 + idx);
                if (pert) z = gauss4(key, probe, (a.w2_dir + idx) >> 2);
            }
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float* d = W2s + (v * C + c) * BN + n4;
                d[0] = fmaf(sig[v], z.x, w.x); d[1] = fmaf(sig[v], z.y, w.y);
                d[2] = fmaf(sig[v], z.z, w.z); d[3] = fmaf(sig[v], z.w, w.w);
            }
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int j = 0; j < CB; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = wm * WM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                        const int col = wn * WN + j * 32 + lr;
                        // columns beyond N hold GELU(0) = 0 and zero W2 weights
                        Hs[row * SH + col] = gelu_erf(acc[v][i][j][r]);
                    }
            __syncthreads();
            for (int row = tid; row < BM; row += kThreads) {
                const int gm = m0 + row;
                if (gm >= M) continue;
                // [eval][tile][class][row]
                float* dst = a.logit_part + ((size_t)ev.out[g][v] * gridDim.x + blockIdx.x) * C * M + gm;
                for (int c = 0; c < C; ++c) {
                    const float* w2 = W2s + (v * C + c) * BN;
                    float p = 0.f;
#pragma unroll 8
                    for (int n = 0; n < BN; ++n) p = fmaf(Hs[row * SH + n], w2[n], p);
                    dst[(size_t)c * M] = p;
                }
            }
            __syncthreads();
        }
    }
}

// loss[e] = (sum of the e-th eval's block partials, fixed order) / (2 M)
__global__ __launch_bounds__(kThreads) void lsq_reduce(const double* __restrict__ part, int n_blocks, int M,
                                                        double* __restrict__ loss)
{
    __shared__ double ws[4];
    const int e = blockIdx.x;
    double s = 0.0;
    for (int b = threadIdx.x; b < n_blocks; b += kThreads) s += part[(size_t)e * n_blocks + b];
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) loss[e] = (((ws[0] + ws[1]) + ws[2]) + ws[3]) / (2.0 * (double)M);
}

// Cross-entropy of each row from the logit partials ([eval][tile][class][row]).
// Block (chunk, e) covers rows 64 chunk .. +63 of evaluation e; wave w sums the hidden tiles
// t = w, w+4, ... in fp64, the four partial logits are added in fixed order,
// and the block writes the fp64 sum of its rows' losses.
__global__ __launch_bounds__(kThreads) void mlp_ce_rows(const float* __restrict__ part, int n_tiles, int M, int C,
                                                         const int32_t* __restrict__ labels,
                                                         double* __restrict__ chunk_sum)
{
    __shared__ double lg_w[4][64][kMaxClasses + 1];
    const int e = blockIdx.y, chunk = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = chunk * 64 + lane;
    double lg[kMaxClasses];
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) lg[c] = 0.0;
    if (m < M) {
        for (int t = wave; t < n_tiles; t += 4) {
            const float* p = part + ((size_t)e * n_tiles + t) * C * M + m;
            // unguarded loads (class index clamped) so they all issue at once
            float v[kMaxClasses];
#pragma unroll
            for (int c = 0; c < kMaxClasses; ++c) v[c] = p[(size_t)min(c, C - 1) * M];
#pragma unroll
            for (int c = 0; c < kMaxClasses; ++c) lg[c] += c < C ? (double)v[c] : 0.0;
        }
    }
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) lg_w[wave][lane][c] = lg[c];
    __syncthreads();
    if (wave != 0) return;
    double v = 0.0;
    if (m < M) {
        const int y = labels[m];
        double mx = -INFINITY, picked = (unsigned)y < (unsigned)C ? 0.0 : (double)NAN;  // bad label: NaN loss
#pragma unroll
        for (int c = 0; c < kMaxClasses; ++c) {
            lg[c] = ((lg_w[0][lane][c] + lg_w[1][lane][c]) + lg_w[2][lane][c]) + lg_w[3][lane][c];
            if (c < C) mx = fmax(mx, lg[c]);
        }
        double se = 0.0;
#pragma unroll
        for (int c = 0; c < kMaxClasses; ++c)
            if (c < C) {
                se += exp(lg[c] - mx);
                if (c == y) picked = lg[c];
            }
        v = (mx + log(se)) - picked;
    }
    v = wave_sum(v);
    if (lane == 0) chunk_sum[(size_t)e * gridDim.x + chunk] = v;
}

// Split perturbation: block (chunk, e2) with e2 = (2 d + v) ps + k covers rows
// 64 chunk .. +63 of branch b = 2 d + v and its theta_2 direction k.  The
// branch's partials are [tile][(1 + ps) C columns: slot * C + class][row].
// The logits at W2 +- eps z2_k are base +- eps dir, base and dir the tile
// sums of slot 0 and slot 1 + k (same fixed-order fp64 tile sums as
// mlp_ce_rows); the block writes the row-loss sums of both signs as
// evaluations 2 e2 and 2 e2 + 1.
__global__ __launch_bounds__(kThreads) void split_ce_rows(const float* __restrict__ part, int n_tiles, int M, int C,
                                                           int ps, double eps,
                                                           const int32_t* __restrict__ labels,
                                                           double* __restrict__ chunk_sum)
{
    __shared__ double lg_w[4][64][2 * kMaxClasses + 1];
    const int e2 = blockIdx.y, chunk = blockIdx.x;
    const int branch = e2 / ps, k = e2 % ps;
    const int Q = (1 + ps) * C;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = chunk * 64 + lane;
    double lb[kMaxClasses], ld[kMaxClasses];
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) lb[c] = ld[c] = 0.0;
    if (m < M) {
        for (int t = wave; t < n_tiles; t += 4) {
            const float* pb = part + ((size_t)branch * n_tiles + t) * Q * M + m;
            const float* pd = pb + (size_t)(1 + k) * C * M;
            float vb[kMaxClasses], vd[kMaxClasses];
#pragma unroll
            for (int c = 0; c < kMaxClasses; ++c) {
                vb[c] = pb[(size_t)min(c, C - 1) * M];
                vd[c] = pd[(size_t)min(c, C - 1) * M];
            }
#pragma unroll
            for (int c = 0; c < kMaxClasses; ++c) {
                lb[c] += c < C ? (double)vb[c] : 0.0;
                ld[c] += c < C ? (double)vd[c] : 0.0;
            }
        }
    }
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) {
        lg_w[wave][lane][c] = lb[c];
        lg_w[wave][lane][kMaxClasses + c] = ld[c];
    }
    __syncthreads();
    if (wave != 0) return;
    double v[2] = {0.0, 0.0};
    if (m < M) {
        const int y = labels[m];
#pragma unroll
        for (int c = 0; c < kMaxClasses; ++c) {
            lb[c] = ((lg_w[0][lane][c] + lg_w[1][lane][c]) + lg_w[2][lane][c]) + lg_w[3][lane][c];
            const int cd = kMaxClasses + c;
            ld[c] = ((lg_w[0][lane][cd] + lg_w[1][lane][cd]) + lg_w[2][lane][cd]) + lg_w[3][lane][cd];
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const double se_ = t == 0 ? eps : -eps;
            double mx = -INFINITY, picked = (unsigned)y < (unsigned)C ? 0.0 : (double)NAN;  // bad label: NaN loss
#pragma unroll
            for (int c = 0; c < kMaxClasses; ++c)
                if (c < C) mx = fmax(mx, lb[c] + se_ * ld[c]);
            double se = 0.0;
#pragma unroll
            for (int c = 0; c < kMaxClasses; ++c)
                if (c < C) {
                    const double l = lb[c] + se_ * ld[c];
                    se += exp(l - mx);
                    if (c == y) picked = l;
                }
            v[t] = (mx + log(se)) - picked;
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const double w = wave_sum(v[t]);
        if (lane == 0) chunk_sum[(size_t)(2 * e2 + t) * gridDim.x + chunk] = w;
    }
}

// g2[m] = (L[2m] - L[2m+1]) / (2 eps) for m < 2 p1 ps; g1[d] = (mean of branch
// (d, +)'s 2 ps losses - mean of branch (d, -)'s) / (2 eps) for d < p1.
__global__ void split_g_kernel(const double* __restrict__ L, int p1, int ps, double eps, double* __restrict__ g1,
                               double* __restrict__ g2)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int p2 = 2 * p1 * ps;
    if (t < p2) {
        g2[t] = (L[2 * t] - L[2 * t + 1]) / (2.0 * eps);
    } else if (t < p2 + p1) {
        const int d = t - p2;
        double sp = 0.0, sm = 0.0;
        for (int j = 0; j < 2 * ps; ++j) {
            sp += L[(size_t)(2 * d) * 2 * ps + j];
            sm += L[(size_t)(2 * d + 1) * 2 * ps + j];
        }
        g1[d] = (sp / (2 * ps) - sm / (2 * ps)) / (2.0 * eps);
    }
}

// loss[e] = (sum of evaluation e's chunk sums, fixed order) / M
__global__ __launch_bounds__(64) void mlp_ce_final(const double* __restrict__ chunk_sum, int n_chunks, int M,
                                                   double* __restrict__ loss)
{
    const int e = blockIdx.x;
    double s = 0.0;
    for (int i = threadIdx.x; i < n_chunks; i += 64) s += chunk_sum[(size_t)e * n_chunks + i];
    s = wave_sum(s);
    if (threadIdx.x == 0) loss[e] = s / (double)M;
}

// ---------------------------------------------------------------- host side
// LSQ tiles: C[512 x 256] per eval in 128 x 64 tiles.  MLP: all 256 rows per
// block so each W1 element's direction value is regenerated once per probe.
// ============================================================ split-bf16 MLP GEMMs
// fp32 products on the bf16 matrix cores.  Each fp32 operand value is split
// exactly into three bf16 parts, x = x0 + x1 + x2 (8 + 8 + 8 significand
// bits), and x w is taken as x0w0 + x0w1 + x1w0 + x0w2 + x1w1 + x2w0: the
// three dropped products weigh at most 2^-24 relative to x0w0, bf16 products
// are exact in fp32 and the MFMA accumulates in fp32, so the result carries
// the error of an fp32 dot product.  On this chip fp32 MFMAs do not overlap
// VALU work while bf16 MFMAs do, and the six bf16 products of a 16-deep k
// step cost 12 cycles per k against 32 for fp32 MFMAs.
//
// The first layer is linear in W1, so for a perturbation sigma z,
// X (W1 + sigma Z)^T = X W1^T + sigma X Z^T: the stored-weight product is
// formed once per call and each evaluation group (one direction, NV signs)
// needs one product with its direction tile, generated into LDS in the main
// loop, instead of NV products with perturbed weights.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t bf16_t;

__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// q = p0 + p1 + p2 exactly (per element), bf16 pairs packed (low, high)
__device__ __forceinline__ void split4(float4 q, uint2 (&p)[3])
{
    uint32_t a = bf16x2_rne(q.x, q.y), b = bf16x2_rne(q.z, q.w);
    p[0] = uint2{a, b};
    float r0 = q.x - bf16_lo(a), r1 = q.y - bf16_hi(a), r2 = q.z - bf16_lo(b), r3 = q.w - bf16_hi(b);
    a = bf16x2_rne(r0, r1);
    b = bf16x2_rne(r2, r3);
    p[1] = uint2{a, b};
    r0 -= bf16_lo(a); r1 -= bf16_hi(a); r2 -= bf16_lo(b); r3 -= bf16_hi(b);
    p[2] = uint2{bf16x2_rne(r0, r1), bf16x2_rne(r2, r3)};
}

// x [n4 quads] -> three bf16 planes, plane k at planes + k * plane_stride
__global__ __launch_bounds__(kThreads) void split_planes_kernel(const float* __restrict__ x, size_t n4,
                                                                bf16_t* __restrict__ planes, size_t plane_stride)
{
    for (size_t q = (size_t)blockIdx.x * kThreads + threadIdx.x; q < n4; q += (size_t)gridDim.x * kThreads) {
        uint2 p[3];
        split4(reinterpret_cast<const float4*>(x)[q], p);
#pragma unroll
        for (int k = 0; k < 3; ++k) reinterpret_cast<uint2*>(planes + k * plane_stride)[q] = p[k];
    }
}

enum { SG_BASE_STORE = 0, SG_BASE_MLP = 1, SG_PROBE_MLP = 2, SG_PROBE_SPLIT = 3, SG_UPDATE = 4 };
constexpr int kSplitMaxPs = 4;  // theta_2 directions per branch in one split-perturbation launch

struct SplitArgs {
    const bf16_t* Xp;   // [3][M][K] bf16 planes of X
    const float* W;     // [N][K] first-layer weights (base modes)
    uint64_t w_dir;     // direction index of W[0][0]
    int M, N, K;
    float* H;           // [M][N] X W^T: written by SG_BASE_STORE, read by SG_PROBE_MLP
    const float* W2;    // [C][N]
    uint64_t w2_dir;
    int C;
    float* logit_part;  // [eval][n_tile][C][M] (split mode: [branch][n_tile][(1 + ps) C][M])
    int ps;             // SG_PROBE_SPLIT: theta_2 directions per branch
    uint32_t z2_probe0; // SG_PROBE_SPLIT: direction index of theta_2 direction 0
    float lr;           // SG_UPDATE: H[m][n] -= lr * acc
    const int* skip;    // SG_UPDATE: nonzero -> write nothing
};

// vmcnt(0) with expcnt / lgkmcnt left at their maxima (gfx9 encoding)
#define ZO_WAIT_VM0() __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8))

// C = X B^T over one BM x BN tile with K % 32 == 0: B = W (base modes) or the
// direction tile Z of group blockIdx.z (probe mode).  NT/64 waves in a
// (NT/128) x 2 grid, each owning (BM/(NT/128)) x (BN/2) as 32x32 MFMA blocks.
// LDS stage: the three X planes (BM rows of 32 bf16, written by direct-to-LDS
// loads) then the three B planes (BN rows, written from registers after the
// split); rows are 64 B with chunk c of row r at c ^ ((r >> 2) & 3).  One
// barrier per k step: the next stage is filled while the current one feeds
// the MFMAs.
//   SG_BASE_STORE: H = acc.
//   SG_BASE_MLP:   stored weights, logits of GELU(acc) against W2.
//   SG_PROBE_MLP:  for each sign v, logits of GELU(H + sigma_v acc) against
//                  W2 + sigma_v z2 (z2 the same direction's W2 part).
//   SG_PROBE_SPLIT: for each sign v of the theta_1 direction, the block-1
//                  output A = GELU(H + sigma_v acc) is reused: partial logits
//                  of A against W2 (slot 0) and against each of the branch's
//                  ps theta_2 directions (slot 1 + k), so that the logits at
//                  W2 +- eps z2_k are slot 0 +- eps slot (1 + k).
template <int BM, int BN, int NT, int MODE, int NV, int QT = 0>
__global__ __launch_bounds__(NT) void sgemm_kernel(SplitArgs a, EvalList ev)
{
    constexpr bool PROBE = MODE == SG_PROBE_MLP || MODE == SG_PROBE_SPLIT;
    constexpr int BK = 32;
    constexpr int WAVES_M = NT / 128, WM = BM / WAVES_M, WN = BN / 2;
    constexpr int RB = WM / 32, CB = WN / 32;
    constexpr int PA = BM * BK, PB = BN * BK;          // bf16 per plane
    constexpr int STAGE = 3 * (PA + PB);
    constexpr int A_INS = 3 * PA / 8 / NT;             // 16-byte loads per thread per stage
    constexpr int B_Q = PB / 4 / NT;                   // B quads per thread per stage
    static_assert(A_INS * NT * 8 == 3 * PA && B_Q * NT * 4 == PB, "tile / thread mismatch");
    static_assert(RB >= 1 && CB >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 blocks");
    extern __shared__ __align__(16) bf16_t lds_bf[];

    const int M = a.M, N = a.N, K = a.K;
    const int tn = blockIdx.x, m0 = blockIdx.y * BM, n0 = tn * BN;
    const int g = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, lh = lane >> 5;
    const Key key = make_key(ev.seed[g]);
    const uint32_t probe = ev.probe[g];

    f32x16 acc[RB][CB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) acc[i][j] = f32x16{};

    // ---- X planes: direct-to-LDS, rows past M clamped (never stored)
    auto issue_a = [&](int st, int k0) {
        bf16_t* base = lds_bf + st * STAGE;
#pragma unroll
        for (int j = 0; j < A_INS; ++j) {
            const int p = j * NT + tid;
            const int plane = p / (BM * 4), rem = p % (BM * 4), row = rem >> 2;
            const int lc = (rem & 3) ^ ((row >> 2) & 3);
            const bf16_t* src = a.Xp + (size_t)plane * M * K + (size_t)min(m0 + row, M - 1) * K + k0 + 8 * lc;
            bf16_t* dst = base + (j * NT + wave * 64) * 8;  // wave-uniform: lane l lands at +16 l bytes
            __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
    };
    // ---- B quads: t-th quad of this thread is row ln = i / 8, k = 4 (i % 8)
    float4 bq[B_Q];
    uint32_t wd[B_Q][4];
    auto b_row = [&](int t) { return (t * NT + tid) >> 3; };
    auto b_k = [&](int t) { return 4 * ((t * NT + tid) & 7); };
    auto load_b = [&](int k0) {  // base modes: W quads (zero past N)
#pragma unroll
        for (int t = 0; t < B_Q; ++t) {
            const int gn = n0 + b_row(t);
            const bool ok = gn < N;
            const float4 v = *reinterpret_cast<const float4*>(a.W + (ok ? (size_t)gn * K + k0 + b_k(t) : 0));
            bq[t] = ok ? v : float4{0.f, 0.f, 0.f, 0.f};
        }
    };
    // probe mode: direction quads in three pieces (Philox block, then each
    // Box-Muller pair) so the VALU work spreads between the MFMAs
    auto z_piece = [&](int piece, int k0) {
        const int t = piece / 3, part = piece % 3;
        const int gn = n0 + b_row(t);
        if (part == 0) {
            const uint64_t q = (a.w_dir + (size_t)min(gn, N - 1) * K + k0 + b_k(t)) >> 2;
            uint32_t c0 = (uint32_t)q, c1 = (uint32_t)(q >> 32), c2 = probe, c3 = 0u;
            philox4x32_10(c0, c1, c2, c3, key);
            wd[t][0] = c0; wd[t][1] = c1; wd[t][2] = c2; wd[t][3] = c3;
        } else {
            float z0, z1;
            box_muller(wd[t][2 * part - 2], wd[t][2 * part - 1], z0, z1);
            const bool ok = gn < N;
            if (part == 1) { bq[t].x = ok ? z0 : 0.f; bq[t].y = ok ? z1 : 0.f; }
            else { bq[t].z = ok ? z0 : 0.f; bq[t].w = ok ? z1 : 0.f; }
        }
    };
    auto store_b = [&](int st) {
        bf16_t* base = lds_bf + st * STAGE + 3 * PA;
#pragma unroll
        for (int t = 0; t < B_Q; ++t) {
            uint2 p[3];
            split4(bq[t], p);
            const int row = b_row(t), k = b_k(t);
            const int off = row * BK + ((((k >> 3) ^ ((row >> 2) & 3))) << 3) + (k & 4);
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) *reinterpret_cast<uint2*>(base + pl * PB + off) = p[pl];
        }
    };
    // ---- 16-deep k steps: fragments in two register sets (one per k half of
    // the stage), six bf16 products per 32x32 block, smallest first
    bf16x8 fa[2][RB][3], fb[2][CB][3];
    auto read_a = [&](int st, int ks, int set) {
        const bf16_t* base = lds_bf + st * STAGE;
        const int lc = 2 * ks + lh;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int row = wm * WM + i * 32 + lr;
            const int off = row * BK + ((lc ^ ((row >> 2) & 3)) << 3);
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) fa[set][i][pl] = *reinterpret_cast<const bf16x8*>(base + pl * PA + off);
        }
    };
    auto read_b = [&](int st, int ks, int set) {
        const bf16_t* base = lds_bf + st * STAGE;
        const int lc = 2 * ks + lh;
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            const int row = wn * WN + j * 32 + lr;
            const int off = row * BK + ((lc ^ ((row >> 2) & 3)) << 3);
#pragma unroll
            for (int pl = 0; pl < 3; ++pl)
                fb[set][j][pl] = *reinterpret_cast<const bf16x8*>(base + 3 * PA + pl * PB + off);
        }
    };
    auto mma_row = [&](int set, int i) {
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            const bf16x8* af = fa[set][i];
            const bf16x8* bfr = fb[set][j];
            f32x16 c = acc[i][j];
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[2], bfr[0], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1], bfr[1], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], bfr[2], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1], bfr[0], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], bfr[1], c, 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], bfr[0], c, 0, 0, 0);
        }
    };
    // The first k half's rows of blocks.  The second half's fragments are read
    // right behind the first row's MFMAs, so those reads land while the other
    // rows compute and the second half's single wait rarely stalls (the
    // scheduling barriers keep the compiler from moving the reads back down).
    auto first_half = [&](int st) {
        read_a(st, 0, 0);
        read_b(st, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            mma_row(0, i);
            __builtin_amdgcn_sched_barrier(0);
            if (i == 0) { read_a(st, 1, 1); read_b(st, 1, 1); }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto second_half = [&]() {
#pragma unroll
        for (int i = 0; i < RB; ++i) mma_row(1, i);
    };
    constexpr int NPIECE = 3 * B_Q;
    auto produce_b = [&](int k0) {
        if constexpr (PROBE) {
#pragma unroll
            for (int pc = 0; pc < NPIECE; ++pc) z_piece(pc, k0);
        } else {
            load_b(k0);
        }
    };

    const int KT = K / BK;
    issue_a(0, 0);
    produce_b(0);
    store_b(0);
    ZO_WAIT_VM0();
    __syncthreads();
    int cur = 0;
    for (int kt = 0; kt + 1 < KT; ++kt) {
        const int kn = (kt + 1) * BK;
        issue_a(cur ^ 1, kn);
        if constexpr (!PROBE) load_b(kn);
        first_half(cur);
        if constexpr (PROBE) {
#pragma unroll
            for (int pc = 0; pc < NPIECE / 2; ++pc) z_piece(pc, kn);
        }
        second_half();
        if constexpr (PROBE) {
#pragma unroll
            for (int pc = NPIECE / 2; pc < NPIECE; ++pc) z_piece(pc, kn);
        }
        store_b(cur ^ 1);
        ZO_WAIT_VM0();
        __syncthreads();
        cur ^= 1;
    }
    first_half(cur);
    second_half();
    // The epilogue can reach its first accumulator read through a branch that
    // skips a whole wave's share of the W2 tile loads, and the compiler's
    // wait-state count for the last MFMAs' results has been seen to miss that
    // path (a stale last accumulator register in the waves that skip).  The
    // empty statements name every accumulator, so they follow the last MFMA of
    // each block; the wait states after them let every result land first.
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) asm volatile("" : "+a"(acc[i][j]));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");

    // accumulator element r of a 32x32 block: row 8 (r/4) + 4 lh + r%4, col lr
    if constexpr (MODE == SG_BASE_STORE) {
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                    const int col = n0 + wn * WN + j * 32 + lr;
                    if (row < M && col < N) a.H[(size_t)row * N + col] = acc[i][j][r];
                }
    } else if constexpr (MODE == SG_UPDATE) {
        // H[m][n] <- fp32(H[m][n] - lr acc): a weight update from its gradient estimate
        if (*a.skip) return;
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                    const int col = n0 + wn * WN + j * 32 + lr;
                    if (row < M && col < N) {
                        float* w = a.H + (size_t)row * N + col;
                        *w = fmaf(-a.lr, acc[i][j][r], *w);
                    }
                }
    } else if constexpr (MODE == SG_PROBE_SPLIT) {
        // Columns q = slot * C + c of the (1 + ps) C partial logits (slot 0:
        // W2, slot 1 + k: theta_2 direction k) are split between the two
        // thread groups, QT per group; their weights sit in LDS as rows of BN,
        // zero past (1 + ps) C, so the dot-product loop has no guards.
        static_assert(NV == 2 && QT > 0, "both signs of the theta_1 direction");
        constexpr int SH = BN + 4;
        constexpr int GROUPS = NT / BM;
        static_assert(GROUPS == 2, "two thread groups per row");
        float* Hs = reinterpret_cast<float*>(lds_bf);    // BM x SH
        float* Wz = Hs + BM * SH;                       // 2 QT rows of BN
        const int C = a.C, ps = a.ps, Q = (1 + ps) * C;
        __syncthreads();  // every wave is done with the stage buffers
        // W2 rows (q < C) and the zero rows past Q, once
        for (int t = tid; t < 2 * QT * (BN / 4); t += NT) {
            const int q = t / (BN / 4), n4 = 4 * (t % (BN / 4));
            const int gn = n0 + n4;
            float4 w = {0.f, 0.f, 0.f, 0.f};
            if (q < C && gn < N) w = *reinterpret_cast<const float4*>(a.W2 + (size_t)q * N + gn);
            if (q < C || q >= Q) *reinterpret_cast<float4*>(Wz + q * BN + n4) = w;
        }
        const int row = tid % BM;
        const int grp = __builtin_amdgcn_readfirstlane(tid / BM);  // wave-uniform
        const int gm = m0 + row;
        const float* wq = Wz + grp * QT * BN;
        const int qlim = Q - grp * QT;  // this group's columns: qq < qlim
#pragma unroll 1
        for (int v = 0; v < 2; ++v) {
            const float sg = ev.sigma[g][v];
            // the stored-weight product under this thread's accumulators, read
            // per sign (L2-resident) so it holds no registers through the dot
            // products; issued before the direction rows are generated
            float hb[RB][CB][16];
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int j = 0; j < CB; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                        const int col = n0 + wn * WN + j * 32 + lr;
                        hb[i][j][r] = (row < M && col < N) ? a.H[(size_t)row * N + col] : 0.f;
                    }
            // this branch's theta_2 directions on W2's elements: rows C .. Q-1
            const uint32_t zp0 = a.z2_probe0 + (2 * probe + v) * (uint32_t)ps;
            for (int t = tid; t < ps * C * (BN / 4); t += NT) {
                const int q = C + t / (BN / 4), n4 = 4 * (t % (BN / 4));
                const int k = q / C - 1, c = q % C;
                const int gn = n0 + n4;
                float4 z = {0.f, 0.f, 0.f, 0.f};
                if (gn < N) z = gauss4(key, zp0 + k, (a.w2_dir + (size_t)c * N + gn) >> 2);
                *reinterpret_cast<float4*>(Wz + q * BN + n4) = z;
            }
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int j = 0; j < CB; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int lrow = wm * WM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                        const int lcol = wn * WN + j * 32 + lr;
                        Hs[lrow * SH + lcol] = gelu_erf(fmaf(sg, acc[i][j][r], hb[i][j][r]));
                    }
            __syncthreads();
            float p[QT];
#pragma unroll
            for (int qq = 0; qq < QT; ++qq) p[qq] = 0.f;
            const float* hrow = Hs + row * SH;
#pragma unroll 1
            for (int n = 0; n < BN; n += 4) {
                const float4 h4 = *reinterpret_cast<const float4*>(hrow + n);
#pragma unroll
                for (int qq = 0; qq < QT; ++qq) {
                    const float4 w4 = *reinterpret_cast<const float4*>(wq + qq * BN + n);
                    float t = p[qq];
                    t = fmaf(h4.x, w4.x, t); t = fmaf(h4.y, w4.y, t);
                    t = fmaf(h4.z, w4.z, t); t = fmaf(h4.w, w4.w, t);
                    p[qq] = t;
                    // at most four rows' reads in flight: keeps the registers for the accumulators
                    if (qq % 4 == 3) asm volatile("" ::: "memory");
                }
            }
            if (gm < M) {
                // branch (g, v): [tile][column q = slot * C + class][row], rows
                // contiguous so that a wave's stores (and the reduction's loads) coalesce
                float* dst = a.logit_part + (((size_t)(g * 2 + v) * gridDim.x + tn) * Q + grp * QT) * M + gm;
#pragma unroll
                for (int qq = 0; qq < QT; ++qq)
                    if (qq < qlim) dst[(size_t)qq * M] = p[qq];
            }
            __syncthreads();  // Hs and the direction rows are rewritten for the next sign
        }
    } else {
        // GELU(H tile) -> LDS, then partial logits over this tile's BN hidden
        // units against the (perturbed) W2 columns n0 .. n0+BN.  Columns past
        // N hold GELU(0) = 0 and meet zero W2 weights.  Classes are split
        // between the NT / BM thread groups of a row, QT each: group grp takes
        // classes grp QT .. grp QT + QT - 1, whose (perturbed) W2 rows sit in
        // LDS, zero past C, so the dot-product loop carries no per-class guards.
        static_assert(QT > 0, "classes per thread group");
        constexpr int SH = BN + 4;  // 16-byte rows; float4 row reads by consecutive rows are bank-even
        constexpr int GROUPS = NT / BM;
        static_assert(GROUPS * BM == NT, "whole thread groups per row");
        constexpr int QR = GROUPS * QT;                 // W2 rows in LDS per sign
        float* Hs = reinterpret_cast<float*>(lds_bf);    // BM x SH
        float* W2s = Hs + BM * SH;                      // NV x QR x BN
        const int C = a.C;
        const bool pert = MODE == SG_PROBE_MLP && ev.perturbed != 0;
        float sig[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) sig[v] = MODE == SG_PROBE_MLP ? ev.sigma[g][v] : 0.f;
        // the stored-weight product under this thread's accumulators, loaded
        // first so its latency hides behind the W2 tile generation
        float hb[RB][CB][16];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < CB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    hb[i][j][r] = 0.f;
                    if constexpr (PROBE) {
                        const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                        const int col = n0 + wn * WN + j * 32 + lr;
                        if (row < M && col < N) hb[i][j][r] = a.H[(size_t)row * N + col];
                    }
                }
        __syncthreads();  // every wave is done with the stage buffers
        for (int q = tid; q < QR * (BN / 4); q += NT) {
            const int c = q / (BN / 4), n4 = 4 * (q % (BN / 4));
            const int gn = n0 + n4;
            float4 w = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
            if (c < C && gn < N) {
                const size_t idx = (size_t)c * N + gn;
                w = *reinterpret_cast<const float4*>(a.W2 + idx);
                if (pert) z = gauss4(key, probe, (a.w2_dir + idx) >> 2);
            }
#pragma unroll
            for (int v = 0; v < NV; ++v)
                *reinterpret_cast<float4*>(W2s + (v * QR + c) * BN + n4) =
                    float4{fmaf(sig[v], z.x, w.x), fmaf(sig[v], z.y, w.y), fmaf(sig[v], z.z, w.z),
                           fmaf(sig[v], z.w, w.w)};
        }
        const int row = tid % BM;
        const int grp = __builtin_amdgcn_readfirstlane(tid / BM);  // wave-uniform
        const int gm = m0 + row;
        const int qlim = C - grp * QT;  // this group's classes: qq < qlim
#pragma unroll 1
        for (int v = 0; v < NV; ++v) {
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int j = 0; j < CB; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int lrow = wm * WM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                        const int lcol = wn * WN + j * 32 + lr;
                        const float h = MODE == SG_PROBE_MLP ? fmaf(sig[v], acc[i][j][r], hb[i][j][r]) : acc[i][j][r];
                        Hs[lrow * SH + lcol] = gelu_erf(h);
                    }
            __syncthreads();
            float p[QT];
#pragma unroll
            for (int qq = 0; qq < QT; ++qq) p[qq] = 0.f;
            const float* hrow = Hs + row * SH;
            const float* wq = W2s + (v * QR + grp * QT) * BN;
#pragma unroll 2
            for (int n = 0; n < BN; n += 4) {
                const float4 h4 = *reinterpret_cast<const float4*>(hrow + n);
#pragma unroll
                for (int qq = 0; qq < QT; ++qq) {
                    const float4 w4 = *reinterpret_cast<const float4*>(wq + qq * BN + n);
                    float t = p[qq];
                    t = fmaf(h4.x, w4.x, t); t = fmaf(h4.y, w4.y, t);
                    t = fmaf(h4.z, w4.z, t); t = fmaf(h4.w, w4.w, t);
                    p[qq] = t;
                }
            }
            if (gm < M) {
                // [eval][tile][class][row]: a wave's stores (and the reduction's loads) coalesce
                float* dst = a.logit_part + (((size_t)ev.out[g][v] * gridDim.x + tn) * C + grp * QT) * M + gm;
#pragma unroll
                for (int qq = 0; qq < QT; ++qq)
                    if (qq < qlim) dst[(size_t)qq * M] = p[qq];
            }
            __syncthreads();  // Hs is rewritten for the next sign
        }
    }
}

constexpr int LSQ_BM = 128, LSQ_BN = 64, LSQ_BK = 32;
constexpr int MLP_BM = 256, MLP_BN = 64, MLP_BK = 32;

int cdiv(int a, int b) { return (a + b - 1) / b; }

// Groups the evaluations: pairs sharing (seed, probe) -> NV = 2, else NV = 1.
int make_evals(const zo_pert* perts, int n, EvalList& ev)
{
    memset(&ev, 0, sizeof ev);
    if (n == 0) {
        ev.n_groups = 1;
        ev.perturbed = 0;
        ev.out[0][0] = 0;
        return 1;
    }
    ev.perturbed = 1;
    bool paired = n % 2 == 0;
    for (int i = 0; paired && i < n; i += 2)
        paired = perts[i].seed == perts[i + 1].seed && perts[i].probe == perts[i + 1].probe;
    const int nv = paired ? 2 : 1;
    ev.n_groups = n / nv;
    for (int gi = 0; gi < (int)ev.n_groups; ++gi) {
        ev.seed[gi] = perts[gi * nv].seed;
        ev.probe[gi] = perts[gi * nv].probe;
        for (int v = 0; v < nv; ++v) {
            ev.sigma[gi][v] = perts[gi * nv + v].sigma;
            ev.out[gi][v] = gi * nv + v;
        }
    }
    return nv;
}

template <int BM, int BN, int BK, bool B_KN, int NV, int EPI, int NT>
zo_status launch_fgemm(const GemmArgs& a, const EvalList& ev, hipStream_t s)
{
    constexpr int SA = BK + 4;
    size_t lds = (size_t)2 * (BM * SA + NV * BN * SA) * sizeof(float);
    if (EPI == EPI_MLP) {
        const size_t epi = (size_t)(BM * (BN + 1) + NV * a.C * BN) * sizeof(float);
        lds = lds > epi ? lds : epi;
    }
    auto kern = fgemm_kernel<BM, BN, BK, B_KN, NV, EPI, NT>;
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return fail(ZO_ERR_HIP, "cannot reserve %zu bytes of LDS", lds);
        attr_set = true;
    }
    dim3 grid(cdiv(a.N, BN), cdiv(a.M, BM), ev.n_groups);
    KernelTimer timer(ev.perturbed ? "gemm_f32" : "gemm_f32_base", s);
    kern<<<grid, NT, lds, s>>>(a, ev);
    return check_launch("fp32 fused GEMM");
}

// Split-bf16 MLP GEMM tiles: probe groups 256 x 128 (8 waves), the stored-
// weight product 64 x 64 (4 waves) so that one call still spreads over the CUs.
constexpr int SP_BM = 256, SP_BN = 128, SP_NT = 512;
constexpr int SB_BM = 64, SB_BN = 64, SB_NT = 256;

template <int BM, int BN, int NT, int MODE, int NV, int QT = 0>
zo_status launch_sgemm(const SplitArgs& a, const EvalList& ev, int groups, hipStream_t s, const char* fam)
{
    constexpr size_t kLdsMax = 160 * 1024;
    constexpr size_t stages = (size_t)2 * 3 * (BM + BN) * 32 * sizeof(bf16_t);
    constexpr size_t epi = MODE == SG_BASE_STORE || MODE == SG_PROBE_SPLIT || MODE == SG_UPDATE
                               ? 0
                               : (size_t)(BM * (BN + 4) + NV * (NT / BM) * QT * BN) * sizeof(float);
    constexpr size_t lds_fixed = stages > epi ? stages : epi;
    static_assert(lds_fixed <= kLdsMax, "LDS budget");
    size_t lds = lds_fixed;
    if constexpr (MODE == SG_PROBE_SPLIT) {
        // GELU tile plus 2 QT weight rows of BN
        const size_t e = (size_t)(BM * (BN + 4) + 2 * QT * BN) * sizeof(float);
        if (e > kLdsMax || (1 + a.ps) * a.C > 2 * QT)
            return fail(ZO_ERR_UNSUPPORTED, "split perturbation: (1 + ps) * classes too large");
        lds = e > lds ? e : lds;
    }
    auto kern = sgemm_kernel<BM, BN, NT, MODE, NV, QT>;
    static bool attr_set = false;
    if (!attr_set) {
        const size_t cap = MODE == SG_PROBE_SPLIT ? kLdsMax : lds_fixed;
        if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)cap) != hipSuccess)
            return fail(ZO_ERR_HIP, "cannot reserve %zu bytes of LDS", cap);
        attr_set = true;
    }
    dim3 grid(cdiv(a.N, BN), cdiv(a.M, BM), groups);
    KernelTimer timer(fam, s);
    kern<<<grid, NT, lds, s>>>(a, ev);
    return check_launch("split-bf16 MLP GEMM");
}

// ================================================================== Dust
// Activation-noise estimator on the MLP (per-token rewards, outer-product
// weight estimates); the steps and their order are those of mlp_dust_step.

// Hidden layer: block (tile tn of DH_BN hidden units, rows m0 .., draw d).
// Draw 0 is the clean forward; draw d >= 1 adds sigma a^(d-1) (noise stream 2,
// element row * N + h) to Y = X W1^T before the GELU.  The tile's partial
// logits against W2 go to part[d][tn][class][row], as in the MLP epilogue:
// QT classes per thread group, W2 rows in LDS zero past C.
constexpr int DH_BM = 64, DH_BN = 128, DH_NT = 256;
template <int QT>
__global__ __launch_bounds__(DH_NT) void dust_hidden_kernel(const float* __restrict__ Y, const float* __restrict__ W2,
                                                            int M, int N, int C, Key key, float sigma,
                                                            float* __restrict__ part)
{
    constexpr int BM = DH_BM, BN = DH_BN, NT = DH_NT, SH = BN + 4;
    constexpr int GROUPS = NT / BM, QR = GROUPS * QT;
    __shared__ __align__(16) float Hs[BM * SH];
    __shared__ __align__(16) float W2s[QR * BN];
    const int tn = blockIdx.x, m0 = blockIdx.y * BM, d = blockIdx.z;
    const int n0 = tn * BN, tid = threadIdx.x;
    for (int q = tid; q < QR * (BN / 4); q += NT) {
        const int c = q / (BN / 4), n4 = 4 * (q % (BN / 4));
        const int gn = n0 + n4;
        float4 w = {0.f, 0.f, 0.f, 0.f};
        if (c < C && gn < N) w = *reinterpret_cast<const float4*>(W2 + (size_t)c * N + gn);
        *reinterpret_cast<float4*>(W2s + c * BN + n4) = w;
    }
    const float sg = d == 0 ? 0.f : sigma;
    for (int q = tid; q < BM * (BN / 4); q += NT) {
        const int r = q / (BN / 4), n4 = 4 * (q % (BN / 4));
        const int gm = m0 + r, gn = n0 + n4;
        float4 h = {0.f, 0.f, 0.f, 0.f};
        if (gm < M && gn < N) {
            const size_t e = (size_t)gm * N + gn;
            const float4 y = *reinterpret_cast<const float4*>(Y + e);
            const float4 z = d > 0 ? gauss4s(key, (uint32_t)(d - 1), 2u, e >> 2) : float4{0.f, 0.f, 0.f, 0.f};
            h = float4{gelu_erf(fmaf(sg, z.x, y.x)), gelu_erf(fmaf(sg, z.y, y.y)), gelu_erf(fmaf(sg, z.z, y.z)),
                       gelu_erf(fmaf(sg, z.w, y.w))};
        }
        *reinterpret_cast<float4*>(Hs + r * SH + n4) = h;
    }
    __syncthreads();
    const int row = tid % BM;
    const int grp = __builtin_amdgcn_readfirstlane(tid / BM);
    const int gm = m0 + row;
    const int qlim = C - grp * QT;
    float p[QT];
#pragma unroll
    for (int qq = 0; qq < QT; ++qq) p[qq] = 0.f;
    const float* hrow = Hs + row * SH;
    const float* wq = W2s + grp * QT * BN;
#pragma unroll 2
    for (int n = 0; n < BN; n += 4) {
        const float4 h4 = *reinterpret_cast<const float4*>(hrow + n);
#pragma unroll
        for (int qq = 0; qq < QT; ++qq) {
            const float4 w4 = *reinterpret_cast<const float4*>(wq + qq * BN + n);
            float t = p[qq];
            t = fmaf(h4.x, w4.x, t); t = fmaf(h4.y, w4.y, t);
            t = fmaf(h4.z, w4.z, t); t = fmaf(h4.w, w4.w, t);
            p[qq] = t;
        }
    }
    if (gm < M) {
        float* dst = part + (((size_t)d * gridDim.x + tn) * C + grp * QT) * M + gm;
#pragma unroll
        for (int qq = 0; qq < QT; ++qq)
            if (qq < qlim) dst[(size_t)qq * M] = p[qq];
    }
}

// Per-token cross-entropy of every draw from the partials (fixed-order fp64
// tile sums as in mlp_ce_rows): loss[d][row]; draw 0's logits (the clean
// ones) also go to Z[row][class].  Block (0, 0) clears the skip flag.
__global__ __launch_bounds__(kThreads) void dust_rows_kernel(const float* __restrict__ part, int n_tiles, int M, int C,
                                                              const int32_t* __restrict__ labels,
                                                              double* __restrict__ loss, double* __restrict__ Z,
                                                              int* __restrict__ skip)
{
    __shared__ double lg_w[4][64][kMaxClasses + 1];
    const int e = blockIdx.y, chunk = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = chunk * 64 + lane;
    if (e == 0 && chunk == 0 && threadIdx.x == 0) *skip = 0;
    double lg[kMaxClasses];
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) lg[c] = 0.0;
    if (m < M) {
        for (int t = wave; t < n_tiles; t += 4) {
            const float* p = part + ((size_t)e * n_tiles + t) * C * M + m;
            float v[kMaxClasses];
#pragma unroll
            for (int c = 0; c < kMaxClasses; ++c) v[c] = p[(size_t)min(c, C - 1) * M];
#pragma unroll
            for (int c = 0; c < kMaxClasses; ++c) lg[c] += c < C ? (double)v[c] : 0.0;
        }
    }
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) lg_w[wave][lane][c] = lg[c];
    __syncthreads();
    if (wave != 0 || m >= M) return;
    const int y = labels[m];
    double mx = -INFINITY, picked = (unsigned)y < (unsigned)C ? 0.0 : (double)NAN;  // bad label: NaN loss
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) {
        lg[c] = ((lg_w[0][lane][c] + lg_w[1][lane][c]) + lg_w[2][lane][c]) + lg_w[3][lane][c];
        if (c < C) mx = fmax(mx, lg[c]);
    }
    double se = 0.0;
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c)
        if (c < C) {
            se += exp(lg[c] - mx);
            if (c == y) picked = lg[c];
            if (e == 0) Z[(size_t)m * C + c] = lg[c];
        }
    loss[(size_t)e * M + m] = (mx + log(se)) - picked;
}

// The k2 head draws on the cached clean logits: thread per (draw i, token t),
// loss2[i][t] = CE(Z_t + sigma2 b_i[t]), b from noise stream 3 (element
// t * C + c).  A non-finite loss sets the skip flag.
__device__ __forceinline__ void logit_draw(Key key, uint32_t i, int t, int C, float* b)
{
    const uint64_t j0 = (uint64_t)t * C;
    const uint64_t q0 = j0 >> 2, q1 = (j0 + C - 1) >> 2;
    for (uint64_t q = q0; q <= q1; ++q) {
        const float4 z = gauss4s(key, i, 3u, q);
        const float zz[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int64_t c = (int64_t)(4 * q + s) - (int64_t)j0;
            if (c >= 0 && c < C) b[c] = zz[s];
        }
    }
}

__global__ __launch_bounds__(kThreads) void dust_head_loss_kernel(const double* __restrict__ Z,
                                                                   const int32_t* __restrict__ labels, int M, int C,
                                                                   int k2, float sigma2, Key key,
                                                                   double* __restrict__ loss2, int* __restrict__ skip)
{
    const size_t n = (size_t)k2 * M;
    for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < n; idx += (size_t)gridDim.x * kThreads) {
        const int i = (int)(idx / M), t = (int)(idx % M);
        float b[kMaxClasses];
        logit_draw(key, (uint32_t)i, t, C, b);
        const int y = labels[t];
        double l[kMaxClasses], mx = -INFINITY, se = 0.0;
        double picked = (unsigned)y < (unsigned)C ? 0.0 : (double)NAN;  // bad label: NaN loss
        for (int c = 0; c < C; ++c) {
            l[c] = Z[(size_t)t * C + c] + (double)sigma2 * (double)b[c];
            mx = fmax(mx, l[c]);
        }
        for (int c = 0; c < C; ++c) {
            se += exp(l[c] - mx);
            if (c == y) picked = l[c];
        }
        const double v = (mx + log(se)) - picked;
        loss2[(size_t)i * M + t] = v;
        if (!isfinite(v)) atomicOr(skip, 1);
    }
}

// Sum over the block's threads in a fixed order (LDS tree), result to all.
__device__ __forceinline__ double block_sum(double v, double* red)
{
    red[threadIdx.x] = v;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    const double r = red[0];
    __syncthreads();
    return r;
}

// Block per token t.  Hidden layer: w[i][t] = (l_i - lbar) / (k1 sigma1), the
// weight of draw i's noise in the token's output error (reward r = lbar - l_i,
// ghat = -(1 / (k1 sigma1)) sum_i r a).  Head: ghat2[t][c] = -(1 / (k2 sigma2))
// sum_i (l2bar - l2_i) b_i[c], the noise regenerated; draws split over the
// threads, sums in a fixed order.
__global__ __launch_bounds__(kThreads) void dust_reward_kernel(const double* __restrict__ loss,
                                                                const double* __restrict__ loss2, int M, int C, int k1,
                                                                int k2, float sigma1, float sigma2, Key key,
                                                                float* __restrict__ w, float* __restrict__ ghat2,
                                                                int* __restrict__ skip)
{
    __shared__ double red[kThreads];
    const int t = blockIdx.x, tid = threadIdx.x;
    double s = 0.0;
    bool bad = false;
    for (int i = tid; i < k1; i += kThreads) {
        const double v = loss[(size_t)(1 + i) * M + t];
        s += v;
        bad |= !isfinite(v);
    }
    const double lbar = block_sum(s, red) / k1;
    const double s1 = (double)k1 * (double)sigma1;
    for (int i = tid; i < k1; i += kThreads) w[(size_t)i * M + t] = (float)((loss[(size_t)(1 + i) * M + t] - lbar) / s1);
    s = 0.0;
    for (int i = tid; i < k2; i += kThreads) s += loss2[(size_t)i * M + t];
    const double l2bar = block_sum(s, red) / k2;
    double g[kMaxClasses];
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) g[c] = 0.0;
    for (int i = tid; i < k2; i += kThreads) {
        float b[kMaxClasses];
        logit_draw(key, (uint32_t)i, t, C, b);
        const double r = l2bar - loss2[(size_t)i * M + t];
        for (int c = 0; c < C; ++c) g[c] += r * (double)b[c];
    }
    const double s2 = (double)k2 * (double)sigma2;
    for (int c = 0; c < C; ++c) {
        const double gc = block_sum(g[c], red);
        if (tid == 0) ghat2[(size_t)t * C + c] = (float)(-gc / s2);
    }
    if (bad && tid == 0) atomicOr(skip, 1);
}

// The hidden layer's output errors G[t][h] = sum_i w[i][t] a_i[t][h] (noise
// regenerated), written transposed as the three bf16 planes of the update
// GEMM's A operand: planes[p][h][t], G^T = p0 + p1 + p2 exactly.  Block: 64
// tokens x 64 hidden units, staged through LDS for the transpose.
constexpr int DG_T = 64, DG_H = 64, DG_MAXK = 128;
__global__ __launch_bounds__(kThreads) void dust_gy_kernel(const float* __restrict__ w, int M, int N, int k1, Key key,
                                                            bf16_t* __restrict__ planes)
{
    __shared__ float wt[DG_MAXK][DG_T];
    __shared__ float Gs[DG_H][DG_T + 4];
    const int t0 = blockIdx.y * DG_T, h0 = blockIdx.x * DG_H, tid = threadIdx.x;
    for (int q = tid; q < k1 * DG_T; q += kThreads) {
        const int i = q / DG_T, tt = q % DG_T;
        wt[i][tt] = t0 + tt < M ? w[(size_t)i * M + t0 + tt] : 0.f;
    }
    __syncthreads();
    // tokens run fastest across the lanes: the four column writes of a lane
    // go to consecutive words of four Gs rows (hidden units fastest would put
    // the 16 lanes of one token on two banks)
    for (int q = tid; q < DG_T * (DG_H / 4); q += kThreads) {
        const int tt = q % DG_T, hq = 4 * (q / DG_T);
        const int t = t0 + tt, h = h0 + hq;
        float4 acc = {0.f, 0.f, 0.f, 0.f};
        if (t < M && h < N) {
            const uint64_t qd = ((uint64_t)t * N + h) >> 2;
            for (int i = 0; i < k1; ++i) {
                const float c = wt[i][tt];
                const float4 a = gauss4s(key, (uint32_t)i, 2u, qd);
                acc.x = fmaf(c, a.x, acc.x); acc.y = fmaf(c, a.y, acc.y);
                acc.z = fmaf(c, a.z, acc.z); acc.w = fmaf(c, a.w, acc.w);
            }
        }
        Gs[hq][tt] = acc.x; Gs[hq + 1][tt] = acc.y; Gs[hq + 2][tt] = acc.z; Gs[hq + 3][tt] = acc.w;
    }
    __syncthreads();
    for (int q = tid; q < DG_H * (DG_T / 4); q += kThreads) {
        const int hh = q / (DG_T / 4), tq = 4 * (q % (DG_T / 4));
        const int h = h0 + hh, t = t0 + tq;
        if (h >= N || t >= M) continue;
        uint2 pp[3];
        split4(*reinterpret_cast<const float4*>(&Gs[hh][tq]), pp);
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
            *reinterpret_cast<uint2*>(planes + (size_t)pl * N * M + (size_t)h * M + t) = pp[pl];
    }
}

// out[c][r] = in[r][c] (fp32), 32 x 32 tiles through LDS.
__global__ __launch_bounds__(kThreads) void transpose_kernel(const float* __restrict__ in, int R, int C,
                                                              float* __restrict__ out)
{
    __shared__ float tile[32][33];
    const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
    for (int q = threadIdx.x; q < 32 * 32; q += kThreads) {
        const int rr = q / 32, cc = q % 32;
        if (r0 + rr < R && c0 + cc < C) tile[rr][cc] = in[(size_t)(r0 + rr) * C + c0 + cc];
    }
    __syncthreads();
    for (int q = threadIdx.x; q < 32 * 32; q += kThreads) {
        const int cc = q / 32, rr = q % 32;
        if (r0 + rr < R && c0 + cc < C) out[(size_t)(c0 + cc) * R + r0 + rr] = tile[rr][cc];
    }
}

// Head update: W2[c][h] <- fp32(W2[c][h] - lr sum_t ghat2[t][c] GELU(Y[t][h])).
// Block: DW_H hidden units x DW_G token groups (group g takes tokens t with
// t % DW_G == g); the groups' sums are added in a fixed order through LDS.
constexpr int DW_H = 32, DW_G = kThreads / DW_H;
__global__ __launch_bounds__(kThreads) void dust_w2_kernel(const float* __restrict__ Y, const float* __restrict__ ghat2,
                                                            int M, int N, int C, float lr,
                                                            const int* __restrict__ skip, float* __restrict__ W2)
{
    __shared__ float red[DW_G][DW_H][kMaxClasses + 1];
    if (*skip) return;
    const int hl = threadIdx.x % DW_H, g = threadIdx.x / DW_H;
    const int h = blockIdx.x * DW_H + hl;
    float acc[kMaxClasses];
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) acc[c] = 0.f;
    if (h < N) {
        for (int t = g; t < M; t += DW_G) {
            const float a = gelu_erf(Y[(size_t)t * N + h]);
            const float* gr = ghat2 + (size_t)t * C;
#pragma unroll
            for (int c = 0; c < kMaxClasses; ++c)
                if (c < C) acc[c] = fmaf(gr[c], a, acc[c]);
        }
    }
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) red[g][hl][c] = acc[c];
    __syncthreads();
    if (g != 0 || h >= N) return;
    for (int c = 0; c < C; ++c) {
        float sum = 0.f;
        for (int q = 0; q < DW_G; ++q) sum += red[q][hl][c];
        W2[(size_t)c * N + h] = fmaf(-lr, sum, W2[(size_t)c * N + h]);
    }
}

}  // namespace

// ----------------------------------------------------------- least squares
zo_status lsq_check(const zo_model_desc& d)
{
    if (d.d_in % 4 || d.d_out % 4) return fail(ZO_ERR_UNSUPPORTED, "least squares needs d_in, d_out multiples of 4");
    if (d.batch > (1 << 24) || d.d_in > (1 << 20) || d.d_out > (1 << 20))
        return fail(ZO_ERR_UNSUPPORTED, "least squares shape too large");
    return ZO_OK;
}

size_t lsq_workspace(const zo_model_desc& d)
{
    const size_t blocks = (size_t)cdiv((int)d.batch, LSQ_BM) * cdiv((int)d.d_out, LSQ_BN);
    return (kMaxEvalsPerCall * blocks * sizeof(double) + 255) / 256 * 256;
}

zo_status lsq_forward(const ModelView& m, const zo_batch& b, const zo_pert* perts, int n, double* loss,
                      hipStream_t s)
{
    const zo_model_desc& d = m.desc;
    EvalList ev;
    const int nv = make_evals(perts, n, ev);
    GemmArgs a = {};
    a.X = (const float*)b.x;
    a.W = (const float*)m.params + m.offsets[0];
    a.w_dir = m.offsets[0];
    a.M = (int)b.batch;
    a.N = (int)d.d_out;
    a.K = (int)d.d_in;
    a.Y = (const float*)b.y;
    a.part = (double*)m.workspace;
    zo_status st = nv == 2 ? launch_fgemm<LSQ_BM, LSQ_BN, LSQ_BK, true, 2, EPI_LSQ, 256>(a, ev, s)
                           : launch_fgemm<LSQ_BM, LSQ_BN, LSQ_BK, true, 1, EPI_LSQ, 256>(a, ev, s);
    if (st) return st;
    const int n_blocks = cdiv(a.M, LSQ_BM) * cdiv(a.N, LSQ_BN);
    const int n_evals = n == 0 ? 1 : n;
    KernelTimer timer("reduce", s);
    lsq_reduce<<<n_evals, kThreads, 0, s>>>(a.part, n_blocks, a.M, loss);
    return check_launch("lsq reduce");
}

// -------------------------------------------------------------------- MLP
zo_status mlp_check(const zo_model_desc& d)
{
    if (d.d_in % 4 || d.hidden % 4) return fail(ZO_ERR_UNSUPPORTED, "MLP needs d_in, hidden multiples of 4");
    if (d.classes > kMaxClasses) return fail(ZO_ERR_UNSUPPORTED, "MLP supports at most %d classes", kMaxClasses);
    if (d.batch > (1 << 20) || d.d_in > (1 << 20) || d.hidden > (1 << 20))
        return fail(ZO_ERR_UNSUPPORTED, "MLP shape too large");
    return ZO_OK;
}

// Workspace of the Dust step, inside the MLP's logit-partial region:
// region A = the draws' partial logits, later (once reduced) the transposed
// output-error planes and X^T; then Z, w, ghat2 and the skip flag.
struct DustLayout {
    size_t planes, xt, z, w, ghat2, skip, total;
};
static DustLayout dust_layout(const zo_model_desc& d, int M, int k1)
{
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t N = d.hidden, D = d.d_in, C = d.classes;
    const size_t part = (size_t)(k1 + 1) * cdiv((int)N, DH_BN) * C * M * sizeof(float);
    const size_t gt = 3 * N * M * sizeof(bf16_t), xt = D * M * sizeof(float);
    DustLayout L;
    L.planes = 0;
    L.xt = al(gt);
    const size_t a = std::max(al(part), L.xt + al(xt));
    L.z = a;
    L.w = L.z + al(M * C * sizeof(double));
    L.ghat2 = L.w + al((size_t)k1 * M * sizeof(float));
    L.skip = L.ghat2 + al(M * C * sizeof(float));
    L.total = L.skip + 256;
    return L;
}

size_t mlp_part_bytes(const zo_model_desc& d)
{
    const size_t tiles = cdiv((int)d.hidden, MLP_BN);
    const size_t probes = (kMaxEvalsPerCall * tiles * d.batch * d.classes * sizeof(float) + 255) / 256 * 256;
    // large enough for a Dust step with the most hidden-layer draws
    return std::max(probes, dust_layout(d, (int)d.batch, DG_MAXK).total);
}

// workspace: logit partials | per-chunk CE sums | X planes (3 M K bf16) | X W1^T (M N fp32)
constexpr int kSplitMaxEvalsPerCall = 256;  // theta_2 evaluations of one split-perturbation launch
size_t mlp_chunk_bytes(const zo_model_desc& d)
{
    const size_t evals = kMaxEvalsPerCall > kSplitMaxEvalsPerCall ? kMaxEvalsPerCall : kSplitMaxEvalsPerCall;
    return (evals * (size_t)cdiv((int)d.batch, 64) * sizeof(double) + 255) / 256 * 256;
}
size_t mlp_planes_bytes(const zo_model_desc& d) { return (3 * (size_t)d.batch * d.d_in * 2 + 255) / 256 * 256; }
size_t mlp_h_bytes(const zo_model_desc& d) { return ((size_t)d.batch * d.hidden * 4 + 255) / 256 * 256; }

size_t mlp_workspace(const zo_model_desc& d)
{
    return mlp_part_bytes(d) + mlp_chunk_bytes(d) + mlp_planes_bytes(d) + mlp_h_bytes(d);
}

zo_status mlp_forward(const ModelView& m, const zo_batch& b, const zo_pert* perts, int n, double* loss,
                      hipStream_t s)
{
    const zo_model_desc& d = m.desc;
    EvalList ev;
    const int nv = make_evals(perts, n, ev);
    const int M = (int)b.batch, N = (int)d.hidden, K = (int)d.d_in;
    char* ws = (char*)m.workspace;
    float* logit_part = (float*)ws;
    double* chunk_sum = (double*)(ws + mlp_part_bytes(d));
    int n_tiles;
    zo_status st;
    if (K % 32 == 0) {
        // split-bf16 path: X planes, then X W1^T, then one product per group
        bf16_t* planes = (bf16_t*)(ws + mlp_part_bytes(d) + mlp_chunk_bytes(d));
        SplitArgs a = {};
        a.Xp = planes;
        a.W = (const float*)m.params + m.offsets[0];
        a.w_dir = m.offsets[0];
        a.M = M;
        a.N = N;
        a.K = K;
        a.H = (float*)((char*)planes + mlp_planes_bytes(d));
        a.W2 = (const float*)m.params + m.offsets[1];
        a.w2_dir = m.offsets[1];
        a.C = (int)d.classes;
        a.logit_part = logit_part;
        {
            const size_t n4 = (size_t)M * K / 4;
            KernelTimer timer("gemm_f32_base", s);
            split_planes_kernel<<<(int)std::min<size_t>((n4 + kThreads - 1) / kThreads, 2048), kThreads, 0, s>>>(
                (const float*)b.x, n4, planes, (size_t)M * K);
        }
        if ((st = check_launch("X split"))) return st;
        // classes per thread group of the logit epilogue, rounded up to an instantiated width
        const int half = ((int)d.classes + 1) / 2;  // two groups per row in the 256 x 128 tiles
        if (n == 0) {  // four thread groups per row in the 64 x 64 tiles
            const int quarter = ((int)d.classes + 3) / 4;
            st = quarter <= 1   ? launch_sgemm<SB_BM, SB_BN, SB_NT, SG_BASE_MLP, 1, 1>(a, ev, 1, s, "gemm_f32_base")
                 : quarter <= 3 ? launch_sgemm<SB_BM, SB_BN, SB_NT, SG_BASE_MLP, 1, 3>(a, ev, 1, s, "gemm_f32_base")
                                : launch_sgemm<SB_BM, SB_BN, SB_NT, SG_BASE_MLP, 1, 4>(a, ev, 1, s, "gemm_f32_base");
            n_tiles = cdiv(N, SB_BN);
        } else {
            st = launch_sgemm<SB_BM, SB_BN, SB_NT, SG_BASE_STORE, 1>(a, ev, 1, s, "gemm_f32_base");
            if (st) return st;
            if (nv == 2)
                st = half <= 2   ? launch_sgemm<SP_BM, SP_BN, SP_NT, SG_PROBE_MLP, 2, 2>(a, ev, ev.n_groups, s, "gemm_f32")
                     : half <= 5 ? launch_sgemm<SP_BM, SP_BN, SP_NT, SG_PROBE_MLP, 2, 5>(a, ev, ev.n_groups, s, "gemm_f32")
                                 : launch_sgemm<SP_BM, SP_BN, SP_NT, SG_PROBE_MLP, 2, 8>(a, ev, ev.n_groups, s, "gemm_f32");
            else
                st = half <= 2   ? launch_sgemm<SP_BM, SP_BN, SP_NT, SG_PROBE_MLP, 1, 2>(a, ev, ev.n_groups, s, "gemm_f32")
                     : half <= 5 ? launch_sgemm<SP_BM, SP_BN, SP_NT, SG_PROBE_MLP, 1, 5>(a, ev, ev.n_groups, s, "gemm_f32")
                                 : launch_sgemm<SP_BM, SP_BN, SP_NT, SG_PROBE_MLP, 1, 8>(a, ev, ev.n_groups, s, "gemm_f32");
            n_tiles = cdiv(N, SP_BN);
        }
    } else {
        GemmArgs a = {};
        a.X = (const float*)b.x;
        a.W = (const float*)m.params + m.offsets[0];
        a.w_dir = m.offsets[0];
        a.M = M;
        a.N = N;
        a.K = K;
        a.W2 = (const float*)m.params + m.offsets[1];
        a.w2_dir = m.offsets[1];
        a.C = (int)d.classes;
        a.logit_part = logit_part;
        st = nv == 2 ? launch_fgemm<MLP_BM, MLP_BN, MLP_BK, false, 2, EPI_MLP, 512>(a, ev, s)
                     : launch_fgemm<MLP_BM, MLP_BN, MLP_BK, false, 1, EPI_MLP, 512>(a, ev, s);
        n_tiles = cdiv(N, MLP_BN);
    }
    if (st) return st;
    const int n_evals = n == 0 ? 1 : n;
    const int n_chunks = cdiv(M, 64);
    KernelTimer timer("reduce", s);
    mlp_ce_rows<<<dim3(n_chunks, n_evals), kThreads, 0, s>>>(logit_part, n_tiles, M, (int)d.classes, b.labels,
                                                              chunk_sum);
    mlp_ce_final<<<n_evals, 64, 0, s>>>(chunk_sum, n_chunks, M, loss);
    return check_launch("mlp cross-entropy");
}

zo_status mlp_split_check(const zo_model_desc& d, int p1, int ps)
{
    if (d.kind != ZO_MODEL_MLP) return fail(ZO_ERR_UNSUPPORTED, "split perturbation is defined for the MLP");
    if (d.d_in % 32) return fail(ZO_ERR_UNSUPPORTED, "split perturbation needs d_in %% 32 == 0");
    if (p1 < 1 || p1 > 1024) return fail(ZO_ERR_INVALID, "p1 must be in 1..1024");
    if (ps < 1 || ps > kSplitMaxPs) return fail(ZO_ERR_INVALID, "ps must be in 1..%d", kSplitMaxPs);
    if ((1 + ps) * d.classes > 56) return fail(ZO_ERR_UNSUPPORTED, "split perturbation: (1 + ps) * classes > 56");
    if (2 * p1 * ps > 1024) return fail(ZO_ERR_INVALID, "2 p1 ps must be at most 1024");
    return ZO_OK;
}

zo_status mlp_split_step(const ModelView& m, const zo_batch& b, uint64_t seed, int p1, int ps, float eps, float lr,
                         double* losses, double* g1, double* g2, hipStream_t s)
{
    const zo_model_desc& d = m.desc;
    const int M = (int)b.batch, N = (int)d.hidden, K = (int)d.d_in, C = (int)d.classes;
    char* ws = (char*)m.workspace;
    bf16_t* planes = (bf16_t*)(ws + mlp_part_bytes(d) + mlp_chunk_bytes(d));
    double* chunk_sum = (double*)(ws + mlp_part_bytes(d));
    SplitArgs a = {};
    a.Xp = planes;
    a.W = (const float*)m.params + m.offsets[0];
    a.w_dir = m.offsets[0];
    a.M = M;
    a.N = N;
    a.K = K;
    a.H = (float*)((char*)planes + mlp_planes_bytes(d));
    a.W2 = (const float*)m.params + m.offsets[1];
    a.w2_dir = m.offsets[1];
    a.C = C;
    a.logit_part = (float*)ws;
    a.ps = ps;
    a.z2_probe0 = (uint32_t)p1;
    const int n_tiles = cdiv(N, SP_BN), n_chunks = cdiv(M, 64);
    // directions per launch: partial slots, chunk sums and eval-list entries
    const size_t slot_bytes = (size_t)n_tiles * M * C * sizeof(float);
    const int by_slots = (int)(mlp_part_bytes(d) / slot_bytes) / (2 * (1 + ps));
    const int by_evals = kSplitMaxEvalsPerCall / (4 * ps);
    const int per_call = std::min(std::min(by_slots, by_evals), kMaxEvalsPerCall);
    if (per_call < 1) return fail(ZO_ERR_WORKSPACE, "split perturbation: workspace too small");
    zo_status st;
    {
        const size_t n4 = (size_t)M * K / 4;
        KernelTimer timer("gemm_f32_base", s);
        split_planes_kernel<<<(int)std::min<size_t>((n4 + kThreads - 1) / kThreads, 2048), kThreads, 0, s>>>(
            (const float*)b.x, n4, planes, (size_t)M * K);
    }
    if ((st = check_launch("X split"))) return st;
    EvalList base;
    make_evals(nullptr, 0, base);
    if ((st = launch_sgemm<SB_BM, SB_BN, SB_NT, SG_BASE_STORE, 1>(a, base, 1, s, "gemm_f32_base"))) return st;
    for (int d0 = 0; d0 < p1; d0 += per_call) {
        const int nd = std::min(per_call, p1 - d0);
        EvalList ev;
        memset(&ev, 0, sizeof ev);
        ev.n_groups = nd;
        ev.perturbed = 1;
        for (int gi = 0; gi < nd; ++gi) {
            ev.seed[gi] = seed;
            ev.probe[gi] = (uint32_t)(d0 + gi);
            ev.sigma[gi][0] = eps;
            ev.sigma[gi][1] = -eps;
        }
        // columns per thread group: (1 + ps) C / 2, rounded up to an instantiated width
        const int q2 = ((1 + ps) * C + 1) / 2;
        st = q2 <= 8    ? launch_sgemm<SP_BM, SP_BN, SP_NT, SG_PROBE_SPLIT, 2, 8>(a, ev, nd, s, "gemm_f32")
             : q2 <= 16 ? launch_sgemm<SP_BM, SP_BN, SP_NT, SG_PROBE_SPLIT, 2, 16>(a, ev, nd, s, "gemm_f32")
                        : launch_sgemm<SP_BM, SP_BN, SP_NT, SG_PROBE_SPLIT, 2, 28>(a, ev, nd, s, "gemm_f32");
        if (st) return st;
        const int n_e2 = nd * 2 * ps;
        KernelTimer timer("reduce", s);
        split_ce_rows<<<dim3(n_chunks, n_e2), kThreads, 0, s>>>(a.logit_part, n_tiles, M, C, ps, (double)eps,
                                                                 b.labels, chunk_sum);
        mlp_ce_final<<<2 * n_e2, 64, 0, s>>>(chunk_sum, n_chunks, M, losses + (size_t)4 * d0 * ps);
        if ((st = check_launch("split cross-entropy"))) return st;
    }
    {
        const int nt = 2 * p1 * ps + p1;
        KernelTimer timer("reduce", s);
        split_g_kernel<<<(nt + 63) / 64, 64, 0, s>>>(losses, p1, ps, (double)eps, g1, g2);
        if ((st = check_launch("split g"))) return st;
    }
    const uint64_t n1 = (uint64_t)N * K, n2 = (uint64_t)C * N;
    if ((st = launch_update((float*)m.params + m.offsets[0], ZO_F32, n1, m.offsets[0], seed, (uint32_t)p1, g1, lr, s)))
        return st;
    return launch_update((float*)m.params + m.offsets[1], ZO_F32, n2, m.offsets[1], seed, (uint32_t)(2 * p1 * ps), g2,
                         lr, s, ZO_DIRS_GAUSS, (uint32_t)p1);
}

zo_status mlp_dust_check(const zo_model_desc& d, const zo_batch& b, int k1, int k2)
{
    if (d.kind != ZO_MODEL_MLP) return fail(ZO_ERR_UNSUPPORTED, "the Dust step is defined for the MLP");
    if (d.d_in % 32) return fail(ZO_ERR_UNSUPPORTED, "the Dust step needs d_in %% 32 == 0");
    if (b.batch % 32) return fail(ZO_ERR_UNSUPPORTED, "the Dust step needs batch %% 32 == 0");
    if (k1 < 1 || k1 > DG_MAXK) return fail(ZO_ERR_INVALID, "k1 must be in 1..%d", DG_MAXK);
    if (k2 < 1 || k2 > (1 << 16)) return fail(ZO_ERR_INVALID, "k2 must be in 1..65536");
    return ZO_OK;
}

zo_status mlp_dust_step(const ModelView& m, const zo_batch& b, uint64_t seed, int k1, int k2, float sigma1,
                        float sigma2, float lr, double* losses, hipStream_t s)
{
    const zo_model_desc& d = m.desc;
    const int M = (int)b.batch, N = (int)d.hidden, K = (int)d.d_in, C = (int)d.classes;
    const DustLayout L = dust_layout(d, M, k1);
    if (L.total > mlp_part_bytes(d)) return fail(ZO_ERR_WORKSPACE, "Dust step: the batch exceeds the model's");
    char* ws = (char*)m.workspace;
    char* region = ws;  // the logit-partial region
    bf16_t* xplanes = (bf16_t*)(ws + mlp_part_bytes(d) + mlp_chunk_bytes(d));
    float* Y = (float*)((char*)xplanes + mlp_planes_bytes(d));
    float* part = (float*)region;
    bf16_t* gplanes = (bf16_t*)(region + L.planes);
    float* xt = (float*)(region + L.xt);
    double* Z = (double*)(region + L.z);
    float* w = (float*)(region + L.w);
    float* ghat2 = (float*)(region + L.ghat2);
    int* skip = (int*)(region + L.skip);
    float* W1 = (float*)m.params + m.offsets[0];
    float* W2 = (float*)m.params + m.offsets[1];
    const Key key = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    zo_status st;
    // 1. the clean first layer Y = X W1^T (split-bf16), cached for every draw
    SplitArgs a = {};
    a.Xp = xplanes;
    a.W = W1;
    a.w_dir = m.offsets[0];
    a.M = M;
    a.N = N;
    a.K = K;
    a.H = Y;
    {
        const size_t n4 = (size_t)M * K / 4;
        KernelTimer timer("gemm_f32_base", s);
        split_planes_kernel<<<(int)std::min<size_t>((n4 + kThreads - 1) / kThreads, 2048), kThreads, 0, s>>>(
            (const float*)b.x, n4, xplanes, (size_t)M * K);
    }
    if ((st = check_launch("X split"))) return st;
    EvalList base;
    make_evals(nullptr, 0, base);
    if ((st = launch_sgemm<SB_BM, SB_BN, SB_NT, SG_BASE_STORE, 1>(a, base, 1, s, "gemm_f32_base"))) return st;
    // 2. the clean and k1 noisy forwards of the layers after W1
    const int n_tiles = cdiv(N, DH_BN);
    {
        const dim3 grid(n_tiles, cdiv(M, DH_BM), k1 + 1);
        const int q = (C + 3) / 4;  // four thread groups per row
        KernelTimer timer("dust", s);
        if (q <= 1)
            dust_hidden_kernel<1><<<grid, DH_NT, 0, s>>>(Y, W2, M, N, C, key, sigma1, part);
        else if (q <= 3)
            dust_hidden_kernel<3><<<grid, DH_NT, 0, s>>>(Y, W2, M, N, C, key, sigma1, part);
        else
            dust_hidden_kernel<4><<<grid, DH_NT, 0, s>>>(Y, W2, M, N, C, key, sigma1, part);
    }
    if ((st = check_launch("dust hidden draws"))) return st;
    // 3. per-token losses of every draw, clean logits; 4. rewards and the head
    {
        KernelTimer timer("reduce", s);
        double* loss2 = losses + (size_t)(k1 + 1) * M;
        dust_rows_kernel<<<dim3(cdiv(M, 64), k1 + 1), kThreads, 0, s>>>(part, n_tiles, M, C, b.labels, losses, Z, skip);
        const size_t nh = (size_t)k2 * M;
        dust_head_loss_kernel<<<(int)std::min<size_t>((nh + kThreads - 1) / kThreads, 4096), kThreads, 0, s>>>(
            Z, b.labels, M, C, k2, sigma2, key, loss2, skip);
        dust_reward_kernel<<<M, kThreads, 0, s>>>(losses, loss2, M, C, k1, k2, sigma1, sigma2, key, w, ghat2, skip);
    }
    if ((st = check_launch("dust rewards"))) return st;
    // 5. hidden output errors (transposed planes), X^T, and W1 -= lr G^T X
    {
        KernelTimer timer("dust", s);
        dust_gy_kernel<<<dim3(cdiv(N, DG_H), cdiv(M, DG_T)), kThreads, 0, s>>>(w, M, N, k1, key, gplanes);
        transpose_kernel<<<dim3(cdiv(K, 32), cdiv(M, 32)), kThreads, 0, s>>>((const float*)b.x, M, K, xt);
    }
    if ((st = check_launch("dust output errors"))) return st;
    SplitArgs u = {};
    u.Xp = gplanes;
    u.W = xt;
    u.M = N;
    u.N = K;
    u.K = M;
    u.H = W1;
    u.lr = lr;
    u.skip = skip;
    if ((st = launch_sgemm<SB_BM, SB_BN, SB_NT, SG_UPDATE, 1>(u, base, 1, s, "update"))) return st;
    // 6. W2 -= lr sum_t ghat2_t GELU(Y_t)^T
    {
        KernelTimer timer("update", s);
        dust_w2_kernel<<<cdiv(N, DW_H), kThreads, 0, s>>>(Y, ghat2, M, N, C, lr, skip, W2);
    }
    return check_launch("dust head update");
}

}  // namespace zo
