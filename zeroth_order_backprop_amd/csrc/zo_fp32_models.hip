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
    float* logit_part;  // [eval][n_tile][M][C]
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

    float4 ra[A_PER], rb[B_PER], zb[B_PER];
    // LDS stage st: A tile at smem + st * STAGE, then NV B tiles
    constexpr int STAGE = BM * SA + NV * BN * SA;
    auto As = [&](int st) { return smem + st * STAGE; };
    auto Bs = [&](int st, int v) { return smem + st * STAGE + BM * SA + v * BN * SA; };
    auto b_coords = [&](int i, int k0, int& ln, int& lk, int& gn, int& gk) {
        if (!B_KN) { ln = i / (BK / 4); lk = 4 * (i % (BK / 4)); }
        else { lk = i / (BN / 4); ln = 4 * (i % (BN / 4)); }
        gn = n0 + ln;
        gk = k0 + lk;
    };
    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int t = 0; t < A_PER; ++t) {
            const int i = tid + t * kThreads;
            const int r = i / (BK / 4), c4 = i % (BK / 4);
            const int gm = m0 + r, gk = k0 + 4 * c4;
            ra[t] = (i < A_VEC && gm < M && gk < K) ? *reinterpret_cast<const float4*>(a.X + (size_t)gm * K + gk)
                                                     : float4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int t = 0; t < B_PER; ++t) {
            const int i = tid + t * kThreads;
            int ln, lk, gn, gk;
            b_coords(i, k0, ln, lk, gn, gk);
            const bool ok = i < B_VEC && gn < N && gk < K;
            const size_t idx = B_KN ? (size_t)gk * N + gn : (size_t)gn * K + gk;
            rb[t] = ok ? *reinterpret_cast<const float4*>(a.W + idx) : float4{0.f, 0.f, 0.f, 0.f};
        }
    };
    // direction values of B quad t of the tile at k0 (zero outside the matrix)
    auto gen_z = [&](int t, int k0) {
        const int i = tid + t * kThreads;
        int ln, lk, gn, gk;
        b_coords(i, k0, ln, lk, gn, gk);
        zb[t] = float4{0.f, 0.f, 0.f, 0.f};
        if (pert && i < B_VEC && gn < N && gk < K) {
            const size_t idx = B_KN ? (size_t)gk * N + gn : (size_t)gn * K + gk;
            zb[t] = gauss4(key, probe, (a.w_dir + idx) >> 2);
        }
    };
    auto store_tiles = [&](int st, int k0) {
#pragma unroll
        for (int t = 0; t < A_PER; ++t) {
            const int i = tid + t * kThreads;
            if (i < A_VEC) {
                const int r = i / (BK / 4), c4 = i % (BK / 4);
                *reinterpret_cast<float4*>(As(st) + r * SA + 4 * c4) = ra[t];
            }
        }
#pragma unroll
        for (int t = 0; t < B_PER; ++t) {
            const int i = tid + t * kThreads;
            if (i >= B_VEC) continue;
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

    load_tiles(0);
#pragma unroll
    for (int t = 0; t < B_PER; ++t) gen_z(t, 0);
    store_tiles(0, 0);
    __syncthreads();
    int cur = 0;
    for (int k0 = 0; k0 < K; k0 += BK) {
        const bool more = k0 + BK < K;
        if (more) load_tiles(k0 + BK);  // in flight during the MFMAs
#pragma unroll
        for (int kk = 0; kk < BK; kk += 8) {
            // lane (lr, lh) supplies k = kk + 4 lh + s in MFMA step s: the
            // same permutation of k on both operands leaves the sum unchanged
            f32x4 af[RB], bf[NV][CB];
#pragma unroll
            for (int i = 0; i < RB; ++i)
                af[i] = *reinterpret_cast<const f32x4*>(As(cur) + (wm * WM + i * 32 + lr) * SA + kk + 4 * lh);
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int j = 0; j < CB; ++j)
                    bf[v][j] = *reinterpret_cast<const f32x4*>(Bs(cur, v) + (wn * WN + j * 32 + lr) * SA + kk + 4 * lh);
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
            // the next tile's direction values, spread over this tile's MFMA
            // groups so the VALU work overlaps the matrix cores
            if (more) {
#pragma unroll
                for (int t = 0; t < B_PER; ++t)
                    if ((t * (BK / 8)) / B_PER == kk / 8) gen_z(t, k0 + BK);
            }
        }
        if (more) store_tiles(cur ^ 1, k0 + BK);
        __syncthreads();
        cur ^= 1;
    }

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
                float* dst = a.logit_part + (((size_t)ev.out[g][v] * gridDim.x + blockIdx.x) * M + gm) * C;
                for (int c = 0; c < C; ++c) {
                    const float* w2 = W2s + (v * C + c) * BN;
                    float p = 0.f;
#pragma unroll 8
                    for (int n = 0; n < BN; ++n) p = fmaf(Hs[row * SH + n], w2[n], p);
                    dst[c] = p;
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

// Cross-entropy of each row from the logit partials.  Block (chunk, e)
// covers rows 64 chunk .. +63 of evaluation e; wave w sums the hidden tiles
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
            const float* p = part + (((size_t)e * n_tiles + t) * M + m) * C;
#pragma unroll
            for (int c = 0; c < kMaxClasses; ++c)
                if (c < C) lg[c] += (double)p[c];
        }
    }
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) lg_w[wave][lane][c] = lg[c];
    __syncthreads();
    if (wave != 0) return;
    double v = 0.0;
    if (m < M) {
        const int y = labels[m];
        double mx = -INFINITY, picked = 0.0;
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
    KernelTimer timer("gemm_f32", s);
    kern<<<grid, NT, lds, s>>>(a, ev);
    return check_launch("fp32 fused GEMM");
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

size_t mlp_part_bytes(const zo_model_desc& d)
{
    const size_t tiles = cdiv((int)d.hidden, MLP_BN);
    return (kMaxEvalsPerCall * tiles * d.batch * d.classes * sizeof(float) + 255) / 256 * 256;
}

size_t mlp_workspace(const zo_model_desc& d)
{
    return mlp_part_bytes(d) + kMaxEvalsPerCall * (size_t)cdiv((int)d.batch, 64) * sizeof(double);
}

zo_status mlp_forward(const ModelView& m, const zo_batch& b, const zo_pert* perts, int n, double* loss,
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
    a.N = (int)d.hidden;
    a.K = (int)d.d_in;
    a.W2 = (const float*)m.params + m.offsets[1];
    a.w2_dir = m.offsets[1];
    a.C = (int)d.classes;
    a.logit_part = (float*)m.workspace;
    zo_status st = nv == 2 ? launch_fgemm<MLP_BM, MLP_BN, MLP_BK, false, 2, EPI_MLP, 512>(a, ev, s)
                           : launch_fgemm<MLP_BM, MLP_BN, MLP_BK, false, 1, EPI_MLP, 512>(a, ev, s);
    if (st) return st;
    const int n_evals = n == 0 ? 1 : n;
    double* chunk_sum = (double*)((char*)m.workspace + mlp_part_bytes(d));
    const int n_chunks = cdiv(a.M, 64);
    KernelTimer timer("reduce", s);
    mlp_ce_rows<<<dim3(n_chunks, n_evals), kThreads, 0, s>>>(a.logit_part, cdiv(a.N, MLP_BN), a.M, a.C, b.labels,
                                                              chunk_sum);
    mlp_ce_final<<<n_evals, 64, 0, s>>>(chunk_sum, n_chunks, a.M, loss);
    return check_launch("mlp cross-entropy");
}

}  // namespace zo
