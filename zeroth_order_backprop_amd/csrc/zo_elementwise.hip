// Memory-bound passes of the SPSA step over a flat parameter vector:
//   perturb: w <- D(fma(sigma, z_i, w))          (in-place +eps / -2 eps / +eps)
//   update:  w <- D(w + sum_i c_i z_i)           (every z_i regenerated)
// where D is the storage rounding (identity for fp32, round-to-nearest-even for
// bf16).  The loop of the method (ZOO blog "Backprop 없이 Transformer를
// 학습시킨다", section "backprop의 메모리 세금", flowchart) perturbs W along N
// random directions, evaluates losses only, and applies W <- W - eta * g_hat;
// the weights are modified in place, inference-mode, with no copy (same page,
// 1.5-SPSA section: OPT-30B trained in place).
//
// Layout: each block iteration covers 2048 consecutive elements; for fp32 a
// thread owns two float4 (one per half, so every load instruction of a wave is
// one contiguous 1 KiB run), for bf16 one 16-byte vector of 8 elements.  All
// HBM traffic is 16-byte vector loads and stores, one read and one write per
// element.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>

#include "zo_dirs8.hpp"
#include "zo_internal.hpp"
#include "zo_rng.hpp"

namespace zo {
namespace {

constexpr int kThreads = 256;
constexpr int kElemsPerIter = kThreads * 8;

// ---- bf16 storage conversions --------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Two fp32 -> packed bf16, round to nearest even (hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x2 f = {lo, hi};
    bf16x2 h = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ void unpack8(uint4 v, float* f)
{
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ uint4 pack8(const float* f)
{
    return uint4{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
                 pack_bf16(f[6], f[7])};
}

// ---- streaming passes over the weights --------------------------------------
// The 8-bit-direction passes that touch each weight once (perturbation;
// updates with one or two directions) are HBM-bound.  They use the access
// pattern that streams fastest here: one 16-byte vector per thread per
// iteration, contiguous across the wave, the next iteration's vector loaded
// before this one is worked on, and four blocks of 256 threads per CU.  Over a
// 2.6 GB buffer that moves 5.3-5.5 TB/s, and 5.9 with non-temporal loads and
// stores, against 4.9 for a thread owning 16 consecutive elements.  The
// non-temporal form keeps the written weights out of the 256 MB last-level
// cache, from which the forward evaluation right after a perturbation reads a
// model that fits (GPT-small shape: its GEMMs 18% slower), so it is used only
// for passes larger than that cache.  (The Gaussian passes are bound by the
// direction generation and measured no faster in this pattern.)
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <typename T, bool NT> struct Vec16;
template <bool NT> struct Vec16<uint16_t, NT> {
    static constexpr int L = 8;  // elements per vector
    typedef u32x4_t raw_t;
    static __device__ __forceinline__ raw_t load(const uint16_t* p)
    {
        const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
        if constexpr (NT) return __builtin_nontemporal_load(q);
        else return *q;
    }
    static __device__ __forceinline__ void unpack(raw_t v, float* f) { unpack8(uint4{v.x, v.y, v.z, v.w}, f); }
    static __device__ __forceinline__ void store(uint16_t* p, const float* f)
    {
        const uint4 v = pack8(f);
        u32x4_t* q = reinterpret_cast<u32x4_t*>(p);
        if constexpr (NT) __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, q);
        else *q = u32x4_t{v.x, v.y, v.z, v.w};
    }
};
template <bool NT> struct Vec16<float, NT> {
    static constexpr int L = 4;
    typedef f32x4_t raw_t;
    static __device__ __forceinline__ raw_t load(const float* p)
    {
        const f32x4_t* q = reinterpret_cast<const f32x4_t*>(p);
        if constexpr (NT) return __builtin_nontemporal_load(q);
        else return *q;
    }
    static __device__ __forceinline__ void unpack(raw_t v, float* f)
    {
        f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
    }
    static __device__ __forceinline__ void store(float* p, const float* f)
    {
        f32x4_t* q = reinterpret_cast<f32x4_t*>(p);
        if constexpr (NT) __builtin_nontemporal_store(f32x4_t{f[0], f[1], f[2], f[3]}, q);
        else *q = f32x4_t{f[0], f[1], f[2], f[3]};
    }
};
constexpr int kStreamBlocks = 1024;
constexpr uint64_t kLastLevelCacheBytes = 256ull << 20;
constexpr uint32_t kStreamMaxProbes = 2;  // updates with more directions are VALU-bound

// Gaussian for one element j (slow path for ragged tails and debug).
__device__ __forceinline__ float gauss1(Key key, uint32_t probe, uint64_t j)
{
    float4 z = gauss4(key, probe, j >> 2);
    switch (j & 3u) {
        case 0: return z.x;
        case 1: return z.y;
        case 2: return z.z;
        default: return z.w;
    }
}

__device__ __forceinline__ float load_elem(const float* w, uint64_t i) { return w[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* w, uint64_t i) { return __uint_as_float((uint32_t)w[i] << 16); }
__device__ __forceinline__ void store_elem(float* w, uint64_t i, float v) { w[i] = v; }
__device__ __forceinline__ void store_elem(uint16_t* w, uint64_t i, float v) { w[i] = (uint16_t)(pack_bf16(v, 0.0f) & 0xFFFFu); }

// ---------------------------------------------------------------- perturb
// Elements [start, n) (the ragged tail, shorter than one block iteration),
// taken by the grid's last block after its full iterations.
template <typename T>
__device__ __forceinline__ void perturb_tail(T* __restrict__ w, uint64_t start, uint64_t n, uint64_t j0, Key key,
                                             uint32_t probe, float sigma)
{
    if (blockIdx.x != gridDim.x - 1) return;
    for (uint64_t i = start + threadIdx.x; i < n; i += kThreads)
        store_elem(w, i, fmaf(sigma, gauss1(key, probe, j0 + i), load_elem(w, i)));
}

__global__ __launch_bounds__(kThreads) void perturb_f32(float* __restrict__ w, uint64_t n_full, uint64_t n,
                                                         uint64_t j0, Key key, uint32_t probe,
                                                         float sigma)
{
    const uint64_t stride = (uint64_t)gridDim.x * kElemsPerIter;
    for (uint64_t base = (uint64_t)blockIdx.x * kElemsPerIter; base < n_full; base += stride) {
        const uint64_t ea = base + 4 * threadIdx.x;
        const uint64_t eb = ea + kElemsPerIter / 2;
        float4 wa = *reinterpret_cast<const float4*>(w + ea);
        float4 wb = *reinterpret_cast<const float4*>(w + eb);
        const float4 za = gauss4(key, probe, (j0 + ea) >> 2);
        const float4 zb = gauss4(key, probe, (j0 + eb) >> 2);
        wa.x = fmaf(sigma, za.x, wa.x); wa.y = fmaf(sigma, za.y, wa.y);
        wa.z = fmaf(sigma, za.z, wa.z); wa.w = fmaf(sigma, za.w, wa.w);
        wb.x = fmaf(sigma, zb.x, wb.x); wb.y = fmaf(sigma, zb.y, wb.y);
        wb.z = fmaf(sigma, zb.z, wb.z); wb.w = fmaf(sigma, zb.w, wb.w);
        *reinterpret_cast<float4*>(w + ea) = wa;
        *reinterpret_cast<float4*>(w + eb) = wb;
    }
    perturb_tail(w, n_full, n, j0, key, probe, sigma);
}

__global__ __launch_bounds__(kThreads) void perturb_bf16(uint16_t* __restrict__ w, uint64_t n_full, uint64_t n,
                                                          uint64_t j0, Key key, uint32_t probe,
                                                          float sigma)
{
    const uint64_t stride = (uint64_t)gridDim.x * kElemsPerIter;
    for (uint64_t base = (uint64_t)blockIdx.x * kElemsPerIter; base < n_full; base += stride) {
        const uint64_t e = base + 8 * threadIdx.x;
        uint4 v = *reinterpret_cast<const uint4*>(w + e);
        const float4 za = gauss4(key, probe, (j0 + e) >> 2);
        const float4 zb = gauss4(key, probe, ((j0 + e) >> 2) + 1);
        float f[8];
        unpack8(v, f);
        f[0] = fmaf(sigma, za.x, f[0]); f[1] = fmaf(sigma, za.y, f[1]);
        f[2] = fmaf(sigma, za.z, f[2]); f[3] = fmaf(sigma, za.w, f[3]);
        f[4] = fmaf(sigma, zb.x, f[4]); f[5] = fmaf(sigma, zb.y, f[5]);
        f[6] = fmaf(sigma, zb.z, f[6]); f[7] = fmaf(sigma, zb.w, f[7]);
        *reinterpret_cast<uint4*>(w + e) = pack8(f);
    }
    perturb_tail(w, n_full, n, j0, key, probe, sigma);
}


// ------------------------------------------------------- perturbed copies
// The copies mode's evaluation weights: from one read of the bf16 arena w,
// copy 2i receives D(w + sigma z_{p0+i}) and copy 2i+1 receives
// D(w - sigma z_{p0+i}), i < np (copies `cstride` elements apart).  The
// values are those a fused evaluation forms in its tiles, fma then one
// rounding to bf16.
__global__ __launch_bounds__(kThreads) void perturb_copies_bf16(const uint16_t* __restrict__ w,
                                                                 uint16_t* __restrict__ out, uint64_t cstride,
                                                                 uint64_t n_full, uint64_t n, Key key, uint32_t p0,
                                                                 uint32_t np, float sigma)
{
    const uint64_t stride = (uint64_t)gridDim.x * kElemsPerIter;
    for (uint64_t base = (uint64_t)blockIdx.x * kElemsPerIter; base < n_full; base += stride) {
        const uint64_t e = base + 8 * threadIdx.x;
        float f[8];
        unpack8(*reinterpret_cast<const uint4*>(w + e), f);
        for (uint32_t i = 0; i < np; ++i) {
            const float4 za = gauss4(key, p0 + i, e >> 2);
            const float4 zb = gauss4(key, p0 + i, (e >> 2) + 1);
            const float z[8] = {za.x, za.y, za.z, za.w, zb.x, zb.y, zb.z, zb.w};
            float a[8], b[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                a[t] = fmaf(sigma, z[t], f[t]);
                b[t] = fmaf(-sigma, z[t], f[t]);
            }
            *reinterpret_cast<uint4*>(out + (uint64_t)(2 * i) * cstride + e) = pack8(a);
            *reinterpret_cast<uint4*>(out + (uint64_t)(2 * i + 1) * cstride + e) = pack8(b);
        }
    }
    if (blockIdx.x != gridDim.x - 1) return;
    for (uint64_t e = n_full + threadIdx.x; e < n; e += kThreads) {
        const float v = bf16_lo(w[e]);
        for (uint32_t i = 0; i < np; ++i) {
            const float z = gauss1(key, p0 + i, e);
            store_elem(out + (uint64_t)(2 * i) * cstride, e, fmaf(sigma, z, v));
            store_elem(out + (uint64_t)(2 * i + 1) * cstride, e, fmaf(-sigma, z, v));
        }
    }
}


// ----------------------------------------------------------------- update
// Coefficients c_i = fp32(-lr * g_i / N) into LDS; returns false when any g_i
// is not finite (then the block writes nothing).
__device__ __forceinline__ bool load_coeffs(const double* __restrict__ g, uint32_t n_probes, float lr,
                                            float* c_lds, int* bad_lds)
{
    if (threadIdx.x == 0) *bad_lds = 0;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n_probes; i += kThreads) {
        const double gi = g[i];
        if (!isfinite(gi)) *bad_lds = 1;
        c_lds[i] = (float)((-(double)lr * gi) / (double)n_probes);
    }
    __syncthreads();
    return *bad_lds == 0;
}

constexpr uint32_t kMaxProbes = 1024;

// The update's ragged tail (see perturb_tail); coefficients already in LDS.
template <typename T>
__device__ __forceinline__ void update_tail(T* __restrict__ w, uint64_t start, uint64_t n, uint64_t j0, Key key,
                                            uint32_t p0, uint32_t n_probes, const float* c)
{
    if (blockIdx.x != gridDim.x - 1) return;
    for (uint64_t i = start + threadIdx.x; i < n; i += kThreads) {
        float acc = 0.f;
        for (uint32_t p = 0; p < n_probes; ++p) acc = fmaf(c[p], gauss1(key, p0 + p, j0 + i), acc);
        store_elem(w, i, load_elem(w, i) + acc);
    }
}

__global__ __launch_bounds__(kThreads) void update_f32(float* __restrict__ w, uint64_t n_full, uint64_t n,
                                                        uint64_t j0, Key key, uint32_t p0, uint32_t n_probes,
                                                        const double* __restrict__ g, float lr)
{
    __shared__ float c[kMaxProbes];
    __shared__ int bad;
    if (!load_coeffs(g, n_probes, lr, c, &bad)) return;
    const uint64_t stride = (uint64_t)gridDim.x * kElemsPerIter;
    for (uint64_t base = (uint64_t)blockIdx.x * kElemsPerIter; base < n_full; base += stride) {
        const uint64_t ea = base + 4 * threadIdx.x;
        const uint64_t eb = ea + kElemsPerIter / 2;
        float4 aa = {0.f, 0.f, 0.f, 0.f}, ab = {0.f, 0.f, 0.f, 0.f};
        for (uint32_t i = 0; i < n_probes; ++i) {
            const float ci = c[i];
            const float4 za = gauss4(key, p0 + i, (j0 + ea) >> 2);
            const float4 zb = gauss4(key, p0 + i, (j0 + eb) >> 2);
            aa.x = fmaf(ci, za.x, aa.x); aa.y = fmaf(ci, za.y, aa.y);
            aa.z = fmaf(ci, za.z, aa.z); aa.w = fmaf(ci, za.w, aa.w);
            ab.x = fmaf(ci, zb.x, ab.x); ab.y = fmaf(ci, zb.y, ab.y);
            ab.z = fmaf(ci, zb.z, ab.z); ab.w = fmaf(ci, zb.w, ab.w);
        }
        float4 wa = *reinterpret_cast<const float4*>(w + ea);
        float4 wb = *reinterpret_cast<const float4*>(w + eb);
        wa.x += aa.x; wa.y += aa.y; wa.z += aa.z; wa.w += aa.w;
        wb.x += ab.x; wb.y += ab.y; wb.z += ab.z; wb.w += ab.w;
        *reinterpret_cast<float4*>(w + ea) = wa;
        *reinterpret_cast<float4*>(w + eb) = wb;
    }
    update_tail(w, n_full, n, j0, key, p0, n_probes, c);
}

__global__ __launch_bounds__(kThreads) void update_bf16(uint16_t* __restrict__ w, uint64_t n_full, uint64_t n,
                                                         uint64_t j0, Key key, uint32_t p0, uint32_t n_probes,
                                                         const double* __restrict__ g, float lr)
{
    __shared__ float c[kMaxProbes];
    __shared__ int bad;
    if (!load_coeffs(g, n_probes, lr, c, &bad)) return;
    const uint64_t stride = (uint64_t)gridDim.x * kElemsPerIter;
    for (uint64_t base = (uint64_t)blockIdx.x * kElemsPerIter; base < n_full; base += stride) {
        const uint64_t e = base + 8 * threadIdx.x;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (uint32_t i = 0; i < n_probes; ++i) {
            const float ci = c[i];
            const float4 za = gauss4(key, p0 + i, (j0 + e) >> 2);
            const float4 zb = gauss4(key, p0 + i, ((j0 + e) >> 2) + 1);
            acc[0] = fmaf(ci, za.x, acc[0]); acc[1] = fmaf(ci, za.y, acc[1]);
            acc[2] = fmaf(ci, za.z, acc[2]); acc[3] = fmaf(ci, za.w, acc[3]);
            acc[4] = fmaf(ci, zb.x, acc[4]); acc[5] = fmaf(ci, zb.y, acc[5]);
            acc[6] = fmaf(ci, zb.z, acc[6]); acc[7] = fmaf(ci, zb.w, acc[7]);
        }
        const uint4 v = *reinterpret_cast<const uint4*>(w + e);
        float f[8];
        unpack8(v, f);
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] += acc[t];
        *reinterpret_cast<uint4*>(w + e) = pack8(f);
    }
    update_tail(w, n_full, n, j0, key, p0, n_probes, c);
}

// ------------------------------------------------- restore fused with update
// The in-place step ends with the last probe's restore w1 = D(fma(sigma,
// z_last, w)) followed by the update w2 = D(w1 + sum_i c_i z_i); nothing reads
// the weights between the two, so one pass applies both: the same two
// roundings in the same order (bit-identical to the two passes), one read and
// one write of every weight instead of two each, and z_last generated once
// (it is one of the update's directions).  When any g_i is not finite only the
// restore is written, as the two separate passes would leave it.
template <typename T>
__device__ __forceinline__ void restore_update_tail(T* __restrict__ w, uint64_t start, uint64_t n, uint64_t j0,
                                                    Key key, uint32_t n_probes, const float* c, bool ok,
                                                    float sigma)
{
    if (blockIdx.x != gridDim.x - 1) return;
    for (uint64_t i = start + threadIdx.x; i < n; i += kThreads) {
        store_elem(w, i, fmaf(sigma, gauss1(key, n_probes - 1, j0 + i), load_elem(w, i)));
        if (!ok) continue;
        float acc = 0.f;
        for (uint32_t p = 0; p < n_probes; ++p) acc = fmaf(c[p], gauss1(key, p, j0 + i), acc);
        store_elem(w, i, load_elem(w, i) + acc);
    }
}

__global__ __launch_bounds__(kThreads) void restore_update_f32(float* __restrict__ w, uint64_t n_full, uint64_t n,
                                                                uint64_t j0, Key key, uint32_t n_probes,
                                                                const double* __restrict__ g, float lr, float sigma)
{
    __shared__ float c[kMaxProbes];
    __shared__ int bad;
    const bool ok = load_coeffs(g, n_probes, lr, c, &bad);
    const uint32_t last = n_probes - 1;
    const uint64_t stride = (uint64_t)gridDim.x * kElemsPerIter;
    for (uint64_t base = (uint64_t)blockIdx.x * kElemsPerIter; base < n_full; base += stride) {
        const uint64_t ea = base + 4 * threadIdx.x;
        const uint64_t eb = ea + kElemsPerIter / 2;
        float4 aa = {0.f, 0.f, 0.f, 0.f}, ab = {0.f, 0.f, 0.f, 0.f};
        float4 ra, rb;
        if (ok) {
            for (uint32_t i = 0; i < n_probes; ++i) {
                const float ci = c[i];
                const float4 za = gauss4(key, i, (j0 + ea) >> 2);
                const float4 zb = gauss4(key, i, (j0 + eb) >> 2);
                if (i == last) {
                    ra = za;
                    rb = zb;
                }
                aa.x = fmaf(ci, za.x, aa.x); aa.y = fmaf(ci, za.y, aa.y);
                aa.z = fmaf(ci, za.z, aa.z); aa.w = fmaf(ci, za.w, aa.w);
                ab.x = fmaf(ci, zb.x, ab.x); ab.y = fmaf(ci, zb.y, ab.y);
                ab.z = fmaf(ci, zb.z, ab.z); ab.w = fmaf(ci, zb.w, ab.w);
            }
        } else {
            ra = gauss4(key, last, (j0 + ea) >> 2);
            rb = gauss4(key, last, (j0 + eb) >> 2);
        }
        float4 wa = *reinterpret_cast<const float4*>(w + ea);
        float4 wb = *reinterpret_cast<const float4*>(w + eb);
        wa.x = fmaf(sigma, ra.x, wa.x); wa.y = fmaf(sigma, ra.y, wa.y);
        wa.z = fmaf(sigma, ra.z, wa.z); wa.w = fmaf(sigma, ra.w, wa.w);
        wb.x = fmaf(sigma, rb.x, wb.x); wb.y = fmaf(sigma, rb.y, wb.y);
        wb.z = fmaf(sigma, rb.z, wb.z); wb.w = fmaf(sigma, rb.w, wb.w);
        if (ok) {
            wa.x += aa.x; wa.y += aa.y; wa.z += aa.z; wa.w += aa.w;
            wb.x += ab.x; wb.y += ab.y; wb.z += ab.z; wb.w += ab.w;
        }
        *reinterpret_cast<float4*>(w + ea) = wa;
        *reinterpret_cast<float4*>(w + eb) = wb;
    }
    restore_update_tail(w, n_full, n, j0, key, n_probes, c, ok, sigma);
}

__global__ __launch_bounds__(kThreads) void restore_update_bf16(uint16_t* __restrict__ w, uint64_t n_full,
                                                                 uint64_t n, uint64_t j0, Key key, uint32_t n_probes,
                                                                 const double* __restrict__ g, float lr, float sigma)
{
    __shared__ float c[kMaxProbes];
    __shared__ int bad;
    const bool ok = load_coeffs(g, n_probes, lr, c, &bad);
    const uint32_t last = n_probes - 1;
    const uint64_t stride = (uint64_t)gridDim.x * kElemsPerIter;
    for (uint64_t base = (uint64_t)blockIdx.x * kElemsPerIter; base < n_full; base += stride) {
        const uint64_t e = base + 8 * threadIdx.x;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float4 ra, rb;
        if (ok) {
            for (uint32_t i = 0; i < n_probes; ++i) {
                const float ci = c[i];
                const float4 za = gauss4(key, i, (j0 + e) >> 2);
                const float4 zb = gauss4(key, i, ((j0 + e) >> 2) + 1);
                if (i == last) {
                    ra = za;
                    rb = zb;
                }
                acc[0] = fmaf(ci, za.x, acc[0]); acc[1] = fmaf(ci, za.y, acc[1]);
                acc[2] = fmaf(ci, za.z, acc[2]); acc[3] = fmaf(ci, za.w, acc[3]);
                acc[4] = fmaf(ci, zb.x, acc[4]); acc[5] = fmaf(ci, zb.y, acc[5]);
                acc[6] = fmaf(ci, zb.z, acc[6]); acc[7] = fmaf(ci, zb.w, acc[7]);
            }
        } else {
            ra = gauss4(key, last, (j0 + e) >> 2);
            rb = gauss4(key, last, ((j0 + e) >> 2) + 1);
        }
        const uint4 v = *reinterpret_cast<const uint4*>(w + e);
        float f[8];
        unpack8(v, f);
        const float zr[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] = fmaf(sigma, zr[t], f[t]);
        if (ok) {
            // the restored weights as stored (bf16), then the update
            const uint4 mid = pack8(f);
            unpack8(mid, f);
#pragma unroll
            for (int t = 0; t < 8; ++t) f[t] += acc[t];
        }
        *reinterpret_cast<uint4*>(w + e) = pack8(f);
    }
    restore_update_tail(w, n_full, n, j0, key, n_probes, c, ok, sigma);
}


// ------------------------------------------------ 8-bit packed directions
// One Philox block gives the codes of 16 consecutive elements; each code is
// looked up in the LDS copy of the quantile table.  Requires j0 % 16 == 0.
// The perturbation and the update with one or two directions stream the
// weights (see above); the update with more directions, VALU-bound, gives a
// thread the 16 elements of one block per iteration (bf16: two 16-byte
// vectors; fp32: four) so that each block is generated once.
constexpr int kQ8PerIter = kThreads * 16;

template <typename T> struct Q8Io;
template <> struct Q8Io<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* w, uint64_t e, float* f)
    {
        unpack8(*reinterpret_cast<const uint4*>(w + e), f);
        unpack8(*reinterpret_cast<const uint4*>(w + e + 8), f + 8);
    }
    static __device__ __forceinline__ void store(uint16_t* w, uint64_t e, const float* f)
    {
        *reinterpret_cast<uint4*>(w + e) = pack8(f);
        *reinterpret_cast<uint4*>(w + e + 8) = pack8(f + 8);
    }
};
template <> struct Q8Io<float> {
    static __device__ __forceinline__ void load(const float* w, uint64_t e, float* f)
    {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float4 x = *reinterpret_cast<const float4*>(w + e + 4 * v);
            f[4 * v] = x.x; f[4 * v + 1] = x.y; f[4 * v + 2] = x.z; f[4 * v + 3] = x.w;
        }
    }
    static __device__ __forceinline__ void store(float* w, uint64_t e, const float* f)
    {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            *reinterpret_cast<float4*>(w + e + 4 * v) = float4{f[4 * v], f[4 * v + 1], f[4 * v + 2], f[4 * v + 3]};
    }
};

// The ragged tails of the 8-bit passes (see perturb_tail); table (and
// coefficients) already in LDS.
template <typename T>
__device__ __forceinline__ void perturb_q8_tail(T* __restrict__ w, uint64_t start, uint64_t n, uint64_t j0,
                                                Key key, uint32_t probe, float sigma, const float* tab)
{
    if (blockIdx.x != gridDim.x - 1) return;
    for (uint64_t i = start + threadIdx.x; i < n; i += kThreads)
        store_elem(w, i, fmaf(sigma, dirs8::value1(tab, key, probe, j0 + i), load_elem(w, i)));
}

template <typename T>
__device__ __forceinline__ void update_q8_tail(T* __restrict__ w, uint64_t start, uint64_t n, uint64_t j0, Key key,
                                               uint32_t p0, uint32_t n_probes, const float* c, const float* tab)
{
    if (blockIdx.x != gridDim.x - 1) return;
    for (uint64_t i = start + threadIdx.x; i < n; i += kThreads) {
        float acc = 0.f;
        for (uint32_t p = 0; p < n_probes; ++p) acc = fmaf(c[p], dirs8::value1(tab, key, p0 + p, j0 + i), acc);
        store_elem(w, i, load_elem(w, i) + acc);
    }
}

// The perturbation pass in the streaming pattern: a vector holds half (bf16)
// or a quarter (fp32) of a Philox block's 16 elements; the lanes that share a
// block each generate it (the pass has VALU to spare).
template <typename T, bool NT>
__global__ __launch_bounds__(kThreads) void perturb_q8(T* __restrict__ w, uint64_t n_full, uint64_t n, uint64_t j0,
                                                        Key key, uint32_t probe, float sigma)
{
    typedef Vec16<T, NT> V;
    constexpr int L = V::L, PER = kThreads * L;
    __shared__ float tab[256];
    dirs8::load_table(tab);
    __syncthreads();
    const uint64_t stride = (uint64_t)gridDim.x * PER;
    // the next iteration's vector is loaded (raw, unconditionally: the last
    // iteration reloads its own) before this one's codes are made
    typename V::raw_t nx = {};
    if ((uint64_t)blockIdx.x * PER < n_full) nx = V::load(w + (uint64_t)blockIdx.x * PER + L * threadIdx.x);
    for (uint64_t base = (uint64_t)blockIdx.x * PER; base < n_full; base += stride) {
        const uint64_t e = base + L * threadIdx.x;
        float f[L];
        V::unpack(nx, f);
        nx = V::load(w + e + (base + stride < n_full ? stride : 0));
        const uint4 c = dirs8::block(key, probe, (j0 + e) >> 4);
        const int w0 = (int)((j0 + e) >> 2) & 3;  // the block's first word for this vector
#pragma unroll
        for (int t = 0; t < L; ++t) {
            const int k = w0 + (t >> 2);
            const uint32_t word = k == 0 ? c.x : k == 1 ? c.y : k == 2 ? c.z : c.w;
            f[t] = fmaf(sigma, dirs8::code(tab, word, t & 3), f[t]);
        }
        V::store(w + e, f);
    }
    perturb_q8_tail(w, n_full, n, j0, key, probe, sigma, tab);
}

// The copies mode's evaluation weights with 8-bit directions: as
// perturb_copies_bf16, the direction values T[code] of one Philox block per
// 16 elements (a thread's 8 elements are half a block, words w0, w0 + 1).
__global__ __launch_bounds__(kThreads) void perturb_copies_q8(const uint16_t* __restrict__ w,
                                                              uint16_t* __restrict__ out, uint64_t cstride,
                                                              uint64_t n_full, uint64_t n, Key key, uint32_t p0,
                                                              uint32_t np, float sigma)
{
    __shared__ float tab[256];
    dirs8::load_table(tab);
    __syncthreads();
    const uint64_t stride = (uint64_t)gridDim.x * kElemsPerIter;
    for (uint64_t base = (uint64_t)blockIdx.x * kElemsPerIter; base < n_full; base += stride) {
        const uint64_t e = base + 8 * threadIdx.x;
        float f[8];
        unpack8(*reinterpret_cast<const uint4*>(w + e), f);
        const int w0 = (int)(e >> 2) & 3;  // 0 or 2
        for (uint32_t i = 0; i < np; ++i) {
            const uint4 c = dirs8::block(key, p0 + i, e >> 4);
            const uint32_t lo = w0 == 0 ? c.x : c.z, hi = w0 == 0 ? c.y : c.w;
            float a[8], b[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float z = dirs8::code(tab, t < 4 ? lo : hi, t & 3);
                a[t] = fmaf(sigma, z, f[t]);
                b[t] = fmaf(-sigma, z, f[t]);
            }
            *reinterpret_cast<uint4*>(out + (uint64_t)(2 * i) * cstride + e) = pack8(a);
            *reinterpret_cast<uint4*>(out + (uint64_t)(2 * i + 1) * cstride + e) = pack8(b);
        }
    }
    if (blockIdx.x != gridDim.x - 1) return;
    for (uint64_t e = n_full + threadIdx.x; e < n; e += kThreads) {
        const float v = bf16_lo(w[e]);
        for (uint32_t i = 0; i < np; ++i) {
            const float z = dirs8::value1(tab, key, p0 + i, e);
            store_elem(out + (uint64_t)(2 * i) * cstride, e, fmaf(sigma, z, v));
            store_elem(out + (uint64_t)(2 * i + 1) * cstride, e, fmaf(-sigma, z, v));
        }
    }
}

// The update for few directions (HBM-bound) in the streaming pattern; more
// directions make it VALU-bound, and update_q8 below generates each block once
// per thread instead.
template <typename T, uint32_t NP, bool NT>
__global__ __launch_bounds__(kThreads) void update_q8_vec(T* __restrict__ w, uint64_t n_full, uint64_t n,
                                                           uint64_t j0, Key key, uint32_t p0,
                                                           const double* __restrict__ g, float lr)
{
    typedef Vec16<T, NT> V;
    constexpr uint32_t n_probes = NP;
    constexpr int L = V::L, PER = kThreads * L;
    __shared__ float tab[256];
    __shared__ float c[kMaxProbes];
    __shared__ int bad;
    dirs8::load_table(tab);
    if (!load_coeffs(g, n_probes, lr, c, &bad)) return;  // its barriers also cover the table
    const uint64_t stride = (uint64_t)gridDim.x * PER;
    // the next iteration's vector is loaded (raw, unconditionally: the last
    // iteration reloads its own) before this one's sum is made
    typename V::raw_t nx = {};
    if ((uint64_t)blockIdx.x * PER < n_full) nx = V::load(w + (uint64_t)blockIdx.x * PER + L * threadIdx.x);
    for (uint64_t base = (uint64_t)blockIdx.x * PER; base < n_full; base += stride) {
        const uint64_t e = base + L * threadIdx.x;
        float f[L];
        V::unpack(nx, f);
        nx = V::load(w + e + (base + stride < n_full ? stride : 0));
        const int w0 = (int)((j0 + e) >> 2) & 3;
        float acc[L];
#pragma unroll
        for (int t = 0; t < L; ++t) acc[t] = 0.0f;
#pragma unroll
        for (uint32_t i = 0; i < n_probes; ++i) {
            const float ci = c[i];
            const uint4 cw = dirs8::block(key, p0 + i, (j0 + e) >> 4);
#pragma unroll
            for (int t = 0; t < L; ++t) {
                const int k = w0 + (t >> 2);
                const uint32_t word = k == 0 ? cw.x : k == 1 ? cw.y : k == 2 ? cw.z : cw.w;
                acc[t] = fmaf(ci, dirs8::code(tab, word, t & 3), acc[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < L; ++t) f[t] += acc[t];
        V::store(w + e, f);
    }
    update_q8_tail(w, n_full, n, j0, key, p0, n_probes, c, tab);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void update_q8(T* __restrict__ w, uint64_t n_full, uint64_t n, uint64_t j0,
                                                       Key key, uint32_t p0, uint32_t n_probes,
                                                       const double* __restrict__ g, float lr)
{
    __shared__ float tab[256];
    __shared__ float c[kMaxProbes];
    __shared__ int bad;
    dirs8::load_table(tab);
    if (!load_coeffs(g, n_probes, lr, c, &bad)) return;  // its barriers also cover the table
    const uint64_t stride = (uint64_t)gridDim.x * kQ8PerIter;
    for (uint64_t base = (uint64_t)blockIdx.x * kQ8PerIter; base < n_full; base += stride) {
        const uint64_t e = base + 16 * threadIdx.x;
        float f[16];
        Q8Io<T>::load(w, e, f);  // issued first, so the loads overlap the generation
        float acc[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[t] = 0.0f;
        for (uint32_t i = 0; i < n_probes; ++i) {
            const float ci = c[i];
            const uint4 cw = dirs8::block(key, p0 + i, (j0 + e) >> 4);
            const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
            for (int t = 0; t < 16; ++t) acc[t] = fmaf(ci, dirs8::code(tab, words[t >> 2], t & 3), acc[t]);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) f[t] += acc[t];
        Q8Io<T>::store(w, e, f);
    }
    update_q8_tail(w, n_full, n, j0, key, p0, n_probes, c, tab);
}

// ------------------------------------------------------------ g scalars
__global__ void gscalar_kernel(const double* __restrict__ losses, uint32_t n, double two_sigma,
                               double* __restrict__ g)
{
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) g[i] = (losses[2 * i] - losses[2 * i + 1]) / two_sigma;
}

// Probe-space diagonal preconditioning from one extra clean evaluation L0 =
// losses[2n]: h_i = (L+_i + L-_i - 2 L0) / sigma^2 estimates z_i^T H z_i, and
// g_i becomes ((L+_i - L-_i) / (2 sigma)) / max(h_i, floor), so directions of
// large curvature move less.  A non-finite loss makes g non-finite, which
// the update treats as a skipped step.
__global__ void precond_kernel(const double* __restrict__ losses, uint32_t n, double sigma, double floor,
                               double* __restrict__ g)
{
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const double lp = losses[2 * i], lm = losses[2 * i + 1], l0 = losses[2 * n];
    const double gi = (lp - lm) / (2.0 * sigma);
    const double hi = ((lp + lm) - 2.0 * l0) / (sigma * sigma);
    // fmax would drop a NaN curvature; a non-finite h must reach the update
    // as a non-finite g so the step is skipped
    g[i] = isfinite(hi) ? gi / fmax(hi, floor) : hi;
}

// ------------------------------------------------------------------ debug
__global__ __launch_bounds__(kThreads) void debug_rng_kernel(Key key, uint32_t probe, uint64_t j0, uint64_t n,
                                                              uint32_t* __restrict__ words,
                                                              float* __restrict__ z)
{
    const uint64_t t = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= n) return;
    const uint64_t j = j0 + t;
    if (words) {
        const uint64_t q = j >> 2;
        uint32_t c0 = (uint32_t)q, c1 = (uint32_t)(q >> 32), c2 = probe, c3 = 0u;
        philox4x32_10(c0, c1, c2, c3, key);
        const uint32_t sel = (uint32_t)(j & 3u);
        words[t] = sel == 0 ? c0 : sel == 1 ? c1 : sel == 2 ? c2 : c3;
    }
    if (z) z[t] = gauss1(key, probe, j);
}

__global__ __launch_bounds__(kThreads) void debug_box_muller_kernel(const uint32_t* __restrict__ pairs,
                                                                     uint64_t n_pairs, float* __restrict__ z)
{
    const uint64_t t = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= n_pairs) return;
    float a, b;
    box_muller(pairs[2 * t], pairs[2 * t + 1], a, b);
    z[2 * t] = a;
    z[2 * t + 1] = b;
}

int grid_for(uint64_t n_full, uint64_t per_iter = kElemsPerIter, uint64_t cap = 256ull * 16ull)
{
    // enough blocks to fill 256 CUs (several times over by default); the loop
    // strides the rest
    const uint64_t iters = n_full / per_iter;
    return (int)(iters < cap ? (iters ? iters : 1) : cap);
}

}  // namespace

template <typename T>
static zo_status launch_perturb_q8(T* w, uint64_t n, uint64_t j0, Key key, uint32_t probe, float sigma,
                                   hipStream_t s)
{
    if (j0 % 16) return fail(ZO_ERR_INVALID, "8-bit directions need j0 %% 16 == 0");
    constexpr uint64_t per = (uint64_t)kThreads * Vec16<T, false>::L;
    const uint64_t n_full = n / per * per;
    const int grid = grid_for(n_full, per, kStreamBlocks);
    KernelTimer timer("perturb", s);
    if (n * sizeof(T) > kLastLevelCacheBytes)
        perturb_q8<T, true><<<grid, kThreads, 0, s>>>(w, n_full, n, j0, key, probe, sigma);
    else
        perturb_q8<T, false><<<grid, kThreads, 0, s>>>(w, n_full, n, j0, key, probe, sigma);
    return check_launch("perturb (8-bit directions)");
}

template <typename T>
static zo_status launch_update_q8(T* w, uint64_t n, uint64_t j0, Key key, uint32_t p0, uint32_t n_probes,
                                  const double* g, float lr, hipStream_t s)
{
    if (j0 % 16) return fail(ZO_ERR_INVALID, "8-bit directions need j0 %% 16 == 0");
    KernelTimer timer("update", s);
    if (n_probes <= kStreamMaxProbes) {
        constexpr uint64_t per = (uint64_t)kThreads * Vec16<T, false>::L;
        const uint64_t n_full = n / per * per;
        const int grid = grid_for(n_full, per, kStreamBlocks);
        const bool nt = n * sizeof(T) > kLastLevelCacheBytes;
        static_assert(kStreamMaxProbes == 2, "instances below");
        auto k = n_probes == 1 ? (nt ? update_q8_vec<T, 1, true> : update_q8_vec<T, 1, false>)
                               : (nt ? update_q8_vec<T, 2, true> : update_q8_vec<T, 2, false>);
        k<<<grid, kThreads, 0, s>>>(w, n_full, n, j0, key, p0, g, lr);
    } else {
        const uint64_t n_full = n / kQ8PerIter * kQ8PerIter;
        update_q8<T><<<grid_for(n_full, kQ8PerIter), kThreads, 0, s>>>(w, n_full, n, j0, key, p0, n_probes, g, lr);
    }
    return check_launch("update (8-bit directions)");
}

zo_status launch_perturb_copies(const void* w, void* out, uint64_t cstride, uint64_t n, uint64_t seed,
                                uint32_t p0, uint32_t np, float sigma, hipStream_t s, int dirs)
{
    if (n == 0 || np == 0) return ZO_OK;
    const Key key = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    const uint64_t n_full = n / kElemsPerIter * kElemsPerIter;
    KernelTimer timer("perturb", s);
    if (dirs == ZO_DIRS_Q8)
        perturb_copies_q8<<<grid_for(n_full), kThreads, 0, s>>>((const uint16_t*)w, (uint16_t*)out, cstride, n_full,
                                                                n, key, p0, np, sigma);
    else
        perturb_copies_bf16<<<grid_for(n_full), kThreads, 0, s>>>((const uint16_t*)w, (uint16_t*)out, cstride,
                                                                  n_full, n, key, p0, np, sigma);
    return check_launch("perturb copies");
}

// Each pass is one launch; the grid's last block also takes the ragged tail.
zo_status launch_perturb(void* w, int dtype, uint64_t n, uint64_t j0, uint64_t seed, uint32_t probe,
                         float sigma, hipStream_t s, int dirs)
{
    if (n == 0) return ZO_OK;
    const Key key = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    if (dirs == ZO_DIRS_Q8)
        return dtype == ZO_F32 ? launch_perturb_q8((float*)w, n, j0, key, probe, sigma, s)
                               : launch_perturb_q8((uint16_t*)w, n, j0, key, probe, sigma, s);
    const uint64_t n_full = n / kElemsPerIter * kElemsPerIter;
    KernelTimer timer("perturb", s);
    if (dtype == ZO_F32)
        perturb_f32<<<grid_for(n_full), kThreads, 0, s>>>((float*)w, n_full, n, j0, key, probe, sigma);
    else
        perturb_bf16<<<grid_for(n_full), kThreads, 0, s>>>((uint16_t*)w, n_full, n, j0, key, probe, sigma);
    return check_launch("perturb");
}

zo_status launch_update(void* w, int dtype, uint64_t n, uint64_t j0, uint64_t seed, uint32_t n_probes,
                        const double* g, float lr, hipStream_t s, int dirs, uint32_t p0)
{
    if (n_probes == 0 || n_probes > kMaxProbes)
        return fail(ZO_ERR_INVALID, "update: n_probes must be in 1..%u", kMaxProbes);
    if (n == 0) return ZO_OK;
    const Key key = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    if (dirs == ZO_DIRS_Q8)
        return dtype == ZO_F32 ? launch_update_q8((float*)w, n, j0, key, p0, n_probes, g, lr, s)
                               : launch_update_q8((uint16_t*)w, n, j0, key, p0, n_probes, g, lr, s);
    const uint64_t n_full = n / kElemsPerIter * kElemsPerIter;
    KernelTimer timer("update", s);
    if (dtype == ZO_F32)
        update_f32<<<grid_for(n_full), kThreads, 0, s>>>((float*)w, n_full, n, j0, key, p0, n_probes, g, lr);
    else
        update_bf16<<<grid_for(n_full), kThreads, 0, s>>>((uint16_t*)w, n_full, n, j0, key, p0, n_probes, g, lr);
    return check_launch("update");
}

zo_status launch_restore_update(void* w, int dtype, uint64_t n, uint64_t seed, uint32_t n_probes, const double* g,
                                float lr, float sigma, hipStream_t s, int dirs)
{
    if (n_probes == 0 || n_probes > kMaxProbes)
        return fail(ZO_ERR_INVALID, "update: n_probes must be in 1..%u", kMaxProbes);
    if (dirs != ZO_DIRS_GAUSS) {
        // 8-bit directions: the two passes
        if (zo_status st = launch_perturb(w, dtype, n, 0, seed, n_probes - 1, sigma, s, dirs)) return st;
        return launch_update(w, dtype, n, 0, seed, n_probes, g, lr, s, dirs, 0);
    }
    if (n == 0) return ZO_OK;
    const Key key = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    const uint64_t n_full = n / kElemsPerIter * kElemsPerIter;
    KernelTimer timer("update", s);
    if (dtype == ZO_F32)
        restore_update_f32<<<grid_for(n_full), kThreads, 0, s>>>((float*)w, n_full, n, 0, key, n_probes, g, lr, sigma);
    else
        restore_update_bf16<<<grid_for(n_full), kThreads, 0, s>>>((uint16_t*)w, n_full, n, 0, key, n_probes, g, lr,
                                                                  sigma);
    return check_launch("restore + update");
}

zo_status launch_gscalar(const double* losses, uint32_t n, float sigma, double* g, hipStream_t s)
{
    KernelTimer timer("reduce", s);
    gscalar_kernel<<<(n + 63) / 64, 64, 0, s>>>(losses, n, 2.0 * (double)sigma, g);
    return check_launch("gscalar");
}

zo_status launch_precond(const double* losses, uint32_t n, float sigma, float floor, double* g, hipStream_t s)
{
    KernelTimer timer("reduce", s);
    precond_kernel<<<(n + 63) / 64, 64, 0, s>>>(losses, n, (double)sigma, (double)floor, g);
    return check_launch("precond");
}

zo_status launch_debug_rng(uint64_t seed, uint32_t probe, uint64_t j0, uint64_t n, uint32_t* words, float* z,
                           hipStream_t s)
{
    if (n == 0) return ZO_OK;
    const Key key = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    KernelTimer timer("debug", s);
    debug_rng_kernel<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, s>>>(key, probe, j0, n, words, z);
    return check_launch("debug_rng");
}

zo_status launch_debug_box_muller(const uint32_t* pairs, uint64_t n_pairs, float* z, hipStream_t s)
{
    if (n_pairs == 0) return ZO_OK;
    KernelTimer timer("debug", s);
    debug_box_muller_kernel<<<(unsigned)((n_pairs + kThreads - 1) / kThreads), kThreads, 0, s>>>(pairs, n_pairs, z);
    return check_launch("debug_box_muller");
}

}  // namespace zo
