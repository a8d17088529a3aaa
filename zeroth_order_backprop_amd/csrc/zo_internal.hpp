// Host-side declarations shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/zo.h"

namespace zo {

// Records a message for zo_last_error() and returns `st`.
zo_status fail(zo_status st, const char* fmt, ...);
// Checks the last launch on this thread; returns ZO_OK or ZO_ERR_HIP.
zo_status check_launch(const char* what);

// True while zo_timing_enable is on (launches are then bracketed one by one).
bool timing_active();

// Brackets the launches made during its lifetime with HIP events on `s` when
// timing is enabled (zo_timing_enable); a no-op otherwise.
class KernelTimer {
public:
    KernelTimer(const char* family, hipStream_t s);
    ~KernelTimer();
    KernelTimer(const KernelTimer&) = delete;
    KernelTimer& operator=(const KernelTimer&) = delete;

private:
    int slot_;
    hipStream_t s_;
};

// ---- element-wise kernels (zo_elementwise.hip) ----
// w[0..n) is direction element j0 .. j0+n-1; j0 % 4 == 0, w 16-byte aligned.
// dirs: zo_dirs (ZO_DIRS_Q8 needs j0 % 16 == 0).
zo_status launch_perturb(void* w, int dtype, uint64_t n, uint64_t j0, uint64_t seed, uint32_t probe,
                         float sigma, hipStream_t s, int dirs = ZO_DIRS_GAUSS);
// w += sum_i c_i z_i, c_i = fp32(-lr * g_i / N) from fp64 g on the device;
// nothing is written when any g_i is not finite.
// Directions p0 .. p0 + n_probes - 1 (c_i pairs with direction p0 + i).
zo_status launch_update(void* w, int dtype, uint64_t n, uint64_t j0, uint64_t seed, uint32_t n_probes,
                        const double* g, float lr, hipStream_t s, int dirs = ZO_DIRS_GAUSS, uint32_t p0 = 0);
// The in-place step's last restore and its update in one pass over w[0..n)
// (direction elements 0 .. n-1): w <- D(D(fma(sigma, z_{N-1}, w)) + sum_i c_i
// z_i), bit-identical to launch_perturb followed by launch_update; when any
// g_i is not finite only the restore is written.
zo_status launch_restore_update(void* w, int dtype, uint64_t n, uint64_t seed, uint32_t n_probes, const double* g,
                                float lr, float sigma, hipStream_t s, int dirs = ZO_DIRS_GAUSS);
zo_status launch_debug_rng(uint64_t seed, uint32_t probe, uint64_t j0, uint64_t n, uint32_t* words,
                           float* z, hipStream_t s);
// Copies 2i / 2i+1 (cstride elements apart, from `out`) = D(w +- sigma z_{p0+i}), i < np; bf16,
// Gaussian or 8-bit directions.
zo_status launch_perturb_copies(const void* w, void* out, uint64_t cstride, uint64_t n, uint64_t seed,
                                uint32_t p0, uint32_t np, float sigma, hipStream_t s, int dirs = ZO_DIRS_GAUSS);
zo_status launch_debug_box_muller(const uint32_t* pairs, uint64_t n_pairs, float* z, hipStream_t s);
// g_i = (L[2i] - L[2i+1]) / (2 (double)sigma), i < n
zo_status launch_gscalar(const double* losses, uint32_t n, float sigma, double* g, hipStream_t s);
zo_status launch_precond(const double* losses, uint32_t n, float sigma, float floor, double* g, hipStream_t s);

}  // namespace zo
