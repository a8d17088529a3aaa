// Independent Philox4x32-10 for cross-checking the oracle: rocRAND's engine,
// called through its public API as a black box on the host.  Test helper only.
#include <rocrand/rocrand_kernel.h>
#include <cstdint>

extern "C" void rocrand_ref_philox(const uint32_t* ctr, const uint32_t* key, uint64_t n,
                                   uint32_t* out)
{
    for (uint64_t t = 0; t < n; ++t) {
        const uint32_t* c = ctr + 4 * t;
        unsigned long long seed = (unsigned long long)key[2 * t] |
                                  ((unsigned long long)key[2 * t + 1] << 32);
        unsigned long long subseq = (unsigned long long)c[2] | ((unsigned long long)c[3] << 32);
        // advance the low 64 counter bits by q blocks in pieces that fit the
        // engine's 64-bit "numbers to skip" argument (4 numbers per block)
        unsigned long long q = (unsigned long long)c[0] | ((unsigned long long)c[1] << 32);
        rocrand_device::philox4x32_10_engine eng(seed, subseq, 0);
        for (int piece = 0; piece < 4; ++piece) eng.discard(4ull * (q >> 2));
        eng.discard(4ull * (q & 3ull));
        for (int w = 0; w < 4; ++w) out[4 * t + w] = eng.next();
    }
}
