// Philox4x64-10, the counter-based random number generator of Salmon, Moraes,
// Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011):
// ten rounds over a 256-bit counter under a 128-bit key. Each round multiplies
// counter words 0 and 2 by two fixed odd 64-bit constants, and mixes the
// high halves of the products with the other two counter words and the key.
// Between rounds the key advances by two Weyl constants (the golden ratio and
// sqrt(3) - 1 in 64-bit fixed point). The same code runs on the host (for the
// library's exported generator) and on the device (for the sampling draw).
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define QRITA_HD __host__ __device__ inline
#else
#define QRITA_HD inline
#endif

namespace qrita {

QRITA_HD void mul_hilo64(uint64_t a, uint64_t b, uint64_t& hi, uint64_t& lo) {
#if defined(__HIP_DEVICE_COMPILE__)
    hi = __umul64hi(a, b);
    lo = a * b;
#else
    const unsigned __int128 p = (unsigned __int128)a * b;
    hi = (uint64_t)(p >> 64);
    lo = (uint64_t)p;
#endif
}

constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

// out = Philox4x64-10(counter, key)
QRITA_HD void philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
    uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        uint64_t hi0, lo0, hi1, lo1;
        mul_hilo64(kPhiloxM0, c0, hi0, lo0);
        mul_hilo64(kPhiloxM1, c2, hi1, lo1);
        const uint64_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

// A uniform double in [0, 1) from the top 53 bits of a 64-bit output.
QRITA_HD double uniform53(uint64_t x) { return (double)(x >> 11) * 0x1p-53; }

// The uniform of row `row` for a draw under (seed, offset): the first output
// of counter (row, offset, 0, 0) under key (seed, 0).
QRITA_HD double row_uniform(uint64_t seed, uint64_t offset, uint64_t row) {
    const uint64_t ctr[4] = {row, offset, 0ull, 0ull};
    const uint64_t key[2] = {seed, 0ull};
    uint64_t out[4];
    philox4x64_10(ctr, key, out);
    return uniform53(out[0]);
}

}  // namespace qrita
