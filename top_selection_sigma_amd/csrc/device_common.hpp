// Device helpers shared by the selection kernels: order-preserving keys,
// candidate encoding, fixed-point softmax mass, and wave/block reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define QRITA_DEV __device__ __forceinline__

namespace qrita {

constexpr int kWave = 64;
constexpr int kMaxWaves = 16;

// ---------------------------------------------------------------------------
// Keys. Every logit maps to an unsigned 32-bit key whose unsigned order is the
// value order: the float32 bit pattern with the sign bit flipped for
// non-negative values and all bits flipped for negative ones. -0.0 is mapped
// to +0.0 first so the two zeros are one value (the pages count equal logits
// as duplicates, "Metodología" §2). bf16 logits use the key of their exact
// float32 widening, so one search handles both dtypes. -inf has the smallest
// key of any non-NaN value.
// ---------------------------------------------------------------------------
QRITA_DEV uint32_t f32_key(uint32_t bits) {
    bits = (bits == 0x80000000u) ? 0u : bits;
    return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

QRITA_DEV float key_value(uint32_t key) {
    uint32_t bits = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
    return __uint_as_float(bits);
}

// A candidate is one 64-bit word: key in the high half, the bitwise complement
// of the vocabulary index in the low half. Vocabulary indices are distinct, so
// candidates are distinct, and descending candidate order is exactly the
// stable order (value descending, index ascending). The set of the K largest
// candidates is therefore {c >= B} for one 64-bit boundary B.
QRITA_DEV uint64_t make_cand(uint32_t key, uint32_t idx) {
    return ((uint64_t)key << 32) | (uint32_t)(~idx);
}
QRITA_DEV uint32_t cand_key(uint64_t c) { return (uint32_t)(c >> 32); }
QRITA_DEV uint32_t cand_low(uint64_t c) { return (uint32_t)c; }
QRITA_DEV uint32_t cand_idx(uint64_t c) { return ~(uint32_t)c; }

// ---------------------------------------------------------------------------
// Softmax mass in fixed point: e = exp(z - ref) in [0, 1] is stored as
// floor(e * 2^44) in 64 bits. Integer sums are exact and associative, so a
// mass does not depend on how candidates are split over lanes, waves or
// workgroups. 2^18 terms of at most 2^44 fit in 63 bits; the truncation error
// is below 2^-44 per term.
// ---------------------------------------------------------------------------
constexpr int kFxShift = 44;

QRITA_DEV uint64_t fx_from_unit_f32(float e) {
    // e * 2^44 is exact in float; split it into two exact 32-bit halves.
    float x = e * 0x1p44f;
    uint32_t hi = (uint32_t)(x * 0x1p-32f);
    float rem = fmaf((float)hi, -0x1p32f, x);
    uint32_t lo = (uint32_t)rem;
    return ((uint64_t)hi << 32) | lo;
}

QRITA_DEV uint64_t fx_from_unit_f64(double e) {
    return (uint64_t)(e * 0x1p44);
}

// exp(z - m) in float64 for a candidate key against the row maximum m.
QRITA_DEV uint64_t mass_fx(uint32_t key, float m) {
    float z = key_value(key);
    if (z == -__builtin_inff()) return 0;
    double d = (double)z - (double)m;  // exact: both operands are floats
    return fx_from_unit_f64(exp(d));
}

// ---------------------------------------------------------------------------
// Wave reductions (wave64). Integer reductions are exact, so the shuffle order
// is immaterial; the float sum uses a fixed butterfly so every lane ends with
// the same bits.
// ---------------------------------------------------------------------------
QRITA_DEV uint32_t wave_sum_u32(uint32_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += (uint32_t)__shfl_xor((int)x, o);
    return x;
}
QRITA_DEV uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t y = (uint32_t)__shfl_xor((int)x, o);
        x = y < x ? y : x;
    }
    return x;
}
QRITA_DEV uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t y = (uint32_t)__shfl_xor((int)x, o);
        x = y > x ? y : x;
    }
    return x;
}
QRITA_DEV uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, o);
        uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), o);
        x += ((uint64_t)hi << 32) | lo;
    }
    return x;
}
QRITA_DEV float wave_sum_f32(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Number of set bits of `mask` in lanes below this lane.
QRITA_DEV uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

QRITA_DEV uint32_t lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

}  // namespace qrita
