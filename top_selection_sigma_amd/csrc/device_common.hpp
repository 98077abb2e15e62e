// Device helpers shared by the selection kernels: order-preserving keys,
// candidate encoding, fixed-point softmax mass, and DPP wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define QRITA_DEV __device__ __forceinline__

namespace qrita {

// Logit element types (the dtype codes of the C ABI): 0 float32, 1 bfloat16,
// 2 float16. Both 16-bit types widen to float32 exactly, and keys are taken
// from the widened value, so ordering and equality are those of the logits.
template <int DT>
inline constexpr bool kW16 = DT != 0;  // 16-bit elements

// The 16-bit element in the low / high half of a 32-bit word, widened.
template <int DT>
QRITA_DEV float lo16(uint32_t w) {
    if constexpr (DT == 1) return __uint_as_float(w << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
template <int DT>
QRITA_DEV float hi16(uint32_t w) {
    if constexpr (DT == 1) return __uint_as_float(w & 0xFFFF0000u);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

constexpr int kWave = 64;
constexpr int kMaxWaves = 16;

// ---------------------------------------------------------------------------
// Keys. Every logit maps to an unsigned 32-bit key whose unsigned order is the
// value order: the float32 bit pattern with the sign bit flipped for
// non-negative values and all bits flipped for negative ones. -0.0 is mapped
// to +0.0 first so the two zeros are one value (the pages count equal logits
// as duplicates, "Metodología" §2). bf16 logits use the key of their exact
// float32 widening, so one search handles both dtypes. -inf has the smallest
// key of any non-NaN value, and every non-NaN key is nonzero.
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
// floor(e * 2^43) in 64 bits. Integer sums are exact and associative, so a
// mass does not depend on how candidates are split over lanes, waves or
// workgroups. 2^18 terms of at most 2^43 fit in 62 bits; the truncation error
// is below 2^-43 per term.
// ---------------------------------------------------------------------------
constexpr int kFxShift = 43;

QRITA_DEV uint64_t fx_from_unit_f32(float e) {
    // e * 2^43 is exact in float; split it into two exact 32-bit halves.
    float x = e * 0x1p43f;
    uint32_t hi = (uint32_t)(x * 0x1p-32f);
    float rem = fmaf((float)hi, -0x1p32f, x);
    uint32_t lo = (uint32_t)rem;
    return ((uint64_t)hi << 32) | lo;
}

// exp(z - m) for a candidate key against the row maximum m, as a float.
// y = (z - m) * log2(e) is formed in float64 (z - m is exact there) and split
// into an integer i <= 0 and a fraction f in [0, 1); the hardware exp2 gives
// 2^f to about one float ulp and ldexp applies 2^i exactly. Relative error
// about 1e-7. The value is a deterministic function of (key, m).
QRITA_DEV float mass_f32(uint32_t key, float m) {
    const float z = key_value(key);
    if (z == -__builtin_inff()) return 0.0f;
    const double y = ((double)z - (double)m) * 1.4426950408889634;
    const double fl = floor(y);
    if (fl < -160.0) return 0.0f;
    return ldexpf(__builtin_amdgcn_exp2f((float)(y - fl)), (int)fl);
}

// Fixed-point softmax mass of a candidate key, floor(exp(z - m) * 2^43).
QRITA_DEV uint64_t mass_fx(uint32_t key, float m) { return fx_from_unit_f32(mass_f32(key, m)); }

// ---------------------------------------------------------------------------
// Wave reductions (wave64) with DPP: row shifts within each 16-lane row, then
// row broadcasts across rows; lane 63 ends with the whole wave's value. No
// LDS traffic and no dependence on lane order for these exact integer ops.
// ---------------------------------------------------------------------------
template <int CTRL, int ROWMASK>
QRITA_DEV uint32_t dpp_mov(uint32_t old, uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROWMASK, 0xF, false);
}
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;
constexpr int kBcast15 = 0x142, kBcast31 = 0x143;

QRITA_DEV uint32_t readlane(uint32_t x, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}

#define QRITA_ROW_STEPS(OP, ID)                         \
    x = OP(x, dpp_mov<kShr1, 0xF>(ID, x));              \
    x = OP(x, dpp_mov<kShr2, 0xF>(ID, x));              \
    x = OP(x, dpp_mov<kShr4, 0xF>(ID, x));              \
    x = OP(x, dpp_mov<kShr8, 0xF>(ID, x));
#define QRITA_WAVE_STEPS(OP, ID)                        \
    QRITA_ROW_STEPS(OP, ID)                             \
    x = OP(x, dpp_mov<kBcast15, 0xA>(ID, x));           \
    x = OP(x, dpp_mov<kBcast31, 0xC>(ID, x));

QRITA_DEV uint32_t op_min(uint32_t a, uint32_t b) { return a < b ? a : b; }
QRITA_DEV uint32_t op_max(uint32_t a, uint32_t b) { return a > b ? a : b; }
QRITA_DEV uint32_t op_add(uint32_t a, uint32_t b) { return a + b; }

// Whole-wave reductions; the result is wave-uniform.
QRITA_DEV uint32_t wave_min_u32(uint32_t x) {
    QRITA_WAVE_STEPS(op_min, 0xFFFFFFFFu)
    return readlane(x, 63);
}
QRITA_DEV uint32_t wave_max_u32(uint32_t x) {
    QRITA_WAVE_STEPS(op_max, 0u)
    return readlane(x, 63);
}
QRITA_DEV uint32_t wave_sum_u32(uint32_t x) {
    QRITA_WAVE_STEPS(op_add, 0u)
    return readlane(x, 63);
}
// Reductions over lanes 0..15 only (lane 15 holds the result).
QRITA_DEV uint32_t row_min_u32(uint32_t x) {
    QRITA_ROW_STEPS(op_min, 0xFFFFFFFFu)
    return readlane(x, 15);
}
QRITA_DEV uint32_t row_max_u32(uint32_t x) {
    QRITA_ROW_STEPS(op_max, 0u)
    return readlane(x, 15);
}
QRITA_DEV uint32_t row_sum_u32(uint32_t x) {
    QRITA_ROW_STEPS(op_add, 0u)
    return readlane(x, 15);
}

template <int CTRL, int ROWMASK>
QRITA_DEV void add64_step(uint32_t& lo, uint32_t& hi) {
    const uint32_t blo = dpp_mov<CTRL, ROWMASK>(0u, lo);
    const uint32_t bhi = dpp_mov<CTRL, ROWMASK>(0u, hi);
    const uint32_t nlo = lo + blo;
    hi = hi + bhi + (nlo < lo ? 1u : 0u);
    lo = nlo;
}
QRITA_DEV uint64_t wave_sum_u64(uint64_t x) {
    uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
    add64_step<kShr1, 0xF>(lo, hi);
    add64_step<kShr2, 0xF>(lo, hi);
    add64_step<kShr4, 0xF>(lo, hi);
    add64_step<kShr8, 0xF>(lo, hi);
    add64_step<kBcast15, 0xA>(lo, hi);
    add64_step<kBcast31, 0xC>(lo, hi);
    return ((uint64_t)readlane(hi, 63) << 32) | readlane(lo, 63);
}
// Wave total of the fixed-point masses hi * 2^22 + lo held per lane as
// 32-bit half sums (each below 2^28): 16-lane row sums stay within 32 bits,
// the cross-row steps run in 64 bits.
QRITA_DEV uint64_t wave_sum_split(uint32_t hi, uint32_t lo) {
    {
        uint32_t x = hi;
        QRITA_ROW_STEPS(op_add, 0u)
        hi = x;
    }
    {
        uint32_t x = lo;
        QRITA_ROW_STEPS(op_add, 0u)
        lo = x;
    }
    const uint64_t v = ((uint64_t)hi << 22) + lo;
    uint32_t vl = (uint32_t)v, vh = (uint32_t)(v >> 32);
    add64_step<kBcast15, 0xA>(vl, vh);
    add64_step<kBcast31, 0xC>(vl, vh);
    return ((uint64_t)readlane(vh, 63) << 32) | readlane(vl, 63);
}

QRITA_DEV uint64_t row_sum_u64(uint64_t x) {
    uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
    add64_step<kShr1, 0xF>(lo, hi);
    add64_step<kShr2, 0xF>(lo, hi);
    add64_step<kShr4, 0xF>(lo, hi);
    add64_step<kShr8, 0xF>(lo, hi);
    return ((uint64_t)readlane(hi, 15) << 32) | readlane(lo, 15);
}

// Float wave sum with DPP steps in a fixed order (the result is the same on
// every call for the same lane values).
QRITA_DEV float wave_sum_f32_dpp(float v) {
    uint32_t x = __float_as_uint(v);
#define QRITA_FADD(CTRL, RM)                                                                         \
    x = __float_as_uint(__uint_as_float(x) + __uint_as_float(dpp_mov<CTRL, RM>(0u, x)));
    QRITA_FADD(kShr1, 0xF)
    QRITA_FADD(kShr2, 0xF)
    QRITA_FADD(kShr4, 0xF)
    QRITA_FADD(kShr8, 0xF)
    QRITA_FADD(kBcast15, 0xA)
    QRITA_FADD(kBcast31, 0xC)
#undef QRITA_FADD
    return __uint_as_float(readlane(x, 63));
}

// Exclusive suffix sum over lanes: lane l gets the sum of lanes l+1 .. 63.
QRITA_DEV uint32_t wave_suffix_sum_excl(uint32_t v) {
    // inclusive prefix sum of the lanes in reverse order
    const uint32_t tot = wave_sum_u32(v);
    uint32_t x = v;
    QRITA_WAVE_STEPS(op_add, 0u)
    return tot - x;  // x = inclusive prefix sum up to this lane
}

// Float sum with a fixed butterfly (every lane ends with the same bits).
QRITA_DEV float wave_sum_f32(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// 1 if f > p, else 0, in vector ALU operations only (a saturating subtract
// and a minimum; the minimum is kept as written so the compiler does not turn
// it back into a compare and a lane-mask select).
QRITA_DEV uint32_t gt01(uint32_t f, uint32_t p) {
    uint32_t d = __builtin_elementwise_sub_sat(f, p);
    asm("v_min_u32 %0, 1, %0" : "+v"(d));
    return d;
}
QRITA_DEV uint32_t ne01(uint32_t a, uint32_t b) {
    uint32_t d = a ^ b;
    asm("v_min_u32 %0, 1, %0" : "+v"(d));
    return d;
}

// A softmax mass e in [0, 1] as floor(e * 2^43) = hi * 2^22 + lo with
// hi <= 2^21 and lo < 2^22 (both exact; the same value as fx_from_unit_f32).
// Per-lane sums of up to 64 such halves, summed over a 16-lane row, stay
// below 2^32.
QRITA_DEV void fx_split(float e, uint32_t& hi, uint32_t& lo) {
    hi = (uint32_t)(e * 0x1p21f);
    lo = (uint32_t)fmaf((float)hi, -0x1p22f, e * 0x1p43f);
}

// threadIdx.x behind an optimisation barrier: address and mask arithmetic
// derived from it is recomputed where it is used, instead of being hoisted to
// kernel entry and held in registers for the whole kernel.
QRITA_DEV uint32_t tid_here() {
    uint32_t t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}
// first thread of this thread's wave, as a wave-uniform (scalar) value
QRITA_DEV uint32_t wave_base_here() { return __builtin_amdgcn_readfirstlane(tid_here() & ~(uint32_t)(kWave - 1)); }

// Workgroup barrier that orders LDS accesses only: global stores issued
// before it are not waited for. For code in which no thread reads global
// memory that another thread of the workgroup wrote during the kernel.
QRITA_DEV void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier over the NT threads that run a step (LDS ordering only): the
// workgroup barrier, or for a step run by one wave alone a fence that
// completes its LDS accesses (the lanes of a wave run in lockstep, and other
// waves are not waiting).
template <int NT>
QRITA_DEV void block_sync() {
    if (NT > kWave) {
        lds_sync();
    } else {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
}

// Number of set bits of `mask` in lanes below this lane.
QRITA_DEV uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace qrita
