// Exact top-k / top-p candidate-set selection: the gfx950 kernels.
//
// The path of the Qrita method (gist.science paper 2602.01518, "Metodología"
// and "Detalles de Implementación") in two launches on one stream:
//
//   pass 1 (one workgroup per (row, slice), see pass1_kernel):
//     a2  sampled mean / standard deviation and the normal-quantile delta
//         table give the truncation threshold t = mu + delta * sigma (§1);
//     a3  one coalesced read of the slice keeps the logits >= t (the
//         truncated set Z_t) as candidates in the row's list, zero-fills the
//         mask slice and, for top-p-only rows, accumulates the softmax mass
//         of the dropped logits (§1, "Resultado": a single pass);
//   tail (one workgroup per row, see tail_kernel):
//     a4  truncation hit test: |Z_t| >= K (or, for top-p, Z_t holds mass p);
//         on a miss the search falls back to the full row (§1);
//     a5  quaternary pivot search over the candidates: three pivots at
//         25/50/75 % of the search range per iteration, counts by wavefront
//         ballot/popcount, and for each pivot the smallest key above it (z_mn)
//         with its multiplicity (N_zmn); the search stops once
//         #{> z_mn} < K <= #{>= z_mn} (§2);
//     a6  the same search over softmax mass for top-p;
//     a7  duplicate resolution: the boundary duplicates kept are the lowest
//         vocabulary indices, found by a second quaternary search over the
//         indices of the tied candidates; then the mask is set and the kept
//         indices are written in rank order ("Pipeline": duplicate-handling
//         mask generation).
#pragma once

#include "device_common.hpp"

namespace qrita {

#include "delta_lut.inc"

struct Params {
    const void* logits;
    uint8_t* mask;
    int32_t* out_idx;
    int32_t* out_count;
    const int32_t* k;
    const float* p;
    uint32_t* hdr;      // [batch][16] per-row header
    uint64_t* glist;    // [batch][list_stride] per-row candidate list
    int32_t* diag;      // [batch][8] or null
    int64_t batch;
    int32_t vocab;
    int32_t idx_cap;
    int32_t slices;
    int32_t slice_len;   // logits per slice (multiple of 16)
    int32_t stage_cap;   // pass 1: candidate capacity of the LDS stage (entries)
    int32_t tail_cap;    // tail: candidates held in LDS (entries)
    int32_t tail_alloc;  // tail: LDS entries allocated (power of two >= max(tail_cap, 2048))
    int32_t list_cap;    // usable entries of the per-row list
    int32_t list_stride;
    int32_t force_miss;
    float delta_scale;
    int32_t pivot_mode;
};

// Per-row header words (all zero between calls).
enum : int {
    H_LIST = 1,     // candidates in the row list (pass-1 atomics)
    H_FLAGS = 2,    // bit 0: list overflow
    H_KMAX = 3,     // largest candidate key (pass-1 atomics)
    H_REST = 4,     // two words: fixed-point mass of dropped logits (top-p rows)
    H_T = 8,        // Gaussian threshold (float bits), written by slice 0
    H_TC = 9,       // collection threshold (float bits)
    H_PRED = 10,    // 1 if a miss was predicted
    H_LAMBDA = 11,  // expected sample count above the K-th value (float bits)
    H_NS = 12,      // sample size
    H_WORDS = 16
};

constexpr int kSampleChunks = 8;
constexpr int kSampleChunk = 256;
constexpr int kSampleN = kSampleChunks * kSampleChunk;

constexpr int kTieDirect = 256;   // tie groups up to this size are ranked directly
constexpr int kRankDirect = 128;  // kept sets up to this size are ranked by counting
constexpr int kSortMax = 8192;    // largest kept set sorted in one piece (E = 32 per thread)

struct Shared {
    uint32_t slot[2][kMaxWaves][16];  // per-wave partial records, double-buffered
    uint32_t ties[kTieDirect];
    float fred[kMaxWaves];
    uint32_t ncand;
    uint32_t flags;
    uint32_t gather_n;
    uint32_t u32[8];
};

extern __shared__ uint64_t qrita_dyn_lds[];

QRITA_DEV uint64_t* lds_cands() { return qrita_dyn_lds; }

struct RowMode {
    bool topk, topp, keep_all;
    uint32_t K;    // top-k size (V when off)
    float p;
    uint32_t K_t;  // ranks the candidate set must contain (0: mass-driven or none)
    bool need_cand;
};

QRITA_DEV RowMode row_mode(const Params& P, int64_t row) {
    RowMode m;
    const int32_t V = P.vocab;
    const int32_t kb = P.k ? P.k[row] : 0;
    const float pb = P.p ? P.p[row] : 1.0f;
    m.topk = kb > 0 && kb < V;
    m.K = m.topk ? (uint32_t)kb : (uint32_t)V;
    m.topp = pb < 1.0f;  // NaN compares false: off
    if (m.topp && !(pb > 0.0f)) {  // p <= 0 keeps exactly one token
        m.topp = false;
        m.topk = true;
        m.K = 1;
    }
    m.p = pb;
    m.keep_all = !m.topk && !m.topp;
    const uint32_t lcap = (P.out_idx && P.idx_cap > 0) ? (uint32_t)P.idx_cap : 0u;
    if (m.topk)
        m.K_t = m.K;
    else if (m.topp)
        m.K_t = 0;
    else
        m.K_t = lcap < (uint32_t)V ? lcap : (uint32_t)V;
    m.need_cand = m.topk || m.topp || m.K_t > 0;
    return m;
}

template <bool BF16>
QRITA_DEV float load_value(const void* rowp, int64_t e) {
    if (BF16) {
        const uint32_t u = ((const uint16_t*)rowp)[e];
        return __uint_as_float(u << 16);
    }
    return ((const float*)rowp)[e];
}

template <bool BF16>
QRITA_DEV const void* row_ptr(const Params& P, int64_t row) {
    const int64_t roff = row * (int64_t)P.vocab;
    return BF16 ? (const void*)((const uint16_t*)P.logits + roff)
                : (const void*)((const float*)P.logits + roff);
}

// ---------------------------------------------------------------------------
// Block-level combination of per-wave values: lane 0 of each wave stores its
// wave's record, one barrier, then lanes 0..NW-1 of every wave load the
// records and reduce them with 16-lane DPP steps, so every thread ends with
// the block's value without a second barrier (the two slot buffers alternate).
// ---------------------------------------------------------------------------
template <int THREADS>
QRITA_DEV void block_sum_min_max(uint32_t& sum, uint32_t& mn, uint32_t& mx, uint64_t& sum64,
                                 Shared& sh, int& rb) {
    constexpr int NW = THREADS / kWave;
    const uint32_t lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    sum = wave_sum_u32(sum);
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    sum64 = wave_sum_u64(sum64);
    uint32_t* s = sh.slot[rb][wave];
    if (lane == 0) {
        s[0] = sum;
        s[1] = mn;
        s[2] = mx;
        s[3] = (uint32_t)sum64;
        s[4] = (uint32_t)(sum64 >> 32);
    }
    __syncthreads();
    const bool v = lane < (uint32_t)NW;
    const uint32_t* q = sh.slot[rb][v ? lane : 0];
    sum = row_sum_u32(v ? q[0] : 0u);
    mn = row_min_u32(v ? q[1] : 0xFFFFFFFFu);
    mx = row_max_u32(v ? q[2] : 0u);
    sum64 = row_sum_u64(v ? ((uint64_t)q[3] | ((uint64_t)q[4] << 32)) : 0ull);
    rb ^= 1;
}

// Three u32 sums, or three u64 plus three u32 sums, or one (min, count at
// min) pair, combined across the block.
template <int THREADS>
QRITA_DEV void block_sum3(uint32_t g[3], Shared& sh, int& rb) {
    constexpr int NW = THREADS / kWave;
    const uint32_t lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    uint32_t* slot = sh.slot[rb][wave];
    if (lane == 0) {
        slot[0] = g[0];
        slot[1] = g[1];
        slot[2] = g[2];
    }
    __syncthreads();
    const bool v = lane < (uint32_t)NW;
    const uint32_t* q = sh.slot[rb][v ? lane : 0];
#pragma unroll
    for (int j = 0; j < 3; ++j) g[j] = row_sum_u32(v ? q[j] : 0u);
    rb ^= 1;
}

template <int THREADS>
QRITA_DEV void block_sum3_64(uint64_t m[3], uint32_t g[3], Shared& sh, int& rb) {
    constexpr int NW = THREADS / kWave;
    const uint32_t lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    uint32_t* slot = sh.slot[rb][wave];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const uint64_t w = wave_sum_u64(m[j]);
        if (lane == 0) {
            slot[3 + 2 * j] = (uint32_t)w;
            slot[4 + 2 * j] = (uint32_t)(w >> 32);
        }
    }
    if (lane == 0) {
        slot[0] = g[0];
        slot[1] = g[1];
        slot[2] = g[2];
    }
    __syncthreads();
    const bool v = lane < (uint32_t)NW;
    const uint32_t* q = sh.slot[rb][v ? lane : 0];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        g[j] = row_sum_u32(v ? q[j] : 0u);
        m[j] = row_sum_u64(v ? ((uint64_t)q[3 + 2 * j] | ((uint64_t)q[4 + 2 * j] << 32)) : 0ull);
    }
    rb ^= 1;
}

// Per-lane (mn, N, mx) -> block (smallest value, its multiplicity, largest
// value of the second set).
template <int THREADS>
QRITA_DEV void block_minmax(uint32_t& mn, uint32_t& N, uint32_t& mx, Shared& sh, int& rb) {
    constexpr int NW = THREADS / kWave;
    const uint32_t lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const uint32_t wm = wave_min_u32(mn);
    const uint32_t wn = wave_sum_u32(mn == wm ? N : 0u);
    const uint32_t wx = wave_max_u32(mx);
    uint32_t* slot = sh.slot[rb][wave];
    if (lane == 0) {
        slot[0] = wm;
        slot[1] = wn;
        slot[2] = wx;
    }
    __syncthreads();
    const bool v = lane < (uint32_t)NW;
    const uint32_t* q = sh.slot[rb][v ? lane : 0];
    const uint32_t lm = v ? q[0] : 0xFFFFFFFFu;
    mn = row_min_u32(lm);
    N = row_sum_u32((v && lm == mn) ? q[1] : 0u);
    mx = row_max_u32(v ? q[2] : 0u);
    rb ^= 1;
}

// ---------------------------------------------------------------------------
// Candidate sources. LdsSrc holds the row's candidates in LDS for the whole
// tail; MemSrc reads them from memory (the row list, or the row itself for the
// full-row fallback of §1). Both keep four loads in flight per thread and
// compact (not fully unrolled) loops. visit(f) calls f(candidate, index,
// valid) for every slot; the loop bounds are uniform across the workgroup.
// ---------------------------------------------------------------------------
template <int THREADS>
struct LdsSrc {
    uint32_t n;
    template <class F>
    QRITA_DEV void visit(F&& f) const {
        constexpr int U = 4;
        const uint64_t* a = qrita_dyn_lds;
        for (uint32_t base = 0; base < n; base += THREADS * U) {
            uint64_t c[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = base + (uint32_t)u * THREADS + threadIdx.x;
                c[u] = i < n ? a[i] : 0ull;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = base + (uint32_t)u * THREADS + threadIdx.x;
                f(c[u], i, i < n);
            }
        }
    }
    static constexpr bool kInLds = true;
};

template <int THREADS, bool ROW, bool BF16>
struct MemSrc {
    const uint64_t* p;  // candidate array (global)
    const void* row;    // row logits (ROW)
    uint32_t n;
    QRITA_DEV uint64_t get(uint32_t i) const {
        if (ROW) return make_cand(f32_key(__float_as_uint(load_value<BF16>(row, i))), i);
        return p[i];
    }
    template <class F>
    QRITA_DEV void visit(F&& f) const {
        constexpr int U = 4;
        for (uint32_t base = 0; base < n; base += THREADS * U) {
            uint64_t c[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = base + (uint32_t)u * THREADS + threadIdx.x;
                c[u] = i < n ? get(i) : 0ull;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = base + (uint32_t)u * THREADS + threadIdx.x;
                f(c[u], i, i < n);
            }
        }
    }
    static constexpr bool kInLds = false;
};

// Per-candidate softmax masses live in LDS (as floats, indexed like the
// source) while a top-p search runs; em == nullptr recomputes them.
QRITA_DEV float* lds_em() { return (float*)qrita_dyn_lds; }

QRITA_DEV void make_pivots(int64_t lo, int64_t hi, int mode, int field, uint32_t piv[3]) {
    const int64_t span = hi - lo;
    bool done = false;
    if (mode == 1 && field == 0 && lo >= 0) {
        const float a = key_value((uint32_t)lo), b = key_value((uint32_t)hi);
        if (__builtin_isfinite(a) && __builtin_isfinite(b)) {
            int64_t prev = lo;
            for (int j = 1; j <= 3; ++j) {
                const double v = (double)a + ((double)b - (double)a) * (0.25 * j);
                int64_t kk = (int64_t)f32_key(__float_as_uint((float)v));
                if (kk <= prev) kk = prev + 1;
                if (kk >= hi) kk = hi - 1;
                if (kk <= lo) kk = lo + 1;
                piv[j - 1] = (uint32_t)kk;
                prev = kk;
            }
            done = true;
        }
    }
    if (!done) {
        for (int j = 1; j <= 3; ++j) {
            int64_t pj = lo + ((span * j) >> 2);
            if (pj <= lo) pj = lo + 1;
            if (pj >= hi) pj = hi - 1;
            piv[j - 1] = (uint32_t)pj;
        }
    }
}

// One pivot evaluation. Phase A: for the three pivots, G = #{x > pivot} by
// wavefront ballot/popcount (and, for the mass search, M = mass of x above
// the pivot). Phase B: only the highest pivot j* whose count (mass) still
// reaches the target can end the search or move its lower end, so z_mn and
// N_zmn are formed for that pivot alone. Pivots ascend and G, M do not
// increase, so j* is found from phase A.
struct Eval {
    uint32_t G[3];
    uint64_t M[3];
    int js;  // -1: no pivot reaches the target
    uint32_t mn, N;
    uint32_t mx;  // largest value <= the pivot above j* (0 if none)
};

QRITA_DEV uint32_t sel3(int j, const uint32_t x[3]) { return j == 2 ? x[2] : (j == 1 ? x[1] : x[0]); }
QRITA_DEV uint64_t sel3(int j, const uint64_t x[3]) { return j == 2 ? x[2] : (j == 1 ? x[1] : x[0]); }

template <int THREADS, class S>
QRITA_DEV Eval eval_pivots(const S& src, uint64_t filter, int field, uint32_t key_eq,
                           const uint32_t piv[3], bool mass, uint32_t K, double T, const float* em,
                           float m, Shared& sh, int& rb) {
    Eval E;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        E.G[j] = 0;
        E.M[j] = 0;
    }
    src.visit([&](uint64_t c, uint32_t i, bool valid) {
        const bool ok = valid && c >= filter && (field == 0 || cand_key(c) == key_eq);
        const uint32_t f = field == 0 ? cand_key(c) : cand_low(c);
        uint64_t e = 0;
        if (mass && ok) e = fx_from_unit_f32(em ? em[i] : mass_f32(f, m));
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const bool gt = ok && f > piv[j];
            E.G[j] += (uint32_t)__popcll(__ballot(gt));
            if (mass) E.M[j] += gt ? e : 0ull;
        }
    });
    if (mass) {
        block_sum3_64<THREADS>(E.M, E.G, sh, rb);
        E.js = (double)E.M[2] >= T ? 2 : ((double)E.M[1] >= T ? 1 : ((double)E.M[0] >= T ? 0 : -1));
    } else {
        block_sum3<THREADS>(E.G, sh, rb);
        E.js = E.G[2] >= K ? 2 : (E.G[1] >= K ? 1 : (E.G[0] >= K ? 0 : -1));
    }
    // Phase B also takes, for the pivot just above j*, the largest value at
    // or below it (z_mx): no value lies between z_mx and that pivot, so z_mx
    // can become the new upper end, mirroring the jump of the lower end to
    // z_mn.
    const uint32_t pj = E.js >= 0 ? sel3(E.js, piv) : 0u;
    const uint32_t pu = E.js < 2 ? sel3(E.js + 1, piv) : 0xFFFFFFFFu;
    uint32_t mn = 0xFFFFFFFFu, N = 0, mx = 0;
    src.visit([&](uint64_t c, uint32_t, bool valid) {
        const bool ok = valid && c >= filter && (field == 0 || cand_key(c) == key_eq);
        const uint32_t f = field == 0 ? cand_key(c) : cand_low(c);
        const bool gt = ok && E.js >= 0 && f > pj;
        const bool lt = gt && f < mn;
        N = lt ? 1u : N + ((gt && f == mn) ? 1u : 0u);
        mn = lt ? f : mn;
        const bool le = ok && f <= pu;
        mx = (le && f > mx) ? f : mx;
    });
    block_minmax<THREADS>(mn, N, mx, sh, rb);
    E.mn = mn;
    E.N = N;
    E.mx = mx;
    return E;
}

struct CountOut {
    uint32_t v, n_gt, N;
};

// Quaternary pivot search for the K-th largest field value (K >= 1) among the
// selected candidates, with duplicates: returns v, n_gt = #{> v} and
// N = #{== v}, so #{> v} < K <= #{>= v}. Invariant: G(lo) >= K > G(hi) with
// G(x) = #{field > x}. Each iteration tests pivots at 25/50/75 % of (lo, hi);
// for a pivot with G >= K, z_mn (smallest value above it) and N_zmn decide
// termination (G - N_zmn < K means z_mn is the boundary value), otherwise
// z_mn itself becomes the new lower end since G(z_mn) = G - N_zmn >= K.
template <int THREADS, class S>
QRITA_DEV CountOut qsearch_count(const S& src, uint64_t filter, int field, uint32_t key_eq,
                                 uint32_t K, int64_t lo, uint32_t G_lo, int64_t hi, uint32_t G_hi,
                                 int mode, Shared& sh, int& rb, int& iters) {
    for (int guard = 0; guard < 80; ++guard) {
        if (hi - lo <= 1) return CountOut{(uint32_t)hi, G_hi, G_lo - G_hi};
        uint32_t piv[3];
        make_pivots(lo, hi, mode, field, piv);
        const Eval E = eval_pivots<THREADS>(src, filter, field, key_eq, piv, false, K, 0.0, nullptr, 0.0f,
                                            sh, rb);
        ++iters;
        if (E.js >= 0) {
            const uint32_t g = sel3(E.js, E.G);
            if (g - E.N < K) return CountOut{E.mn, g - E.N, E.N};
            lo = E.mn;
            G_lo = g - E.N;
        }
        if (E.js < 2) {
            // G(z_mx) = G(pivot): nothing lies in (z_mx, pivot]
            const int64_t pu = sel3(E.js + 1, piv);
            hi = ((int64_t)E.mx > lo) ? (int64_t)E.mx : pu;
            G_hi = sel3(E.js + 1, E.G);
        }
    }
    return CountOut{(uint32_t)hi, G_hi, G_lo - G_hi};  // not reached for consistent inputs
}

struct MassOut {
    uint32_t v, n_gt, N;
    uint64_t M_gt;
};

// The same quaternary search over softmax mass: finds the key v with
// M(> v) < T <= M(>= v) among candidates c >= filter.
template <int THREADS, class S>
QRITA_DEV MassOut qsearch_mass(const S& src, uint64_t filter, double T, const float* em, float m,
                               int64_t lo, uint64_t M_lo, uint32_t G_lo, int64_t hi, int mode,
                               Shared& sh, int& rb, int& iters) {
    uint64_t M_hi = 0;
    uint32_t G_hi = 0;
    for (int guard = 0; guard < 80; ++guard) {
        if (hi - lo <= 1) return MassOut{(uint32_t)hi, G_hi, G_lo - G_hi, M_hi};
        uint32_t piv[3];
        make_pivots(lo, hi, mode, 0, piv);
        const Eval E = eval_pivots<THREADS>(src, filter, 0, 0u, piv, true, 0u, T, em, m, sh, rb);
        ++iters;
        if (E.js >= 0) {
            const uint64_t above = sel3(E.js, E.M) - (uint64_t)E.N * mass_fx(E.mn, m);
            const uint32_t g = sel3(E.js, E.G);
            if ((double)above < T) return MassOut{E.mn, g - E.N, E.N, above};
            lo = E.mn;
            M_lo = above;
            G_lo = g - E.N;
        }
        if (E.js < 2) {
            const int64_t pu = sel3(E.js + 1, piv);
            hi = ((int64_t)E.mx > lo) ? (int64_t)E.mx : pu;
            M_hi = sel3(E.js + 1, E.M);
            G_hi = sel3(E.js + 1, E.G);
        }
    }
    return MassOut{(uint32_t)hi, G_hi, G_lo - G_hi, M_hi};
}

// Boundary of "the `need` lowest-index candidates with key v, plus everything
// above v", restricted to c >= filter; N = #{key == v, c >= filter}. A small
// tie group is ranked directly in LDS; a large one by a quaternary search
// over the tied candidates' indices.
template <int THREADS, class S>
QRITA_DEV uint64_t tie_boundary(const S& src, uint64_t filter, uint32_t v, uint32_t need, uint32_t N,
                                uint32_t V, Shared& sh, int& rb, int& iters) {
    uint64_t b = (uint64_t)v << 32;
    if (need < N) {
        if (N <= kTieDirect) {
            __syncthreads();
            if (threadIdx.x == 0) sh.gather_n = 0;
            __syncthreads();
            src.visit([&](uint64_t c, uint32_t, bool valid) {
                if (valid && c >= filter && cand_key(c) == v) {
                    const uint32_t pos = atomicAdd(&sh.gather_n, 1u);
                    if (pos < (uint32_t)kTieDirect) sh.ties[pos] = cand_low(c);
                }
            });
            __syncthreads();
            // the tie whose complemented index has exactly need - 1 larger ones
            for (uint32_t i = threadIdx.x; i < N; i += THREADS) {
                const uint32_t x = sh.ties[i];
                uint32_t above = 0;
                for (uint32_t j = 0; j < N; ++j) above += sh.ties[j] > x ? 1u : 0u;
                if (above == need - 1) sh.u32[6] = x;
            }
            __syncthreads();
            b |= sh.u32[6];
        } else {
            const int64_t lo = (int64_t)(0xFFFFFFFFu - (uint32_t)(V - 1)) - 1;
            const CountOut t = qsearch_count<THREADS>(src, filter, 1, v, need, lo, N,
                                                      (int64_t)0xFFFFFFFFu, 0u, 0, sh, rb, iters);
            b |= t.v;
        }
    }
    return b > filter ? b : filter;
}

// Boundary B of the K largest candidates among c >= filter, which holds
// `total` >= K candidates with keys in (lo_key, kmax].
template <int THREADS, class S>
QRITA_DEV uint64_t select_boundary(const S& src, uint64_t filter, uint32_t K, uint32_t total,
                                   int64_t lo_key, uint32_t kmax, uint32_t V, int mode, Shared& sh,
                                   int& rb, int& iters) {
    const CountOut r = qsearch_count<THREADS>(src, filter, 0, 0u, K, lo_key, total, (int64_t)kmax,
                                              0u, mode, sh, rb, iters);
    return tie_boundary<THREADS>(src, filter, r.v, K - r.n_gt, r.N, V, sh, rb, iters);
}

QRITA_DEV uint32_t next_pow2(uint32_t x) {
    uint32_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

// Bitonic sort, descending, of the THREADS * E entries of a[] (any order),
// then out[g] = index of rank g for g < cnt. Thread t holds the logical
// elements g = t * E + e in registers; LDS holds element (t, e) at
// e * THREADS + t, so every LDS access of a wave touches consecutive
// addresses. Stages whose partner distance is below E run in registers, the
// others exchange through LDS.
template <int THREADS, int E>
QRITA_DEV void bitonic_tile(uint64_t* a, int32_t* out, uint32_t cnt) {
    constexpr uint32_t NP = (uint32_t)THREADS * E;
    const uint32_t t = threadIdx.x;
    uint64_t x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = a[e * THREADS + t];
    for (uint32_t k = 2; k <= NP; k <<= 1) {
        // partner distance j >= E: through LDS
        for (uint32_t j = k >> 1; j >= (uint32_t)E; j >>= 1) {
            __syncthreads();
#pragma unroll
            for (int e = 0; e < E; ++e) a[e * THREADS + t] = x[e];
            __syncthreads();
            const uint32_t pt = t ^ (j / E);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const uint64_t y = a[e * THREADS + pt];
                const uint32_t g = t * E + e;
                // the lower position of a descending pair keeps the larger value
                const bool keep_max = ((g & j) == 0) == ((g & k) == 0);
                x[e] = keep_max ? (x[e] > y ? x[e] : y) : (x[e] < y ? x[e] : y);
            }
        }
        // partner distance j < E: inside this thread's registers (constant j)
#pragma unroll
        for (int j = E / 2; j >= 1; j >>= 1) {
            if ((uint32_t)j < k) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if ((e & j) == 0) {
                        const bool desc = ((t * E + e) & k) == 0;
                        const uint64_t p = x[e], q = x[e | j];
                        const bool sw = desc ? (p < q) : (p > q);
                        x[e] = sw ? q : p;
                        x[e | j] = sw ? p : q;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t g = t * E + e;
        if (g < cnt) out[g] = (int32_t)cand_idx(x[e]);
    }
    __syncthreads();
}

template <int THREADS>
QRITA_DEV void sort_desc(uint64_t* a, uint32_t np, int32_t* out, uint32_t cnt) {
    switch (np / THREADS) {
        case 0:
        case 1: bitonic_tile<THREADS, 1>(a, out, cnt); break;
        case 2: bitonic_tile<THREADS, 2>(a, out, cnt); break;
        case 4: bitonic_tile<THREADS, 4>(a, out, cnt); break;
        case 8: bitonic_tile<THREADS, 8>(a, out, cnt); break;
        case 16: bitonic_tile<THREADS, 16>(a, out, cnt); break;
        default: bitonic_tile<THREADS, 32>(a, out, cnt); break;
    }
}

// Gather the candidates in [lo_b, hi_b) (exactly `cnt` <= tail_alloc of them)
// into LDS, put them in rank order and write their indices to
// out_idx[row][off ...]. Up to kRankDirect entries are ranked by counting;
// larger sets are sorted.
template <int THREADS, class S>
QRITA_DEV void emit_indices(const Params& P, int64_t row, const S& src, uint64_t lo_b, uint64_t hi_b,
                            uint32_t cnt, uint32_t off, Shared& sh) {
    uint64_t* a = lds_cands();
    __syncthreads();
    if (threadIdx.x == 0) sh.gather_n = 0;
    __syncthreads();
    if (S::kInLds) {
        // in place: a round reads its THREADS entries before any write of that
        // round, and the writes land below the next round's entries
        const uint32_t n = src.n;
        for (uint32_t base = 0; base < n; base += THREADS) {
            const uint32_t i = base + threadIdx.x;
            const uint64_t c = i < n ? a[i] : 0ull;
            const bool take = i < n && c >= lo_b && c < hi_b;
            __syncthreads();
            if (take) a[atomicAdd(&sh.gather_n, 1u)] = c;
        }
    } else {
        const uint32_t cap = (uint32_t)P.tail_alloc;
        src.visit([&](uint64_t c, uint32_t, bool valid) {
            if (valid && c >= lo_b && c < hi_b) {
                const uint32_t pos = atomicAdd(&sh.gather_n, 1u);
                if (pos < cap) a[pos] = c;
            }
        });
    }
    __syncthreads();
    int32_t* out = P.out_idx + row * (int64_t)P.idx_cap + off;
    if (cnt <= (uint32_t)kRankDirect) {
        for (uint32_t i = threadIdx.x; i < cnt; i += THREADS) {
            const uint64_t x = a[i];
            uint32_t r = 0;
            for (uint32_t j = 0; j < cnt; ++j) r += a[j] > x ? 1u : 0u;
            out[r] = (int32_t)cand_idx(x);
        }
        __syncthreads();
        return;
    }
    uint32_t np = next_pow2(cnt);
    if (np < (uint32_t)THREADS) np = THREADS;
    for (uint32_t i = cnt + threadIdx.x; i < np; i += THREADS) a[i] = 0ull;
    __syncthreads();
    sort_desc<THREADS>(a, np, out, cnt);
}

struct TailDiag {
    int32_t n_t;
    int32_t iters;
};

// Steps a4-a7 of the path on one candidate source. All candidates have keys
// in (key_lo, kmax]; rest_fx is the fixed-point mass, relative to rest_ref, of
// the logits left out of the source (top-p-only rows). Returns false when the
// source does not contain the answer (a truncation miss), in which case
// nothing has been written.
template <int THREADS, bool ROW, class S>
QRITA_DEV bool finish_row(const Params& P, int64_t row, const RowMode& md, const S& src, int64_t key_lo,
                          uint32_t kmax, uint64_t rest_fx, float rest_ref, float t_gauss, Shared& sh,
                          int& rb, TailDiag& dg) {
    const uint32_t V = (uint32_t)P.vocab;
    const uint32_t n = src.n;
    if (P.diag) {  // #{z >= Gaussian t} among the candidates, for diagnostics
        const uint32_t key_t = f32_key(__float_as_uint(t_gauss));
        uint32_t c = 0, d0 = 0, d1 = 0;
        uint64_t d2 = 0;
        src.visit([&](uint64_t x, uint32_t, bool valid) { c += (valid && cand_key(x) >= key_t) ? 1u : 0u; });
        block_sum_min_max<THREADS>(c, d0, d1, d2, sh, rb);
        dg.n_t = (int32_t)c;
    }
    bool topk = md.topk, topp = md.topp;
    uint32_t K = md.K;
    // a4: truncation hit test
    if (md.K_t > 0 && n < md.K_t) return false;
    if (topp && n == 0) return false;
    const float m = key_value(kmax);
    if (topp && m == -__builtin_inff()) {  // all -inf: keep one token
        topp = false;
        topk = true;
        K = 1;
    }
    uint64_t B = 0ull;  // kept set = {c >= B}
    uint32_t L = V;     // kept count
    uint32_t setn = n;  // candidates with c >= B
    if (topk) {
        B = select_boundary<THREADS>(src, 0ull, K, n, key_lo, kmax, V, P.pivot_mode, sh, rb, dg.iters);
        L = K;
        setn = K;
    }
    if (topp) {
        // per-candidate masses in LDS after the candidates, when they fit
        float* em = nullptr;
        if (S::kInLds) {
            if ((size_t)n * 12 <= (size_t)P.tail_alloc * 8) em = (float*)(qrita_dyn_lds + n);
        } else if ((size_t)n * 4 <= (size_t)P.tail_alloc * 8) {
            em = lds_em();
        }
        uint32_t d0 = 0, d1 = 0, d2 = 0;
        uint64_t ms = 0;
        __syncthreads();
        src.visit([&](uint64_t c, uint32_t i, bool valid) {
            if (valid) {
                const float e = mass_f32(cand_key(c), m);
                if (em) em[i] = e;
                if (c >= B) ms += fx_from_unit_f32(e);
            }
        });
        block_sum_min_max<THREADS>(d0, d1, d2, ms, sh, rb);
        double mass_all = (double)ms;
        if (!topk && rest_fx) mass_all += (double)rest_fx * exp((double)rest_ref - (double)m);
        const double T = (double)md.p * mass_all;
        if (!topk && (double)ms < T) return false;  // mass p not inside the candidates
        const int64_t lo = B ? (int64_t)cand_key(B) - 1 : key_lo;
        const MassOut mo = qsearch_mass<THREADS>(src, B, T, em, m, lo, ms, setn, (int64_t)kmax,
                                                 P.pivot_mode, sh, rb, dg.iters);
        // smallest number of duplicates at v that reaches T
        const uint64_t e = mass_fx(mo.v, m);
        uint32_t need = mo.N;
        if (e > 0) {
            const double x = (T - (double)mo.M_gt) / (double)e;
            uint64_t j = x <= 1.0 ? 1ull : (x >= (double)mo.N ? (uint64_t)mo.N : (uint64_t)ceil(x));
            if (j > mo.N) j = mo.N;
            if (j < 1) j = 1;
            while (j > 1 && (double)(mo.M_gt + (j - 1) * e) >= T) --j;
            while (j < mo.N && (double)(mo.M_gt + j * e) < T) ++j;
            need = (uint32_t)j;
        }
        B = tie_boundary<THREADS>(src, B, mo.v, need, mo.N, V, sh, rb, dg.iters);
        L = mo.n_gt + need;
        setn = L;
    }
    const int64_t roff = row * (int64_t)V;
    // a7: mask (keep-all rows were written in pass 1)
    if (P.mask && !md.keep_all) {
        uint8_t* mrow = P.mask + roff;
        src.visit([&](uint64_t c, uint32_t i, bool valid) {
            if (ROW) {
                if (valid) mrow[i] = c >= B ? 1 : 0;
            } else if (valid && c >= B) {
                mrow[cand_idx(c)] = 1;
            }
        });
    }
    // a7: indices in rank order
    if (P.out_idx && P.idx_cap > 0) {
        const uint32_t Lout = L < (uint32_t)P.idx_cap ? L : (uint32_t)P.idx_cap;
        const uint32_t cap = (uint32_t)kSortMax;
        if (Lout <= cap || S::kInLds) {
            uint64_t Bo = B;
            if (Lout < L)
                Bo = select_boundary<THREADS>(src, B, Lout, setn, B ? (int64_t)cand_key(B) - 1 : key_lo,
                                              kmax, V, P.pivot_mode, sh, rb, dg.iters);
            emit_indices<THREADS>(P, row, src, Bo, ~0ull, Lout, 0u, sh);
        } else {
            // rank windows of `cap` entries, each found by its own boundary
            uint64_t prev = ~0ull;
            for (uint32_t done = 0; done < Lout;) {
                const uint32_t cnt = min(cap, Lout - done);
                const uint64_t Bn = select_boundary<THREADS>(src, 0ull, done + cnt, n, key_lo, kmax, V,
                                                             P.pivot_mode, sh, rb, dg.iters);
                emit_indices<THREADS>(P, row, src, Bn, prev, cnt, done, sh);
                prev = Bn;
                done += cnt;
            }
        }
    }
    if (P.out_count && threadIdx.x == 0) P.out_count[row] = (int32_t)L;
    return true;
}

// ---------------------------------------------------------------------------
// a2: sampled statistics and the threshold.
// ---------------------------------------------------------------------------
struct Thresh {
    float t;   // Gaussian threshold mu + delta * sigma
    float tc;  // threshold used for collection
    bool predicted;
    uint32_t n_s;
    float lambda;
};

QRITA_DEV int lut_k_index(float ratio) {
    const float x = log2f(ratio);
    const float f = ceilf((x - QRITA_LUT_K_MIN) * QRITA_LUT_K_STEPS);
    return (int)fminf(fmaxf(f, 0.0f), (float)(QRITA_LUT_K_N - 1));
}

// Load the row's sample into registers: 8 chunks of 256 consecutive logits at
// evenly spaced offsets (the whole row when it has at most 2048 logits).
template <bool BF16>
QRITA_DEV void load_sample(const void* rowp, int32_t V, float x[8], bool in[8]) {
    const int tid = threadIdx.x;
    const bool whole = V <= kSampleN;
    const int64_t pos0 =
        whole ? (int64_t)tid * 8
              : ((int64_t)(tid >> 5) * (int64_t)(V - kSampleChunk)) / (kSampleChunks - 1) + (int64_t)(tid & 31) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t e = pos0 + i;
        in[i] = tid < kSampleN / 8 && e < V;
        x[i] = in[i] ? load_value<BF16>(rowp, e) : 0.0f;
    }
}

// r-th largest key of the sample (1 <= r <= number of sample entries), by the
// same quaternary search over the sample held in LDS.
template <int THREADS, bool BF16>
QRITA_DEV float sample_rank_value(const void* rowp, int32_t V, uint32_t r, Shared& sh, int& rb) {
    float x[8];
    bool in[8];
    load_sample<BF16>(rowp, V, x, in);
    uint64_t* a = lds_cands();
    __syncthreads();
    if (threadIdx.x < kSampleN / 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            a[threadIdx.x * 8 + i] =
                in[i] ? make_cand(f32_key(__float_as_uint(x[i])), threadIdx.x * 8 + i) : 0ull;
    }
    __syncthreads();
    const LdsSrc<THREADS> src{(uint32_t)kSampleN};
    const uint32_t ns = (uint32_t)min(V, kSampleN);
    int it = 0;
    const CountOut o = qsearch_count<THREADS>(src, 1ull, 0, 0u, r, -1, ns, (int64_t)0xFFFFFFFFu, 0u, 0,
                                              sh, rb, it);
    __syncthreads();
    return key_value(o.v);
}

template <int THREADS, bool BF16>
QRITA_DEV Thresh compute_threshold(const Params& P, const RowMode& md, const void* rowp, Shared& sh,
                                   int& rb) {
    constexpr int NW = THREADS / kWave;
    const float kInf = __builtin_inff();
    Thresh th{kInf, kInf, false, 0u, 0.0f};
    if (!md.need_cand) return th;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int32_t V = P.vocab;
    float x[8];
    bool in[8];
    load_sample<BF16>(rowp, V, x, in);
    // mean over finite sample values, fixed reduction order
    float sum = 0.0f;
    uint32_t nf = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const bool ok = in[i] && __builtin_isfinite(x[i]);
        sum += ok ? x[i] : 0.0f;
        nf += ok ? 1u : 0u;
    }
    sum = wave_sum_f32(sum);
    nf = wave_sum_u32(nf);
    if (lane == 0) {
        sh.fred[wave] = sum;
        sh.slot[rb][wave][0] = nf;
    }
    __syncthreads();
    float tot = 0.0f;
    uint32_t n = 0;
    for (int w = 0; w < NW; ++w) {
        tot += sh.fred[w];
        n += sh.slot[rb][w][0];
    }
    rb ^= 1;
    __syncthreads();
    const float mu = n ? tot / (float)n : 0.0f;
    float d2 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const bool ok = in[i] && __builtin_isfinite(x[i]);
        const float d = x[i] - mu;
        d2 += ok ? d * d : 0.0f;
    }
    d2 = wave_sum_f32(d2);
    if (lane == 0) sh.fred[wave] = d2;
    __syncthreads();
    float var = 0.0f;
    for (int w = 0; w < NW; ++w) var += sh.fred[w];
    __syncthreads();
    const float sigma = n ? sqrtf(var / (float)n) : 0.0f;
    const uint32_t ns = (uint32_t)min(V, kSampleN);
    th.n_s = ns;
    float t;
    if (n < 2) {
        t = -kInf;
    } else {
        float delta;
        const float cap = qrita_lut_k[lut_k_index(1.0f / (float)V)];
        if (md.K_t > 0) {
            delta = qrita_lut_k[lut_k_index((float)md.K_t / (float)V)];
        } else {
            // top-p: softmax mass of N(mu, sigma^2) above t is
            // 1 - Phi((t - mu)/sigma - sigma); keep at least p of it, less a margin.
            const float s = 1.0f - md.p;
            const float f = floorf((log2f(s) - QRITA_LUT_P_MIN) * QRITA_LUT_P_STEPS);
            const int i = (int)fminf(fmaxf(f, 0.0f), (float)(QRITA_LUT_P_N - 1));
            delta = fminf(sigma + qrita_lut_p[i] - 0.5f, cap);
        }
        t = mu + P.delta_scale * delta * sigma;
    }
    th.t = t;
    th.tc = t;
    // Miss prediction: the sample should hold about lambda = ns * K_t / V
    // values at or above the K_t-th largest logit of the row, and with the
    // table's factor-2 target about 2 * lambda values >= t. Fewer than
    // 1.25 * lambda + 2 suggests t lies above that logit (a truncation miss);
    // then collect down to a sample order statistic instead, so the miss is
    // served from the same single pass.
    if (md.K_t > 0 && n >= 2 && __builtin_isfinite(t)) {
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) c += (in[i] && x[i] >= t) ? 1u : 0u;
        c = wave_sum_u32(c);
        if (lane == 0) sh.slot[rb][wave][0] = c;
        __syncthreads();
        uint32_t ct = 0;
        for (int w = 0; w < NW; ++w) ct += sh.slot[rb][w][0];
        rb ^= 1;
        __syncthreads();
        const float lam = (float)ns * (float)md.K_t / (float)V;
        th.lambda = lam;
        if (lam >= 4.0f && (float)ct < 1.25f * lam + 2.0f) {
            const uint32_t r = min((uint32_t)ceilf(lam + 5.0f * sqrtf(lam) + 5.0f), ns);
            const float tfb = sample_rank_value<THREADS, BF16>(rowp, V, r, sh, rb);
            th.tc = fminf(t, tfb);
            th.predicted = true;
        }
    }
    if (P.force_miss) th.tc = kInf;
    return th;
}

// ---------------------------------------------------------------------------
// a3: the single streaming pass over one slice.
// ---------------------------------------------------------------------------

// Compact the survivors (f >= tc) of 16 logits per lane into the candidate
// stage: wavefront ballots count them, one LDS atomic per wave reserves
// space, mbcnt gives each lane its slot. Logit j of this lane has vocabulary
// index idx0 + (j / VE) * vstride + (j % VE). Survivors past the stage go
// straight to the row list (with their key, for the list's max).
template <int THREADS, bool BF16, bool REST, int VE>
QRITA_DEV void consume16(const Params& P, int64_t row, const float f[16], uint32_t valid, uint32_t idx0,
                         uint32_t vstride, float tc, Shared& sh, uint64_t& rest, uint32_t& spill_kmax) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const bool v = (valid >> j) & 1u;
        const bool s = v && f[j] >= tc;
        tot += (uint32_t)__popcll(__ballot(s));
        if (REST && v && !s) rest += fx_from_unit_f32(__expf(f[j] - tc));
    }
    if (tot == 0) return;
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&sh.ncand, tot);
    base = readlane(base, 0);
    const uint32_t cap = (uint32_t)P.stage_cap;
    const uint32_t spill_from = base > cap ? base : cap;
    uint32_t gbase = 0;
    if (base + tot > cap) {
        const uint32_t nover = base + tot - spill_from;
        if (lane == 0) gbase = atomicAdd(&P.hdr[row * H_WORDS + H_LIST], nover);
        gbase = readlane(gbase, 0);
    }
    uint64_t* a = lds_cands();
    uint32_t run = base;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const bool s = ((valid >> j) & 1u) && f[j] >= tc;
        const uint64_t b = __ballot(s);
        if (b) {
            if (s) {
                const uint32_t pos = run + lanes_below(b);
                const uint32_t bits = __float_as_uint(f[j]);
                const uint32_t idx = idx0 + (uint32_t)(j / VE) * vstride + (uint32_t)(j % VE);
                if (pos < cap) {
                    a[pos] = ((uint64_t)bits << 32) | idx;
                } else {
                    const uint32_t gp = gbase + (pos - spill_from);
                    const uint32_t key = f32_key(bits);
                    spill_kmax = key > spill_kmax ? key : spill_kmax;
                    if (gp < (uint32_t)P.list_cap)
                        P.glist[row * (int64_t)P.list_stride + gp] = make_cand(key, idx);
                    else
                        atomicOr(&sh.flags, 1u);
                }
            }
            run += (uint32_t)__popcll(b);
        }
    }
}

template <int THREADS, bool BF16, bool REST>
QRITA_DEV void stream_slice(const Params& P, int64_t row, int64_t e0, int64_t e1, float tc, uint8_t fill,
                            Shared& sh, uint64_t& rest, uint32_t& spill_kmax) {
    const int64_t roff = row * (int64_t)P.vocab;
    const void* rowp = row_ptr<BF16>(P, row);
    uint8_t* mrow = P.mask ? P.mask + roff : nullptr;
    const int tid = threadIdx.x;
    // head: up to 15 logits before the first 16-element-aligned position
    int64_t a = e0 + ((16 - ((roff + e0) & 15)) & 15);
    if (a > e1) a = e1;
    if (a > e0) {
        float f[16];
        uint32_t valid = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) f[j] = 0.0f;
        const int64_t e = e0 + tid;
        if (e < a) {
            f[0] = load_value<BF16>(rowp, e);
            valid = 1;
            if (mrow) mrow[e] = fill;
        }
        if (tid < kWave)
            consume16<THREADS, BF16, REST, 16>(P, row, f, valid, (uint32_t)e, 0u, tc, sh, rest, spill_kmax);
    }
    constexpr int VE = BF16 ? 8 : 4;  // logits per 16-byte vector
    constexpr int NV = 16 / VE;       // vectors per thread per tile
    constexpr int TB = THREADS * 16;  // logits per tile
    const uint64_t fill8 = 0x0101010101010101ull * fill;
    for (int64_t tile = a; tile < e1; tile += TB) {
        float f[16];
        uint32_t valid = 0;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int64_t e = tile + (int64_t)q * THREADS * VE + (int64_t)tid * VE;
            if (e + VE <= e1) {
                if (BF16) {
                    const uint4 w = *(const uint4*)((const uint16_t*)rowp + e);
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        f[q * 8 + 2 * r] = __uint_as_float(ws[r] << 16);
                        f[q * 8 + 2 * r + 1] = __uint_as_float(ws[r] & 0xFFFF0000u);
                    }
                } else {
                    const float4 w = *(const float4*)((const float*)rowp + e);
                    f[q * 4 + 0] = w.x;
                    f[q * 4 + 1] = w.y;
                    f[q * 4 + 2] = w.z;
                    f[q * 4 + 3] = w.w;
                }
                valid |= ((1u << VE) - 1u) << (q * VE);
                if (mrow) {
                    if (BF16)
                        *(uint64_t*)(mrow + e) = fill8;
                    else
                        *(uint32_t*)(mrow + e) = (uint32_t)fill8;
                }
            } else {
#pragma unroll
                for (int r = 0; r < VE; ++r) {
                    const int64_t er = e + r;
                    if (er < e1) {
                        f[q * VE + r] = load_value<BF16>(rowp, er);
                        valid |= 1u << (q * VE + r);
                        if (mrow) mrow[er] = fill;
                    } else {
                        f[q * VE + r] = 0.0f;
                    }
                }
            }
        }
        consume16<THREADS, BF16, REST, VE>(P, row, f, valid, (uint32_t)(tile + (int64_t)tid * VE),
                                           (uint32_t)(THREADS * VE), tc, sh, rest, spill_kmax);
    }
}

// Pass 1: one workgroup per (row, slice). Workgroup g runs on XCD g mod 8;
// rows are dealt so that all slices of row r share XCD r mod 8 and therefore
// one L2, which also holds the row list when the row's tail reads it.
template <int THREADS, bool BF16>
__global__ __launch_bounds__(THREADS) void pass1_kernel(Params P) {
    __shared__ Shared sh;
    int rb = 0;
    const uint32_t g = blockIdx.x;
    const uint32_t xcd = g & 7u, jj = g >> 3;
    const uint32_t rloc = jj / (uint32_t)P.slices, slice = jj % (uint32_t)P.slices;
    const int64_t row = (int64_t)rloc * 8 + xcd;
    if (row >= P.batch) return;
    const int32_t V = P.vocab;
    const int64_t roff = row * (int64_t)V;
    const void* rowp = row_ptr<BF16>(P, row);
    uint32_t* hdr = P.hdr + row * H_WORDS;
    const RowMode md = row_mode(P, row);
    if (threadIdx.x == 0) {
        sh.ncand = 0;
        sh.flags = 0;
    }
    // a2: every slice computes the same threshold from the same sample
    const Thresh th = compute_threshold<THREADS, BF16>(P, md, rowp, sh, rb);
    if (slice == 0 && threadIdx.x == 0) {
        hdr[H_T] = __float_as_uint(th.t);
        hdr[H_TC] = __float_as_uint(th.tc);
        hdr[H_PRED] = th.predicted ? 1u : 0u;
        hdr[H_LAMBDA] = __float_as_uint(th.lambda);
        hdr[H_NS] = th.n_s;
    }
    __syncthreads();
    // a3: this workgroup's slice; slices after the first start 16-aligned
    const int64_t A = (16 - (roff & 15)) & 15;
    int64_t e0 = slice == 0 ? 0 : A + (int64_t)slice * P.slice_len;
    int64_t e1 = A + (int64_t)(slice + 1) * P.slice_len;
    if (slice + 1 == (uint32_t)P.slices || e1 > V) e1 = V;
    if (e0 > V) e0 = V;
    const uint8_t fill = md.keep_all ? 1 : 0;
    const bool rest_on = md.topp && !md.topk;
    uint64_t rest = 0;
    uint32_t kmax = 0;
    if (rest_on)
        stream_slice<THREADS, BF16, true>(P, row, e0, e1, th.tc, fill, sh, rest, kmax);
    else
        stream_slice<THREADS, BF16, false>(P, row, e0, e1, th.tc, fill, sh, rest, kmax);
    __syncthreads();
    // publish: the staged candidates go to the row list in one reservation
    const uint32_t nst = min(sh.ncand, (uint32_t)P.stage_cap);
    if (threadIdx.x == 0) sh.u32[0] = nst ? atomicAdd(&hdr[H_LIST], nst) : 0u;
    __syncthreads();
    const uint32_t gb = sh.u32[0];
    uint64_t* a = lds_cands();
    uint64_t* lst = P.glist + row * (int64_t)P.list_stride;
    bool over = false;
    for (uint32_t i = threadIdx.x; i < nst; i += THREADS) {
        const uint64_t r = a[i];
        const uint32_t key = f32_key((uint32_t)(r >> 32));
        kmax = key > kmax ? key : kmax;
        if (gb + i < (uint32_t)P.list_cap)
            lst[gb + i] = make_cand(key, (uint32_t)r);
        else
            over = true;
    }
    if (over) atomicOr(&sh.flags, 1u);
    uint32_t d0 = 0, d1 = 0;
    block_sum_min_max<THREADS>(d0, d1, kmax, rest, sh, rb);
    if (threadIdx.x == 0) {
        if (kmax) atomicMax(&hdr[H_KMAX], kmax);
        if (rest) atomicAdd((unsigned long long*)(hdr + H_REST), (unsigned long long)rest);
        if (sh.flags) atomicOr(&hdr[H_FLAGS], 1u);
    }
}

// Re-collect the row's candidates >= tr into the per-row list (full-row
// fallback after a miss). Returns the number of candidates (capped at the
// list capacity); *overflow is set when the list was too small, *kmax_out is
// the largest key and *rest_out the fixed-point mass (relative to tr) of the
// logits below tr.
template <int THREADS, bool BF16>
QRITA_DEV uint32_t collect_row(const Params& P, int64_t row, float tr, bool rest_on, Shared& sh, int& rb,
                               uint64_t& rest_out, uint32_t& kmax_out, bool& overflow) {
    const int32_t V = P.vocab;
    const void* rowp = row_ptr<BF16>(P, row);
    uint64_t* lst = P.glist + row * (int64_t)P.list_stride;
    __syncthreads();
    if (threadIdx.x == 0) {
        sh.gather_n = 0;
        sh.flags = 0;
    }
    __syncthreads();
    const uint32_t lane = threadIdx.x & (kWave - 1);
    uint64_t rest = 0;
    uint32_t kmax = 0;
    for (int64_t base = 0; base < V; base += THREADS) {
        const int64_t e = base + threadIdx.x;
        const float f = e < V ? load_value<BF16>(rowp, e) : 0.0f;
        const bool s = e < V && f >= tr;
        if (rest_on && e < V && !s) rest += fx_from_unit_f32(__expf(f - tr));
        const uint64_t b = __ballot(s);
        if (b) {
            uint32_t g = 0;
            if (lane == 0) g = atomicAdd(&sh.gather_n, (uint32_t)__popcll(b));
            g = readlane(g, 0);
            if (s) {
                const uint32_t pos = g + lanes_below(b);
                const uint32_t key = f32_key(__float_as_uint(f));
                kmax = key > kmax ? key : kmax;
                if (pos < (uint32_t)P.list_cap)
                    lst[pos] = make_cand(key, (uint32_t)e);
                else
                    atomicOr(&sh.flags, 1u);
            }
        }
    }
    uint32_t d0 = 0, d1 = 0;
    block_sum_min_max<THREADS>(d0, d1, kmax, rest, sh, rb);
    __syncthreads();
    rest_out = rest;
    kmax_out = kmax;
    const uint32_t cnt = sh.gather_n;
    overflow = sh.flags != 0 || cnt > (uint32_t)P.list_cap;
    __syncthreads();
    return cnt < (uint32_t)P.list_cap ? cnt : (uint32_t)P.list_cap;
}

// Tail: one workgroup per row, after pass 1 has completed for every row. The
// row's candidates are held in LDS (up to tail_cap of them).
template <int THREADS, bool BF16>
__global__ __launch_bounds__(THREADS) void tail_kernel(Params P) {
    __shared__ Shared sh;
    int rb = 0;
    const int64_t row = blockIdx.x;
    if (row >= P.batch) return;
    const int32_t V = P.vocab;
    const void* rowp = row_ptr<BF16>(P, row);
    uint32_t* hdr = P.hdr + row * H_WORDS;
    uint64_t* lst = P.glist + row * (int64_t)P.list_stride;
    const RowMode md = row_mode(P, row);
    const float t = __uint_as_float(hdr[H_T]);
    const float tc = __uint_as_float(hdr[H_TC]);
    const uint32_t nlist = hdr[H_LIST];
    const uint32_t kmax = hdr[H_KMAX];
    const bool overflow = hdr[H_FLAGS] != 0 || nlist > (uint32_t)P.list_cap;
    const uint64_t rest = (uint64_t)hdr[H_REST] | ((uint64_t)hdr[H_REST + 1] << 32);
    const float lambda = __uint_as_float(hdr[H_LAMBDA]);
    const uint32_t ns_h = hdr[H_NS];
    const bool predicted = hdr[H_PRED] != 0;
    uint64_t* a = lds_cands();

    TailDiag dg{-1, 0};
    int path = 0;
    bool done = false;
    if (!md.need_cand) {
        if (P.out_count && threadIdx.x == 0) P.out_count[row] = V;
        done = true;
    } else {
        // every candidate has z >= tc, so its key exceeds key(tc) - 1
        const int64_t key_lo = (int64_t)f32_key(__float_as_uint(tc)) - 1;
        if (!overflow) {
            if (nlist <= (uint32_t)P.tail_cap) {
                constexpr int U = 8;
                for (uint32_t base = 0; base < nlist; base += THREADS * U) {
                    uint64_t c[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const uint32_t i = base + (uint32_t)u * THREADS + threadIdx.x;
                        c[u] = i < nlist ? lst[i] : 0ull;
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const uint32_t i = base + (uint32_t)u * THREADS + threadIdx.x;
                        if (i < nlist) a[i] = c[u];
                    }
                }
                __syncthreads();
                const LdsSrc<THREADS> src{nlist};
                done = finish_row<THREADS, false>(P, row, md, src, key_lo, kmax, rest, tc, t, sh, rb, dg);
            } else {
                path = 1;
                const MemSrc<THREADS, false, BF16> src{lst, nullptr, nlist};
                done = finish_row<THREADS, false>(P, row, md, src, key_lo, kmax, rest, tc, t, sh, rb, dg);
            }
        }
        // a4 fallback: re-collect with lower thresholds taken from the sample's
        // order statistics, then search the full row.
        if (!done) {
            path = 2;
            const uint32_t ns = ns_h ? ns_h : (uint32_t)min(V, kSampleN);
            const float r0 = md.K_t > 0 ? ceilf(lambda + 5.0f * sqrtf(lambda) + 5.0f) : 64.0f;
            float prev = tc;
            for (int attempt = 1; attempt <= 8 && !done; ++attempt) {
                const float rr = r0 * (float)(1u << (2 * attempt));
                float tr;
                if (rr < (float)ns)
                    tr = sample_rank_value<THREADS, BF16>(rowp, V, (uint32_t)rr, sh, rb);
                else if (prev > -__builtin_inff())
                    tr = -__builtin_inff();
                else
                    break;
                if (!(tr < prev)) continue;
                prev = tr;
                uint64_t rest2 = 0;
                uint32_t kmax2 = 0;
                bool ovf = false;
                const uint32_t cnt =
                    collect_row<THREADS, BF16>(P, row, tr, md.topp && !md.topk, sh, rb, rest2, kmax2, ovf);
                if (ovf) break;
                const MemSrc<THREADS, false, BF16> src{lst, nullptr, cnt};
                done = finish_row<THREADS, false>(P, row, md, src, (int64_t)f32_key(__float_as_uint(tr)) - 1,
                                                  kmax2, rest2, tr, t, sh, rb, dg);
                if (tr == -__builtin_inff()) break;
            }
            if (!done) {
                path = 3;
                uint32_t kr = 0, d0 = 0, d1 = 0;
                uint64_t d2 = 0;
                for (int64_t e = threadIdx.x; e < V; e += THREADS) {
                    const uint32_t key = f32_key(__float_as_uint(load_value<BF16>(rowp, e)));
                    kr = key > kr ? key : kr;
                }
                block_sum_min_max<THREADS>(d0, d1, kr, d2, sh, rb);
                const MemSrc<THREADS, true, BF16> src{nullptr, rowp, (uint32_t)V};
                done = finish_row<THREADS, true>(P, row, md, src, -1, kr, 0ull, 0.0f, t, sh, rb, dg);
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 0; w < H_WORDS; ++w) hdr[w] = 0u;
        if (P.diag) {
            int32_t* d = P.diag + row * 8;
            d[0] = (int32_t)__float_as_uint(t);
            d[1] = (int32_t)__float_as_uint(tc);
            d[2] = dg.n_t;
            d[3] = (int32_t)nlist;
            d[4] = path;
            d[5] = (md.K_t > 0 && dg.n_t >= 0) ? (dg.n_t >= (int32_t)md.K_t) : (path <= 1 ? 1 : 0);
            d[6] = dg.iters;
            d[7] = predicted ? 1 : 0;
        }
    }
}

__global__ void zero_fill_kernel(uint32_t* p, uint64_t words) {
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < words;
         i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace qrita
