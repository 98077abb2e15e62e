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
//   tail (one workgroup per row, see tail_kernel; the row's candidates are
//   held in registers while the searches run):
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

#include <type_traits>

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
    int32_t tail_cap;    // tail: largest list searched in registers
    int32_t tail_alloc;  // tail: LDS entries for sorting kept sets (indices follow)
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

constexpr int kTieDirect = 256;  // tie groups up to this size are ranked directly
constexpr int kTailR = 32;       // tail: candidates per thread held in registers
constexpr int kWaveR = 32;       // tail, one-wave mode: candidates per lane (2048 per row)

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kHistBins = 256;  // pass 1: sample histogram for the miss prediction

struct Shared {
    alignas(16) uint32_t slot[2][kMaxWaves][16];  // per-wave partial records, double-buffered
    alignas(16) uint32_t ties[kTieDirect + 4];
    uint32_t hist[kHistBins];
    float fred[2 * kMaxWaves];
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

// ---------------------------------------------------------------------------
// Tail block combination (NT threads, NW = NT / 64 waves). Each wave reduces
// its lanes with DPP; lane 0 stores the wave's record in LDS; after one
// barrier every lane reads all NW records (broadcast reads) and reduces them,
// so every thread holds the block's value without a second barrier (the two
// record buffers alternate).
// ---------------------------------------------------------------------------
// UNIFORM: the inputs are already wave totals.
template <int NT, bool UNIFORM = false>
QRITA_DEV void comb_sum3(uint32_t g[3], Shared& sh, int& rb) {
    constexpr int NW = NT / kWave;
    const uint32_t w0 = UNIFORM ? g[0] : wave_sum_u32(g[0]);
    const uint32_t w1 = UNIFORM ? g[1] : wave_sum_u32(g[1]);
    const uint32_t w2 = UNIFORM ? g[2] : wave_sum_u32(g[2]);
    if (NW == 1) {
        g[0] = w0;
        g[1] = w1;
        g[2] = w2;
        return;
    }
    const uint32_t lane = tid_here() & (kWave - 1), wave = wave_base_here() / kWave;
    if (lane == 0) *(uint4*)sh.slot[rb][wave] = make_uint4(w0, w1, w2, 0u);
    __syncthreads();
    uint32_t a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint4 q = *(const uint4*)sh.slot[rb][w];
        a0 += q.x;
        a1 += q.y;
        a2 += q.z;
    }
    g[0] = a0;
    g[1] = a1;
    g[2] = a2;
    rb ^= 1;
}

template <int NT, bool UNIFORM = false>
QRITA_DEV void comb_sum3_64(uint64_t m[3], uint32_t g[3], Shared& sh, int& rb) {
    constexpr int NW = NT / kWave;
    uint32_t gw[3];
    uint64_t mw[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        gw[j] = UNIFORM ? g[j] : wave_sum_u32(g[j]);
        mw[j] = UNIFORM ? m[j] : wave_sum_u64(m[j]);
    }
    if (NW == 1) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            g[j] = gw[j];
            m[j] = mw[j];
        }
        return;
    }
    const uint32_t lane = tid_here() & (kWave - 1), wave = wave_base_here() / kWave;
    if (lane == 0) {
        uint4* s = (uint4*)sh.slot[rb][wave];
        s[0] = make_uint4(gw[0], gw[1], gw[2], 0u);
        s[1] = make_uint4((uint32_t)mw[0], (uint32_t)(mw[0] >> 32), (uint32_t)mw[1], (uint32_t)(mw[1] >> 32));
        s[2] = make_uint4((uint32_t)mw[2], (uint32_t)(mw[2] >> 32), 0u, 0u);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        g[j] = 0;
        m[j] = 0;
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint4* s = (const uint4*)sh.slot[rb][w];
        const uint4 a = s[0], b = s[1], c = s[2];
        g[0] += a.x;
        g[1] += a.y;
        g[2] += a.z;
        m[0] += (uint64_t)b.x | ((uint64_t)b.y << 32);
        m[1] += (uint64_t)b.z | ((uint64_t)b.w << 32);
        m[2] += (uint64_t)c.x | ((uint64_t)c.y << 32);
    }
    rb ^= 1;
}

// Per-lane (mn, N, mx) -> block (smallest value, its multiplicity, largest
// value of the second set).
template <int NT>
QRITA_DEV void comb_minmax(uint32_t& mn, uint32_t& N, uint32_t& mx, Shared& sh, int& rb) {
    constexpr int NW = NT / kWave;
    const uint32_t wm = wave_min_u32(mn);
    const uint32_t wn = wave_sum_u32(mn == wm ? N : 0u);
    const uint32_t wx = wave_max_u32(mx);
    if (NW == 1) {
        mn = wm;
        N = wn;
        mx = wx;
        return;
    }
    const uint32_t lane = tid_here() & (kWave - 1), wave = wave_base_here() / kWave;
    if (lane == 0) *(uint4*)sh.slot[rb][wave] = make_uint4(wm, wn, wx, 0u);
    __syncthreads();
    uint4 q[NW];
    uint32_t bm = 0xFFFFFFFFu, bx = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        q[w] = *(const uint4*)sh.slot[rb][w];
        bm = q[w].x < bm ? q[w].x : bm;
        bx = q[w].z > bx ? q[w].z : bx;
    }
    uint32_t bn = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) bn += q[w].x == bm ? q[w].y : 0u;
    mn = bm;
    N = bn;
    mx = bx;
    rb ^= 1;
}

template <int NT>
QRITA_DEV void comb_min2(uint32_t& a, uint32_t& b, Shared& sh, int& rb) {
    constexpr int NW = NT / kWave;
    const uint32_t wa = wave_min_u32(a), wb = wave_min_u32(b);
    if (NW == 1) {
        a = wa;
        b = wb;
        return;
    }
    const uint32_t lane = tid_here() & (kWave - 1), wave = wave_base_here() / kWave;
    if (lane == 0) *(uint2*)sh.slot[rb][wave] = make_uint2(wa, wb);
    __syncthreads();
    uint32_t ma = 0xFFFFFFFFu, mb = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint2 q = *(const uint2*)sh.slot[rb][w];
        ma = q.x < ma ? q.x : ma;
        mb = q.y < mb ? q.y : mb;
    }
    a = ma;
    b = mb;
    rb ^= 1;
}

template <int NT>
QRITA_DEV uint64_t comb_sum64(uint64_t v, Shared& sh, int& rb) {
    uint64_t m[3] = {v, 0ull, 0ull};
    uint32_t g[3] = {0u, 0u, 0u};
    comb_sum3_64<NT>(m, g, sh, rb);
    return m[0];
}

template <int NT>
QRITA_DEV uint32_t comb_sum32(uint32_t v, Shared& sh, int& rb) {
    uint32_t g[3] = {v, 0u, 0u};
    comb_sum3<NT>(g, sh, rb);
    return g[0];
}

// ---------------------------------------------------------------------------
// Candidate sources of the tail. A source hands every candidate to a visitor
// as (key, low, r): key 0 marks an empty slot or a candidate outside the
// current set (every real key is nonzero); low is the complemented
// vocabulary index (passed only to visits that ask for it: duplicate
// resolution, the mask and the index output); r is a register slot (RegSet
// only).
// restrict_to(B) shrinks the set to the candidates c >= B; prepare_mass(m)
// makes mass_at() return a candidate's softmax mass exp(z - m) relative to
// the maximum m (0 outside the set).
//
// RegSet keeps up to NT * R candidate keys in registers, slot (r, thread t)
// holding candidate r * NT + t, so every count evaluation reads registers
// only; the complemented indices and, during the mass search, the softmax
// masses wait in LDS under the same slot numbering. Slot rows past the last
// candidate are skipped per wave.
// ---------------------------------------------------------------------------
// Exclusive prefix over the waves of a workgroup of per-wave counts c (wave
// uniform): returns the sum over the lower waves and sets total to the sum
// over all of them.
template <int NT>
QRITA_DEV uint32_t wave_prefix(uint32_t c, uint32_t& total, Shared& sh, int& rb) {
    constexpr int NW = NT / kWave;
    if (NW == 1) {
        total = c;
        return 0u;
    }
    const uint32_t lane = tid_here() & (kWave - 1), wave = wave_base_here() / kWave;
    if (lane == 0) sh.slot[rb][wave][0] = c;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t q = sh.slot[rb][w][0];
        before += (uint32_t)w < wave ? q : 0u;
        all += q;
    }
    rb ^= 1;
    total = all;
    return before;
}

// Calls f(std::integral_constant<int, C>) for C = B .. E-1 (compile-time
// register indices).
template <int B, int E, class F>
QRITA_DEV void unroll_rows(F& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        unroll_rows<B + 1, E>(f);
    }
}

template <int NT, int R>
struct RegSet {
    static constexpr int kChunk = 8;  // slot rows handled per guard
    static_assert(R % kChunk == 0, "slot rows come in chunks");
    uint32_t key[R];
    uint32_t* lows;    // LDS, [R * NT]
    float* em;         // LDS, [R * NT]: exp(z - m) after prepare_mass
    uint32_t nslots;   // slots r * NT + t < nslots may hold candidates

    // number of slot rows holding candidates of this thread's wave (uniform)
    QRITA_DEV int rows_here() const {
        const uint32_t wb = wave_base_here();
        const uint32_t ns = __builtin_amdgcn_readfirstlane(nslots);
        return wb < ns ? (int)((ns - wb + NT - 1) / NT) : 0;
    }

    // f(row) for every row of the chunks that hold this wave's candidates:
    // one uniform branch per chunk of 8 rows, rows past the last candidate
    // inside the last chunk hold key 0.
    template <int C, class F>
    QRITA_DEV void chunks_from(F& f, int nr) const {
        if constexpr (C < R) {
            if (C < nr) {
                unroll_rows<C, C + kChunk>(f);
                chunks_from<C + kChunk>(f, nr);
            }
        }
    }
    template <class F>
    QRITA_DEV void for_rows(F&& f) const {
        chunks_from<0>(f, rows_here());
    }

    // f(key, low, r) for every visited slot; with LOWS the complemented
    // indices are first read from LDS in one batch (else low is 0).
    template <bool LOWS, class F>
    QRITA_DEV void visit(F&& f) const {
        if constexpr (LOWS) {
            const uint32_t* lp = lows + tid_here();
            uint32_t lw[R];
            for_rows([&](auto rc) {
                constexpr int r = decltype(rc)::value;
                lw[r] = lp[r * NT];
            });
            for_rows([&](auto rc) {
                constexpr int r = decltype(rc)::value;
                f(key[r], lw[r], r);
            });
        } else {
            for_rows([&](auto rc) {
                constexpr int r = decltype(rc)::value;
                f(key[r], 0u, r);
            });
        }
    }
    QRITA_DEV float mass_at(int r, uint32_t) const { return em[tid_here() + r * NT]; }

    // the n candidates of a row list, in list order: every load is issued
    // before the first index is stored
    QRITA_DEV void load(const uint64_t* lst, uint32_t n) {
        nslots = n;
        const uint32_t t = tid_here();
        uint32_t lw[R];
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const uint32_t i = (uint32_t)r * NT + t;
            const uint64_t c = lst[i < n ? i : n - 1];
            key[r] = i < n ? cand_key(c) : 0u;
            lw[r] = cand_low(c);
        });
        uint32_t* lp = lows + t;
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            lp[r * NT] = lw[r];
        });
        block_sync<NT>();
    }
    // Keys through LDS (slot i at kb[i]), to hand a set to a different number
    // of threads; the indices stay in `lows`, which every layout indexes by
    // slot.
    QRITA_DEV void store_keys(uint32_t* kb) const {
        const uint32_t t = tid_here();
        const uint32_t ns = nslots;
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const uint32_t i = (uint32_t)r * NT + t;
            if (i < ns) kb[i] = key[r];
        });
    }
    QRITA_DEV void load_keys(const uint32_t* kb, uint32_t n) {
        nslots = n;
        const uint32_t t = tid_here();
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const uint32_t i = (uint32_t)r * NT + t;
            key[r] = i < n ? kb[i] : 0u;
        });
    }

    // The same from candidates already loaded into pre[r] (slot r * NT + t).
    QRITA_DEV void load_from(const uint64_t (&pre)[R], uint32_t n) {
        nslots = n;
        const uint32_t t = tid_here();
        uint32_t* lp = lows + t;
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const uint32_t i = (uint32_t)r * NT + t;
            key[r] = i < n ? cand_key(pre[r]) : 0u;
            lp[r * NT] = cand_low(pre[r]);
        });
        block_sync<NT>();
    }
    QRITA_DEV void restrict_to(uint64_t B) {
        const uint32_t bk = cand_key(B), bl = cand_low(B);
        const uint32_t* lp = lows + tid_here();
        uint32_t lw[R];
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            lw[r] = lp[r * NT];
        });
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const uint32_t k = key[r];
            const bool keep = k > bk || (k == bk && lw[r] >= bl);
            key[r] = keep ? k : 0u;
        });
    }
    // Move the candidates still in the set (key != 0) to the first slots,
    // keeping their slot order, through buf (room for cap pairs); nothing
    // moves when more than cap remain. Later visits then skip the emptied
    // slot rows.
    QRITA_DEV void compact(uint32_t* buf, uint32_t cap, Shared& sh, int& rb) {
        uint32_t c = 0;
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            c += (uint32_t)__popcll(__ballot(key[r] != 0u));
        });
        uint32_t total = 0;
        uint32_t run = wave_prefix<NT>(c, total, sh, rb);
        if (total > cap) return;
        const uint32_t t = tid_here();
        const uint32_t* lp = lows + t;
        uint32_t lw[R];
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            lw[r] = lp[r * NT];
        });
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const uint32_t k = key[r];
            const uint64_t b = __ballot(k != 0u);
            if (k != 0u) {
                const uint32_t pos = run + lanes_below(b);
                buf[pos] = k;
                buf[cap + pos] = lw[r];
            }
            run += (uint32_t)__popcll(b);
        });
        block_sync<NT>();
        nslots = total;
        uint32_t* lq = lows + t;
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const uint32_t i = (uint32_t)r * NT + t;
            key[r] = i < total ? buf[i] : 0u;
            lw[r] = i < total ? buf[cap + i] : 0u;
        });
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            lq[r * NT] = lw[r];
        });
        block_sync<NT>();
    }

    QRITA_DEV void prepare_mass(float m) {
        float* ep = em + tid_here();
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            ep[r * NT] = key[r] ? mass_f32(key[r], m) : 0.0f;
        });
    }
    static constexpr bool kRegs = true;
};

// MemSrc streams the candidates from memory on every visit: the row list, or
// (ROW) the row's logits themselves for the full-row fallback (§1). Four
// loads per thread are kept in flight.
template <int NT, bool ROW, bool BF16>
struct MemSrc {
    const uint64_t* p;  // candidate array (global)
    const void* row;    // row logits (ROW)
    uint32_t n;
    uint64_t filter;
    float m;

    QRITA_DEV uint64_t get(uint32_t i) const {
        if (ROW) return make_cand(f32_key(__float_as_uint(load_value<BF16>(row, i))), i);
        return p[i];
    }
    template <bool LOWS, class F>
    QRITA_DEV void visit(F&& f) const {
        constexpr int U = 4;
        const uint32_t t = tid_here();
        for (uint32_t base = 0; base < n; base += NT * U) {
            uint64_t c[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = base + (uint32_t)u * NT + t;
                c[u] = i < n ? get(i) : 0ull;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = base + (uint32_t)u * NT + t;
                const bool ok = i < n && c[u] >= filter;
                f(ok ? cand_key(c[u]) : 0u, cand_low(c[u]), 0);
            }
        }
    }
    QRITA_DEV float mass_at(int, uint32_t key) const { return key ? mass_f32(key, m) : 0.0f; }
    QRITA_DEV void restrict_to(uint64_t B) { filter = B > filter ? B : filter; }
    QRITA_DEV void prepare_mass(float mm) { m = mm; }
    static constexpr bool kRegs = false;
};

// Three pivots at 25/50/75 % of the open range (lo, hi) of field values
// (hi - lo >= 2): of the key range (mode 0), or of the value range (mode 1,
// keys only, finite ends). Pivots are distinct and lie strictly inside.
QRITA_DEV void make_pivots(uint32_t lo, uint32_t hi, int mode, int field, uint32_t piv[3]) {
    const uint32_t span = hi - lo;
    bool done = false;
    if (mode == 1 && field == 0) {
        const float a = key_value(lo), b = key_value(hi);
        if (__builtin_isfinite(a) && __builtin_isfinite(b)) {
            uint32_t prev = lo;
#pragma unroll
            for (int j = 1; j <= 3; ++j) {
                const double v = (double)a + ((double)b - (double)a) * (0.25 * j);
                uint32_t kk = f32_key(__float_as_uint((float)v));
                kk = kk <= prev ? prev + 1 : kk;
                kk = kk >= hi ? hi - 1 : kk;
                kk = kk <= lo ? lo + 1 : kk;
                piv[j - 1] = kk;
                prev = kk;
            }
            done = true;
        }
    }
    if (!done) {
#pragma unroll
        for (int j = 1; j <= 3; ++j) {
            uint32_t pj = lo + (uint32_t)(((uint64_t)span * (uint32_t)j) >> 2);
            pj = pj <= lo ? lo + 1 : pj;
            pj = pj >= hi ? hi - 1 : pj;
            piv[j - 1] = pj;
        }
    }
}

// One pivot evaluation. Phase A: for the three pivots, G = #{x > pivot} by
// wavefront ballot/popcount (and, for the mass search, M = mass of x above
// the pivot). Phase B: only the highest pivot j* whose count (mass) still
// reaches the target can end the search or move its lower end, so z_mn and
// N_zmn are formed for that pivot alone; pivots ascend and G, M do not
// increase, so j* is known after phase A. Phase B also takes, for the pivot
// just above j*, the largest value at or below it (z_mx): nothing lies
// between z_mx and that pivot, so z_mx can become the new upper end,
// mirroring the jump of the lower end to z_mn.
struct Eval {
    uint32_t G[3];
    uint64_t M[3];
    int js;  // -1: no pivot reaches the target
    uint32_t mn, N;
    uint32_t mx;  // largest value <= the pivot above j* (0 if none)
};

QRITA_DEV uint32_t sel3(int j, const uint32_t x[3]) { return j == 2 ? x[2] : (j == 1 ? x[1] : x[0]); }
QRITA_DEV uint64_t sel3(int j, const uint64_t x[3]) { return j == 2 ? x[2] : (j == 1 ? x[1] : x[0]); }

// Field 0 searches keys; field 1 searches the complemented indices of the
// candidates whose key is v_eq (duplicate resolution).
template <int FIELD>
QRITA_DEV uint32_t field_of(uint32_t key, uint32_t low, uint32_t v_eq) {
    if (FIELD == 0) return key;
    return key == v_eq ? low : 0u;
}

template <int NT, int FIELD, bool MASS, class S>
QRITA_DEV Eval eval_pivots(const S& src, uint32_t v_eq, const uint32_t piv[3], uint32_t K, double T,
                           Shared& sh, int& rb) {
    Eval E;
    // phase A: per-lane counts (and masses) above each pivot. A register
    // set holds at most 32 slots per lane, so its masses are summed as 32-bit
    // halves; a streamed source sums them in 64 bits.
    uint32_t g[3] = {0u, 0u, 0u};
    uint32_t mh[3] = {0u, 0u, 0u}, ml[3] = {0u, 0u, 0u};
    uint64_t mm[3] = {0ull, 0ull, 0ull};
    const uint32_t p0 = piv[0], p1 = piv[1], p2 = piv[2];
    src.template visit<FIELD == 1>([&](uint32_t key, uint32_t low, int r) {
        const uint32_t f = field_of<FIELD>(key, low, v_eq);
        const uint32_t b0 = gt01(f, p0), b1 = gt01(f, p1), b2 = gt01(f, p2);
        g[0] += b0;
        g[1] += b1;
        g[2] += b2;
        if (MASS) {
            if (S::kRegs) {
                uint32_t eh, el;
                fx_split(src.mass_at(r, key), eh, el);
                mh[0] += __umul24(b0, eh);
                ml[0] += __umul24(b0, el);
                mh[1] += __umul24(b1, eh);
                ml[1] += __umul24(b1, el);
                mh[2] += __umul24(b2, eh);
                ml[2] += __umul24(b2, el);
            } else {
                const uint64_t e = fx_from_unit_f32(src.mass_at(r, key));
                mm[0] += b0 ? e : 0ull;
                mm[1] += b1 ? e : 0ull;
                mm[2] += b2 ? e : 0ull;
            }
        }
    });
    if (MASS) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            g[j] = wave_sum_u32(g[j]);
            mm[j] = S::kRegs ? wave_sum_split(mh[j], ml[j]) : wave_sum_u64(mm[j]);
        }
        comb_sum3_64<NT, true>(mm, g, sh, rb);
        E.js = (double)mm[2] >= T ? 2 : ((double)mm[1] >= T ? 1 : ((double)mm[0] >= T ? 0 : -1));
    } else {
        comb_sum3<NT, false>(g, sh, rb);
        E.js = g[2] >= K ? 2 : (g[1] >= K ? 1 : (g[0] >= K ? 0 : -1));
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        E.G[j] = g[j];
        E.M[j] = mm[j];
    }
    // phase B: z_mn above pivot j* as the smallest f - (pj + 1) (values at or
    // below pj wrap above every value above it), z_mx below the next pivot
    // as the smallest pu - f
    const uint32_t pj1 = (E.js >= 0 ? sel3(E.js, piv) : 0xFFFFFFFEu) + 1u;
    const uint32_t pu = E.js < 2 ? sel3(E.js + 1, piv) : 0xFFFFFFFFu;
    uint32_t du = 0xFFFFFFFFu, dv = 0xFFFFFFFFu;
    src.template visit<FIELD == 1>([&](uint32_t key, uint32_t low, int) {
        const uint32_t f = field_of<FIELD>(key, low, v_eq);
        const uint32_t u = f - pj1, v = pu - f;
        du = u < du ? u : du;
        dv = v < dv ? v : dv;
    });
    comb_min2<NT>(du, dv, sh, rb);
    E.mn = du + pj1;
    E.mx = dv <= pu ? pu - dv : 0u;
    // phase C: N_zmn, the multiplicity of z_mn
    E.N = 0;
    if (E.js >= 0) {
        const uint32_t mn = E.mn;
        uint32_t ne = 0, cnt = 0;
        src.template visit<FIELD == 1>([&](uint32_t key, uint32_t low, int) {
            const uint32_t f = field_of<FIELD>(key, low, v_eq);
            ne += ne01(f, mn);
            ++cnt;
        });
        E.N = comb_sum32<NT>(cnt - ne, sh, rb);
    }
    return E;
}

struct CountOut {
    uint32_t v, n_gt, N;
};

// Quaternary pivot search for the K-th largest field value (K >= 1) among the
// source's candidates, with duplicates: returns v, n_gt = #{> v} and
// N = #{== v}, so #{> v} < K <= #{>= v}. Invariant: G(lo) >= K > G(hi) with
// G(x) = #{field > x}. Each iteration tests pivots at 25/50/75 % of (lo, hi);
// for a pivot with G >= K, z_mn (smallest value above it) and N_zmn decide
// termination (G - N_zmn < K means z_mn is the boundary value), otherwise
// z_mn itself becomes the new lower end since G(z_mn) = G - N_zmn >= K.
template <int NT, int FIELD, class S>
QRITA_DEV CountOut qsearch_count(const S& src, uint32_t v_eq, uint32_t K, int64_t lo_in, uint32_t G_lo,
                                 int64_t hi_in, uint32_t G_hi, int mode, Shared& sh, int& rb, int& iters) {
    // every field value is nonzero, so a lower end below 0 is the same as 0
    uint32_t lo = lo_in > 0 ? (uint32_t)lo_in : 0u;
    uint32_t hi = (uint32_t)hi_in;
#pragma unroll 1
    for (int guard = 0; guard < 80; ++guard) {
        if (hi - lo <= 1) return CountOut{hi, G_hi, G_lo - G_hi};
        uint32_t piv[3];
        make_pivots(lo, hi, mode, FIELD, piv);
        const Eval E = eval_pivots<NT, FIELD, false>(src, v_eq, piv, K, 0.0, sh, rb);
        ++iters;
        if (E.js >= 0) {
            const uint32_t g = sel3(E.js, E.G);
            if (g - E.N < K) return CountOut{E.mn, g - E.N, E.N};
            lo = E.mn;
            G_lo = g - E.N;
        }
        if (E.js < 2) {
            // G(z_mx) = G(pivot): nothing lies in (z_mx, pivot]
            const uint32_t pu = sel3(E.js + 1, piv);
            hi = E.mx > lo ? E.mx : pu;
            G_hi = sel3(E.js + 1, E.G);
        }
    }
    return CountOut{hi, G_hi, G_lo - G_hi};  // not reached for consistent inputs
}

struct MassOut {
    uint32_t v, n_gt, N;
    uint64_t M_gt;
};

// The same quaternary search over softmax mass: finds the key v with
// M(> v) < T <= M(>= v) among the source's candidates.
template <int NT, class S>
QRITA_DEV MassOut qsearch_mass(const S& src, double T, float m, int64_t lo_in, uint64_t M_lo, uint32_t G_lo,
                               int64_t hi_in, int mode, Shared& sh, int& rb, int& iters) {
    uint32_t lo = lo_in > 0 ? (uint32_t)lo_in : 0u;
    uint32_t hi = (uint32_t)hi_in;
    uint64_t M_hi = 0;
    uint32_t G_hi = 0;
#pragma unroll 1
    for (int guard = 0; guard < 80; ++guard) {
        if (hi - lo <= 1) return MassOut{hi, G_hi, G_lo - G_hi, M_hi};
        uint32_t piv[3];
        make_pivots(lo, hi, mode, 0, piv);
        const Eval E = eval_pivots<NT, 0, true>(src, 0u, piv, 0u, T, sh, rb);
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
            const uint32_t pu = sel3(E.js + 1, piv);
            hi = E.mx > lo ? E.mx : pu;
            M_hi = sel3(E.js + 1, E.M);
            G_hi = sel3(E.js + 1, E.G);
        }
    }
    return MassOut{hi, G_hi, G_lo - G_hi, M_hi};
}

// Boundary of "the `need` lowest-index candidates with key v, plus everything
// above v" among the source's candidates (N of them have key v), never below
// `floor`. A small tie group is ranked directly in LDS; a large one by a
// quaternary search over the tied candidates' indices.
template <int NT, class S>
QRITA_DEV uint64_t tie_boundary(const S& src, uint32_t v, uint32_t need, uint32_t N, uint32_t V,
                                uint64_t floor, Shared& sh, int& rb, int& iters) {
    uint64_t b = (uint64_t)v << 32;
    if (need < N) {
        if (N <= kTieDirect) {
            const uint32_t lane = tid_here() & (kWave - 1);
            block_sync<NT>();
            if (threadIdx.x == 0) sh.gather_n = 0;
            // zeros after the ties (below every complemented index) round the
            // list up to whole uint4 reads
            if (threadIdx.x < 4u && N + threadIdx.x < (uint32_t)kTieDirect) sh.ties[N + threadIdx.x] = 0u;
            if constexpr (S::kRegs) {
                // slots from per-wave counts, no atomics
                uint32_t c = 0;
                src.template visit<false>([&](uint32_t key, uint32_t, int) { c += (uint32_t)__popcll(__ballot(key == v)); });
                uint32_t total = 0;
                uint32_t run = wave_prefix<NT>(c, total, sh, rb);
                src.template visit<true>([&](uint32_t key, uint32_t low, int) {
                    const bool tie = key == v;
                    const uint64_t bb = __ballot(tie);
                    const uint32_t pos = run + lanes_below(bb);
                    if (tie && pos < (uint32_t)kTieDirect) sh.ties[pos] = low;
                    run += (uint32_t)__popcll(bb);
                });
            } else {
                block_sync<NT>();
                src.template visit<true>([&](uint32_t key, uint32_t low, int) {
                    const bool tie = key == v;
                    const uint64_t bb = __ballot(tie);
                    if (bb) {
                        uint32_t base = 0;
                        if (lane == 0) base = atomicAdd(&sh.gather_n, (uint32_t)__popcll(bb));
                        base = readlane(base, 0);
                        const uint32_t pos = base + lanes_below(bb);
                        if (tie && pos < (uint32_t)kTieDirect) sh.ties[pos] = low;
                    }
                });
            }
            block_sync<NT>();
            // the tie whose complemented index has exactly need - 1 larger ones
            const uint32_t n4 = (N + 3u) / 4u;
            for (uint32_t i = threadIdx.x; i < N; i += NT) {
                const uint32_t x = sh.ties[i];
                uint32_t above = 0;
                for (uint32_t j = 0; j < n4; ++j) {
                    const uint4 q = *(const uint4*)&sh.ties[4 * j];
                    above += (q.x > x ? 1u : 0u) + (q.y > x ? 1u : 0u) + (q.z > x ? 1u : 0u) + (q.w > x ? 1u : 0u);
                }
                if (above == need - 1) sh.u32[6] = x;
            }
            block_sync<NT>();
            b |= sh.u32[6];
        } else {
            const int64_t lo = (int64_t)(0xFFFFFFFFu - (uint32_t)(V - 1)) - 1;
            const CountOut t = qsearch_count<NT, 1>(src, v, need, lo, N, (int64_t)0xFFFFFFFFu, 0u, 0, sh, rb,
                                                    iters);
            b |= t.v;
        }
    }
    return b > floor ? b : floor;
}

// Boundary B of the K largest of the source's `total` candidates, whose keys
// lie in (lo_key, kmax].
template <int NT, class S>
QRITA_DEV uint64_t select_boundary(const S& src, uint32_t K, uint32_t total, int64_t lo_key, uint32_t kmax,
                                   uint32_t V, int mode, uint64_t floor, Shared& sh, int& rb, int& iters) {
    const CountOut r =
        qsearch_count<NT, 0>(src, 0u, K, lo_key, total, (int64_t)kmax, 0u, mode, sh, rb, iters);
    return tie_boundary<NT>(src, r.v, K - r.n_gt, r.N, V, floor, sh, rb, iters);
}

QRITA_DEV uint32_t next_pow2(uint32_t x) {
    uint32_t p = 1;
    while (p < x) p <<= 1;
    return p;
}


// Bitonic sort, descending, of the NT * E entries a[0 .. NT*E) (any order),
// then out[g] = index of rank g for g < cnt. Thread t holds the logical
// elements g = t * E + e in registers. By partner distance j a stage runs in
// the thread's registers (j < E), across lanes of the wave with shuffles
// (E <= j < 64 E) or across waves through LDS (j >= 64 E; element (t, e) at
// a[e * NT + t], so the accesses of a wave are consecutive).
template <int NT, int E>
QRITA_DEV void bitonic_sort(uint64_t* a, int32_t* out, uint32_t cnt) {
    constexpr uint32_t NP = (uint32_t)NT * E;
    const uint32_t t = tid_here() % NT;
    uint64_t x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = a[e * NT + t];
    for (uint32_t k = 2; k <= NP; k <<= 1) {
        for (uint32_t j = k >> 1; j >= 64u * E; j >>= 1) {
            block_sync<NT>();
#pragma unroll
            for (int e = 0; e < E; ++e) a[e * NT + t] = x[e];
            block_sync<NT>();
            const uint32_t pt = t ^ (j / E);
            const uint32_t g0 = t * E;
            // the lower position of a descending pair keeps the larger value
            const bool keep_max = ((g0 & j) == 0) == ((g0 & k) == 0);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const uint64_t y = a[e * NT + pt];
                x[e] = ((x[e] > y) == keep_max) ? x[e] : y;
            }
        }
        for (uint32_t j = min(k >> 1, 32u * E); j >= (uint32_t)E; j >>= 1) {
            const uint32_t g0 = t * E;
            const bool keep_max = ((g0 & j) == 0) == ((g0 & k) == 0);
            const uint32_t d = j / E;
            {
                // every exchange of the stage is issued before the first compare
                const int src_lane = (int)(((t ^ d) & (kWave - 1)) << 2);
                uint32_t ylo[E], yhi[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    ylo[e] = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane, (int)(uint32_t)x[e]);
                    yhi[e] = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane, (int)(uint32_t)(x[e] >> 32));
                }
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const uint64_t y = ((uint64_t)yhi[e] << 32) | ylo[e];
                    x[e] = ((x[e] > y) == keep_max) ? x[e] : y;
                }
            }
        }
        // direction of element e: descending iff bit k of t * E + e is clear;
        // for k >= E that is one lane mask for all e, below it depends on e only
        const bool desc_t = ((t * E) & k) == 0;
#pragma unroll
        for (int j = E / 2; j >= 1; j >>= 1) {
            if ((uint32_t)j < k) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if ((e & j) == 0) {
                        const bool desc = k >= (uint32_t)E ? desc_t : (((uint32_t)e & k) == 0);
                        const uint64_t p = x[e], q = x[e | j];
                        // equal entries (only padding) may swap either way
                        const bool sw = (p < q) == desc;
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
}

// Rank order of the cnt <= sort_cap<NT>() candidates in a[0 .. cnt): up to
// 128 of them are sorted by one wave without barriers, larger sets by all NT
// threads.
//
// Kept out of line: the sort's registers are then allocated on their own
// instead of on top of everything live at each of its call sites.
template <int NT>
QRITA_DEV uint32_t sort_cap(const Params& P) {
    return NT == kWave ? (uint32_t)(kWave * kWaveR) : min((uint32_t)P.tail_alloc, 16u * NT);
}
template <int NT>
__device__ __attribute__((noinline)) void sort_emit(uint32_t cnt, int32_t* out) {
    uint64_t* a = lds_cands();
    if (cnt <= 128) {
        const uint32_t np = cnt <= 64 ? 64 : 128;
        for (uint32_t i = cnt + threadIdx.x; i < np; i += NT) a[i] = 0ull;
        block_sync<NT>();
        if (threadIdx.x < (uint32_t)kWave) {
            if (np == 64)
                bitonic_sort<kWave, 1>(a, out, cnt);
            else
                bitonic_sort<kWave, 2>(a, out, cnt);
        }
        block_sync<NT>();
        return;
    }
    // a one-wave step hands sets above 128 to the whole workgroup's sort
    if constexpr (NT > kWave) {
        uint32_t np = next_pow2(cnt);
        if (np < (uint32_t)NT) np = NT;
        for (uint32_t i = cnt + threadIdx.x; i < np; i += NT) a[i] = 0ull;
        block_sync<NT>();
        switch (np / NT) {
            case 1: bitonic_sort<NT, 1>(a, out, cnt); break;
            case 2: bitonic_sort<NT, 2>(a, out, cnt); break;
            case 4: bitonic_sort<NT, 4>(a, out, cnt); break;
            case 8: bitonic_sort<NT, 8>(a, out, cnt); break;
            default: bitonic_sort<NT, 16>(a, out, cnt); break;
        }
        block_sync<NT>();
    }
}

// Gather the candidates c with lo_b <= c < hi_b (exactly cnt <= tail_alloc of
// them) into LDS with one reservation per wave and write their indices in
// rank order to out_idx[row][off ...].
template <int NT, class S>
QRITA_DEV void emit_indices(const Params& P, int64_t row, const S& src, uint64_t lo_b, uint64_t hi_b,
                            uint32_t cnt, uint32_t off, Shared& sh, int& rb, bool defer = false) {
    uint64_t* a = lds_cands();
    const uint32_t lane = tid_here() & (kWave - 1);
    const uint32_t cap = (uint32_t)P.tail_alloc;
    block_sync<NT>();
    if (threadIdx.x == 0) sh.gather_n = 0;
    block_sync<NT>();
    const uint32_t lk = cand_key(lo_b), ll = cand_low(lo_b), hk = cand_key(hi_b), hl = cand_low(hi_b);
    auto takes = [&](uint32_t key, uint32_t lw) {
        return key != 0 && (key > lk || (key == lk && lw >= ll)) && (key < hk || (key == hk && lw < hl));
    };
    if constexpr (S::kRegs) {
        // positions from per-wave counts, no atomics
        uint32_t c = 0;
        src.template visit<true>([&](uint32_t key, uint32_t low, int) { c += (uint32_t)__popcll(__ballot(takes(key, low))); });
        uint32_t total = 0;
        uint32_t run = wave_prefix<NT>(c, total, sh, rb);
        src.template visit<true>([&](uint32_t key, uint32_t lw, int) {
            const bool take = takes(key, lw);
            const uint64_t b = __ballot(take);
            const uint32_t pos = run + lanes_below(b);
            if (take && pos < cap) a[pos] = ((uint64_t)key << 32) | lw;
            run += (uint32_t)__popcll(b);
        });
    } else {
        src.template visit<true>([&](uint32_t key, uint32_t lw, int) {
            const bool take = takes(key, lw);
            const uint64_t b = __ballot(take);
            if (b) {
                uint32_t base = 0;
                if (lane == 0) base = atomicAdd(&sh.gather_n, (uint32_t)__popcll(b));
                base = readlane(base, 0);
                const uint32_t pos = base + lanes_below(b);
                if (take && pos < cap) a[pos] = ((uint64_t)key << 32) | lw;
            }
        });
    }
    block_sync<NT>();
    if (defer) {
        // a step run by one wave leaves the sort to the whole workgroup
        if (threadIdx.x == 0) {
            sh.u32[4] = cnt;
            sh.u32[5] = 1u;
        }
        return;
    }
    sort_emit<NT>(cnt, P.out_idx + row * (int64_t)P.idx_cap + off);
}

struct TailDiag {
    int32_t n_t;
    int32_t iters;
};

// What finish_head leaves for finish_rest: the kept set {c >= B} of L
// tokens, setn of them among the candidates, and the row's facts.
struct RowState {
    uint64_t B;
    uint32_t L, setn, n, kmax;
    int64_t key_lo;
    uint64_t rest_fx;
    float rest_ref, m;
    bool topk, topp;
};

// Rank windows of sort_cap entries of the kept set {c >= B} (Lout of its
// `setn` candidates, keys in (lo_b, kmax]), each window found by its own
// boundary.
template <int NT, class S>
QRITA_DEV void emit_windows_src(const Params& P, int64_t row, const S& src, uint64_t B, uint32_t Lout,
                                uint32_t setn, int64_t lo_b, uint32_t kmax, Shared& sh, int& rb, TailDiag& dg) {
    const uint32_t cap = sort_cap<NT>(P);
    uint64_t prev = ~0ull;
    for (uint32_t done = 0; done < Lout;) {
        const uint32_t cnt = min(cap, Lout - done);
        const uint64_t Bn = select_boundary<NT>(src, done + cnt, setn, lo_b, kmax, (uint32_t)P.vocab,
                                                P.pivot_mode, B, sh, rb, dg.iters);
        emit_indices<NT>(P, row, src, Bn, prev, cnt, done, sh, rb);
        prev = Bn;
        done += cnt;
    }
}

// The same over the row's list in memory (the n candidates the register set
// was loaded from), for kept sets larger than one sort. Returns the
// iterations spent in iters and the record-buffer parity in n_t.
template <int NT>
__device__ __attribute__((noinline)) TailDiag emit_windows(const Params& P, int64_t row, uint32_t n, uint64_t B,
                                                           uint32_t Lout, uint32_t setn, int64_t lo_b,
                                                           uint32_t kmax, Shared& sh, int rb) {
    MemSrc<NT, false, false> src{P.glist + row * (int64_t)P.list_stride, nullptr, n, B, 0.0f};
    TailDiag dg{0, 0};
    emit_windows_src<NT>(P, row, src, B, Lout, setn, lo_b, kmax, sh, rb, dg);
    dg.n_t = rb;
    return dg;
}

// Steps a4-a7 of the path on one candidate source holding n candidates, all
// with keys in (key_lo, kmax]; rest_fx is the fixed-point mass, relative to
// rest_ref, of the logits left out of the source (top-p-only rows). Returns
// false when the source does not contain the answer (a truncation miss); then
// nothing has been written.
template <int NT, class S>
QRITA_DEV bool finish_head(const Params& P, int64_t row, const RowMode& md, S& src, uint32_t n,
                           int64_t key_lo, uint32_t kmax, uint64_t rest_fx, float rest_ref, float t_gauss,
                           Shared& sh, int& rb, TailDiag& dg, RowState& st) {
    const uint32_t V = (uint32_t)P.vocab;
    if (P.diag) {  // #{z >= Gaussian t} among the candidates, for diagnostics
        const uint32_t key_t = f32_key(__float_as_uint(t_gauss));
        uint32_t c = 0;
        src.template visit<false>([&](uint32_t key, uint32_t, int) { c += key >= key_t ? 1u : 0u; });
        dg.n_t = (int32_t)comb_sum32<NT>(c, sh, rb);
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
        B = select_boundary<NT>(src, K, n, key_lo, kmax, V, P.pivot_mode, 0ull, sh, rb, dg.iters);
        L = K;
        setn = K;
        src.restrict_to(B);
        if constexpr (S::kRegs) src.compact((uint32_t*)lds_cands(), (uint32_t)P.tail_alloc, sh, rb);
    }
    st = RowState{B, L, setn, n, kmax, key_lo, rest_fx, rest_ref, m, topk, topp};
    return true;
}

// Steps a6-a7 after finish_head (possibly on a register set handed to
// fewer threads). Returns false only for a top-p-only row whose candidates
// do not hold mass p (a truncation miss; nothing has been written).
template <int NT, class S>
QRITA_DEV bool finish_rest(const Params& P, int64_t row, const RowMode& md, S& src, const RowState& st,
                           Shared& sh, int& rb, TailDiag& dg) {
    const uint32_t V = (uint32_t)P.vocab;
    const bool topk = st.topk, topp = st.topp;
    const uint32_t n = st.n, kmax = st.kmax;
    const int64_t key_lo = st.key_lo;
    const uint64_t rest_fx = st.rest_fx;
    const float rest_ref = st.rest_ref, m = st.m;
    uint64_t B = st.B;
    uint32_t L = st.L, setn = st.setn;
    if (topp) {
        src.prepare_mass(m);
        uint64_t ms = 0;
        src.template visit<false>([&](uint32_t key, uint32_t, int r) { ms += fx_from_unit_f32(src.mass_at(r, key)); });
        ms = comb_sum64<NT>(ms, sh, rb);
        double mass_all = (double)ms;
        // the dropped logits' mass was taken relative to rest_ref <= m
        if (!topk && rest_fx) mass_all += (double)rest_fx * (double)mass_f32(f32_key(__float_as_uint(rest_ref)), m);
        const double T = (double)md.p * mass_all;
        if (!topk && (double)ms < T) return false;  // mass p not inside the candidates
        const int64_t lo = B ? (int64_t)cand_key(B) - 1 : key_lo;
        const MassOut mo = qsearch_mass<NT>(src, T, m, lo, ms, setn, (int64_t)kmax, P.pivot_mode, sh, rb,
                                            dg.iters);
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
        B = tie_boundary<NT>(src, mo.v, need, mo.N, V, B, sh, rb, dg.iters);
        L = mo.n_gt + need;
        setn = L;
        src.restrict_to(B);
        if constexpr (S::kRegs) src.compact((uint32_t*)lds_cands(), (uint32_t)P.tail_alloc, sh, rb);
    }
    // a7: mask (pass 1 zero-filled the row; keep-all rows were filled there)
    if (P.mask && !md.keep_all) {
        uint8_t* mrow = P.mask + row * (int64_t)V;
        const uint32_t bk = cand_key(B), bl = cand_low(B);
        src.template visit<true>([&](uint32_t key, uint32_t lw, int) {
            if (key != 0 && (key > bk || (key == bk && lw >= bl))) mrow[~lw] = 1;
        });
    }
    // a7: indices in rank order
    if (P.out_idx && P.idx_cap > 0) {
        const uint32_t Lout = L < (uint32_t)P.idx_cap ? L : (uint32_t)P.idx_cap;
        const int64_t lo_b = B ? (int64_t)cand_key(B) - 1 : key_lo;
        const uint32_t cap = sort_cap<NT>(P);
        if (Lout <= cap) {
            uint64_t Bo = B;
            if (Lout < L) {
                Bo = select_boundary<NT>(src, Lout, setn, lo_b, kmax, V, P.pivot_mode, B, sh, rb, dg.iters);
                src.restrict_to(Bo);
            }
            emit_indices<NT>(P, row, src, Bo, ~0ull, Lout, 0u, sh, rb, NT == kWave && Lout > 128);
        } else if constexpr (S::kRegs) {
            // a kept set larger than one sort: windows over the row list
            const TailDiag w = emit_windows<NT>(P, row, n, B, Lout, setn, lo_b, kmax, sh, rb);
            dg.iters += w.iters;
            rb = w.n_t;
        } else {
            emit_windows_src<NT>(P, row, src, B, Lout, setn, lo_b, kmax, sh, rb, dg);
        }
    }
    if (P.out_count && threadIdx.x == 0) P.out_count[row] = (int32_t)L;
    return true;
}

template <int NT, class S>
QRITA_DEV bool finish_row(const Params& P, int64_t row, const RowMode& md, S& src, uint32_t n, int64_t key_lo,
                          uint32_t kmax, uint64_t rest_fx, float rest_ref, float t_gauss, Shared& sh, int& rb,
                          TailDiag& dg) {
    RowState st;
    if (!finish_head<NT>(P, row, md, src, n, key_lo, kmax, rest_fx, rest_ref, t_gauss, sh, rb, dg, st))
        return false;
    return finish_rest<NT>(P, row, md, src, st, sh, rb, dg);
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
// evenly spaced offsets (the whole row when it has at most 2048 logits). A
// thread's 8 logits are consecutive; away from the row's ends each run is
// moved down to a 16-byte boundary and read with vector loads.
template <bool BF16>
QRITA_DEV void load_sample(const void* rowp, int32_t V, float x[8], bool in[8]) {
    const int tid = threadIdx.x;
    const bool whole = V <= kSampleN;
    int64_t pos0 =
        whole ? (int64_t)tid * 8
              : ((int64_t)(tid >> 5) * (int64_t)(V - kSampleChunk)) / (kSampleChunks - 1) + (int64_t)(tid & 31) * 8;
    constexpr int64_t ES = BF16 ? 2 : 4;
    const int64_t mis = (int64_t)(((uintptr_t)rowp / ES + (uint64_t)pos0) & (BF16 ? 7 : 3));
    if (!whole && tid < kSampleN / 8 && pos0 >= mis && pos0 - mis + 8 <= V) {
        pos0 -= mis;
#pragma unroll
        for (int i = 0; i < 8; ++i) in[i] = true;
        if (BF16) {
            const u32x4_t w = *(const u32x4_t*)((const uint16_t*)rowp + pos0);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[2 * r] = __uint_as_float(ws[r] << 16);
                x[2 * r + 1] = __uint_as_float(ws[r] & 0xFFFF0000u);
            }
        } else {
            const f32x4_t a = *(const f32x4_t*)((const float*)rowp + pos0);
            const f32x4_t b = *(const f32x4_t*)((const float*)rowp + pos0 + 4);
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t e = pos0 + i;
        in[i] = tid < kSampleN / 8 && e < V;
        x[i] = in[i] ? load_value<BF16>(rowp, e) : 0.0f;
    }
}

// r-th largest key of the sample (1 <= r <= number of sample entries), by the
// same quaternary search over the sample held in registers.
template <int THREADS, bool BF16>
QRITA_DEV float sample_rank_value(const void* rowp, int32_t V, uint32_t r, Shared& sh, int& rb) {
    float x[8];
    bool in[8];
    load_sample<BF16>(rowp, V, x, in);
    // only keys are searched: the indices (duplicate order) are never read
    RegSet<THREADS, 8> s;
    s.nslots = 8u * THREADS;
    s.lows = nullptr;
    s.em = nullptr;
#pragma unroll
    for (int i = 0; i < 8; ++i) s.key[i] = in[i] ? f32_key(__float_as_uint(x[i])) : 0u;
    const uint32_t ns = (uint32_t)min(V, kSampleN);
    int it = 0;
    const CountOut o =
        qsearch_count<THREADS, 0>(s, 0u, r, (int64_t)0, ns, (int64_t)0xFFFFFFFFu, 0u, 0, sh, rb, it);
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
    for (int i = threadIdx.x; i < kHistBins; i += THREADS) sh.hist[i] = 0u;
    float x[8];
    bool in[8];
    load_sample<BF16>(rowp, V, x, in);
    // mean, variance and range of the finite sample values in one reduction
    // (moments about the row's first logit, fixed reduction order)
    float c0 = load_value<BF16>(rowp, 0);
    c0 = __builtin_isfinite(c0) ? c0 : 0.0f;
    float s1 = 0.0f, s2 = 0.0f;
    uint32_t nf = 0, kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const bool ok = in[i] && __builtin_isfinite(x[i]);
        const float d = ok ? x[i] - c0 : 0.0f;
        s1 += d;
        s2 += d * d;
        nf += ok ? 1u : 0u;
        const uint32_t k = f32_key(__float_as_uint(x[i]));
        kmn = ok && k < kmn ? k : kmn;
        kmx = ok && k > kmx ? k : kmx;
    }
    s1 = wave_sum_f32_dpp(s1);
    s2 = wave_sum_f32_dpp(s2);
    nf = wave_sum_u32(nf);
    kmn = wave_min_u32(kmn);
    kmx = wave_max_u32(kmx);
    if (lane == 0) *(uint4*)sh.slot[rb][wave] = make_uint4(__float_as_uint(s1), __float_as_uint(s2), nf, 0u);
    if (lane == 0) *(uint2*)&sh.slot[rb][wave][4] = make_uint2(kmn, kmx);
    __syncthreads();
    float t1 = 0.0f, t2 = 0.0f;
    uint32_t n = 0;
    kmn = 0xFFFFFFFFu;
    kmx = 0u;
    for (int w = 0; w < NW; ++w) {
        const uint4 q = *(const uint4*)sh.slot[rb][w];
        const uint2 r = *(const uint2*)&sh.slot[rb][w][4];
        t1 += __uint_as_float(q.x);
        t2 += __uint_as_float(q.y);
        n += q.z;
        kmn = r.x < kmn ? r.x : kmn;
        kmx = r.y > kmx ? r.y : kmx;
    }
    rb ^= 1;
    const float m1 = n ? t1 / (float)n : 0.0f;
    const float mu = c0 + m1;
    const float var = n ? fmaxf(t2 / (float)n - m1 * m1, 0.0f) : 0.0f;
    const float sigma = sqrtf(var);
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
    // then collect down to about the r-th largest sample value instead
    // (r = lambda + 5 sqrt(lambda) + 5), so the miss is served from the same
    // single pass. That value is read off a 256-bin histogram of the sample
    // over its range: the lower edge of the bin where the count from the top
    // reaches r, less half a bin, is at or below the r-th largest value.
    if (md.K_t > 0 && n >= 2 && __builtin_isfinite(t)) {
        const float lo = key_value(kmn), hi = key_value(kmx);
        const float w = (hi - lo) * (1.0f / kHistBins);
        const float inv = w > 0.0f ? 1.0f / w : 0.0f;
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool ok = in[i] && __builtin_isfinite(x[i]);
            c += (ok && x[i] >= t) ? 1u : 0u;
            if (ok) {
                const int b = (int)fminf(fmaxf((x[i] - lo) * inv, 0.0f), (float)(kHistBins - 1));
                atomicAdd(&sh.hist[b], 1u);
            }
        }
        c = wave_sum_u32(c);
        if (lane == 0) sh.slot[rb][wave][0] = c;
        __syncthreads();
        uint32_t ct = 0;
        for (int v = 0; v < NW; ++v) ct += sh.slot[rb][v][0];
        rb ^= 1;
        const float lam = (float)ns * (float)md.K_t / (float)V;
        th.lambda = lam;
        if (lam >= 4.0f && (float)ct < 1.25f * lam + 2.0f) {
            const uint32_t r = min((uint32_t)ceilf(lam + 5.0f * sqrtf(lam) + 5.0f), ns);
            // every wave scans the histogram from the top: lane l holds bins
            // 4l .. 4l+3, and the suffix counts come from a DPP scan
            const uint32_t b0 = sh.hist[4 * lane], b1 = sh.hist[4 * lane + 1], b2 = sh.hist[4 * lane + 2],
                           b3 = sh.hist[4 * lane + 3];
            const uint32_t own = b0 + b1 + b2 + b3;
            const uint32_t above = wave_suffix_sum_excl(own);  // bins of higher lanes
            // highest bin whose count from the top reaches r
            int bin = -1;
            const uint32_t c3 = above + b3, c2 = c3 + b2, c1 = c2 + b1, cz = c1 + b0;
            bin = c3 >= r ? 4 * lane + 3 : (c2 >= r ? 4 * lane + 2 : (c1 >= r ? 4 * lane + 1 : (cz >= r ? 4 * lane : -1)));
            const uint64_t has = __ballot(bin >= 0);
            // the reaching bin sits in the highest lane that has one
            const int src = has ? 63 - (int)__builtin_clzll(has) : 0;
            const int best = __shfl(bin, src);
            const float tfb = best >= 0 ? lo + ((float)best - 0.5f) * w : -kInf;
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
// index idx0 + (j / VE) * vstride + (j % VE); bit j of `valid` marks it as
// present. Survivors past the stage go straight to the row list (with their
// key, for the list's max). For top-p-only rows (REST) the dropped logits'
// masses exp(f - tc) are summed per lane in float over the 16 and added to
// the fixed-point `rest` once, so the total does not depend on lane order.
template <int THREADS, bool BF16, bool REST, int VE>
QRITA_DEV void consume16(const Params& P, int64_t row, const float f[16], uint32_t valid, uint32_t idx0,
                         uint32_t vstride, float tc, Shared& sh, uint64_t& rest, uint32_t& spill_kmax) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    uint32_t tot = 0;
    float dropped = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const bool v = (valid >> j) & 1u;
        const bool s = v && f[j] >= tc;
        tot += (uint32_t)__popcll(__ballot(s));
        if (REST) dropped += (v && !s) ? __expf(f[j] - tc) : 0.0f;
    }
    if (REST) rest += fx_from_unit_f32(fminf(dropped * 0x1p-5f, 1.0f)) << 5;
    if (tot == 0) return;
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&sh.ncand, tot);
    base = readlane(base, 0);
    const uint32_t cap = (uint32_t)P.stage_cap;
    uint64_t* a = lds_cands();
    uint32_t run = base;
    if (base + tot <= cap) {
        // the whole group fits the stage
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const bool s = ((valid >> j) & 1u) && f[j] >= tc;
            const uint64_t b = __ballot(s);
            if (b) {
                if (s)
                    a[run + lanes_below(b)] = ((uint64_t)__float_as_uint(f[j]) << 32) |
                                              (idx0 + (uint32_t)(j / VE) * vstride + (uint32_t)(j % VE));
                run += (uint32_t)__popcll(b);
            }
        }
        return;
    }
    const uint32_t spill_from = base > cap ? base : cap;
    const uint32_t nover = base + tot - spill_from;
    uint32_t gbase = 0;
    if (lane == 0) gbase = atomicAdd(&P.hdr[row * H_WORDS + H_LIST], nover);
    gbase = readlane(gbase, 0);
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

// One tile (THREADS * 16 logits from `tile`, all inside the slice): vector
// loads marked non-temporal (the logits are read once) into f.
template <int THREADS, bool BF16>
QRITA_DEV void load_tile(const void* rowp, int64_t tile, float f[16]) {
    constexpr int VE = BF16 ? 8 : 4;
    constexpr int NV = 16 / VE;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        const int64_t e = tile + (int64_t)q * THREADS * VE + (int64_t)threadIdx.x * VE;
        if (BF16) {
            const u32x4_t w = __builtin_nontemporal_load((const u32x4_t*)((const uint16_t*)rowp + e));
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                f[q * 8 + 2 * r] = __uint_as_float(ws[r] << 16);
                f[q * 8 + 2 * r + 1] = __uint_as_float(ws[r] & 0xFFFF0000u);
            }
        } else {
            const f32x4_t w = __builtin_nontemporal_load((const f32x4_t*)((const float*)rowp + e));
            f[q * 4 + 0] = w.x;
            f[q * 4 + 1] = w.y;
            f[q * 4 + 2] = w.z;
            f[q * 4 + 3] = w.w;
        }
    }
}

// The mask bytes of one full tile (this lane's 16 entries).
template <int THREADS, bool BF16>
QRITA_DEV void fill_tile(uint8_t* mrow, int64_t tile, uint8_t fill) {
    constexpr int VE = BF16 ? 8 : 4;
    constexpr int NV = 16 / VE;
    const uint64_t fill8 = 0x0101010101010101ull * fill;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        const int64_t e = tile + (int64_t)q * THREADS * VE + (int64_t)threadIdx.x * VE;
        if (BF16)
            __builtin_nontemporal_store(fill8, (uint64_t*)(mrow + e));
        else
            __builtin_nontemporal_store((uint32_t)fill8, (uint32_t*)(mrow + e));
    }
}

// First 16-element-aligned position of the slice [e0, e1) of a row starting
// at element roff of the batch.
QRITA_DEV int64_t aligned_start(int64_t roff, int64_t e0, int64_t e1) {
    const int64_t a = e0 + ((16 - ((roff + e0) & 15)) & 15);
    return a > e1 ? e1 : a;
}

// The streaming pass over [e0, e1); f0 holds the slice's first full tile
// (loaded before the threshold was known) when there is one.
template <int THREADS, bool BF16, bool REST>
QRITA_DEV void stream_slice(const Params& P, int64_t row, int64_t e0, int64_t e1, float tc, uint8_t fill,
                            const float (&f0)[16], Shared& sh, uint64_t& rest, uint32_t& spill_kmax) {
    const int64_t roff = row * (int64_t)P.vocab;
    const void* rowp = row_ptr<BF16>(P, row);
    uint8_t* mrow = P.mask ? P.mask + roff : nullptr;
    const int tid = threadIdx.x;
    // head: up to 15 logits before the first 16-element-aligned position
    const int64_t a = aligned_start(roff, e0, e1);
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
    // full tiles: the next tile's loads are issued before this one is consumed
    const int64_t nfull = (e1 - a) / TB;
    float f[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) f[j] = f0[j];
    for (int64_t i = 0; i < nfull; ++i) {
        const int64_t tile = a + i * TB;
        float g[16];
        if (i + 1 < nfull) load_tile<THREADS, BF16>(rowp, tile + TB, g);
        if (mrow) fill_tile<THREADS, BF16>(mrow, tile, fill);
        consume16<THREADS, BF16, REST, VE>(P, row, f, 0xFFFFu, (uint32_t)(tile + (int64_t)tid * VE),
                                           (uint32_t)(THREADS * VE), tc, sh, rest, spill_kmax);
#pragma unroll
        for (int j = 0; j < 16; ++j) f[j] = g[j];
    }
    // ragged last tile, element by element
    const int64_t tile = a + nfull * TB;
    if (tile < e1) {
        uint32_t valid = 0;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
#pragma unroll
            for (int r = 0; r < VE; ++r) {
                const int64_t er = tile + (int64_t)q * THREADS * VE + (int64_t)tid * VE + r;
                if (er < e1) {
                    f[q * VE + r] = load_value<BF16>(rowp, er);
                    valid |= 1u << (q * VE + r);
                    if (mrow) mrow[er] = fill;
                } else {
                    f[q * VE + r] = 0.0f;
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
    // this workgroup's slice; slices after the first start 16-aligned
    const int64_t A = (16 - (roff & 15)) & 15;
    int64_t e0 = slice == 0 ? 0 : A + (int64_t)slice * P.slice_len;
    int64_t e1 = A + (int64_t)(slice + 1) * P.slice_len;
    if (slice + 1 == (uint32_t)P.slices || e1 > V) e1 = V;
    if (e0 > V) e0 = V;
    // the first full tile is loaded before the threshold is known
    float f0[16];
    {
        const int64_t a = aligned_start(roff, e0, e1);
        if (e1 - a >= (int64_t)THREADS * 16) load_tile<THREADS, BF16>(rowp, a, f0);
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
    // a3: the single streaming pass over the slice
    const uint8_t fill = md.keep_all ? 1 : 0;
    const bool rest_on = md.topp && !md.topk;
    uint64_t rest = 0;
    uint32_t kmax = 0;
    if (rest_on)
        stream_slice<THREADS, BF16, true>(P, row, e0, e1, th.tc, fill, f0, sh, rest, kmax);
    else
        stream_slice<THREADS, BF16, false>(P, row, e0, e1, th.tc, fill, f0, sh, rest, kmax);
    __syncthreads();
    // publish: the staged candidates go to the row list in one reservation,
    // whose round trip overlaps the maximum over the stage
    const uint32_t nst = min(sh.ncand, (uint32_t)P.stage_cap);
    uint32_t gb = 0;
    if (threadIdx.x == 0 && nst) gb = atomicAdd(&hdr[H_LIST], nst);
    constexpr int PER = kSampleN / THREADS;  // stage entries per thread (stage_cap <= 2048)
    const uint64_t* a = lds_cands();
    uint32_t keys[PER], lows[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const uint32_t i = (uint32_t)u * THREADS + threadIdx.x;
        const uint64_t r = i < nst ? a[i] : 0ull;
        keys[u] = i < nst ? f32_key((uint32_t)(r >> 32)) : 0u;
        lows[u] = ~(uint32_t)r;
        kmax = keys[u] > kmax ? keys[u] : kmax;
    }
    if (threadIdx.x == 0) sh.u32[0] = gb;
    uint32_t d0 = 0, d1 = 0;
    block_sum_min_max<THREADS>(d0, d1, kmax, rest, sh, rb);
    gb = sh.u32[0];
    uint64_t* lst = P.glist + row * (int64_t)P.list_stride;
    bool over = false;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const uint32_t i = (uint32_t)u * THREADS + threadIdx.x;
        if (i < nst) {
            if (gb + i < (uint32_t)P.list_cap)
                lst[gb + i] = ((uint64_t)keys[u] << 32) | lows[u];
            else
                over = true;
        }
    }
    if (over) atomicOr(&hdr[H_FLAGS], 1u);
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


struct TailOut {
    int32_t done, path, n_t, iters, rb;
};

// The tail's slow paths, kept out of line so their registers are allocated
// apart from the register-set paths: a row list too long for registers
// (searched in memory), and after a truncation miss the re-collection of the
// row with thresholds lowered to sample order statistics and, as the last
// resort, the search of the full row (§1).
template <int NT, bool BF16>
__device__ __attribute__((noinline)) TailOut tail_fallback(const Params& P, int64_t row, RowMode md, float t,
                                                           float tc, uint32_t nlist, uint32_t kmax, uint64_t rest,
                                                           bool overflow, bool list_tried, float lambda,
                                                           uint32_t ns_h, int32_t n_t, Shared& sh, int rb) {
    const int32_t V = P.vocab;
    const void* rowp = row_ptr<BF16>(P, row);
    uint64_t* lst = P.glist + row * (int64_t)P.list_stride;
    const float kInf = __builtin_inff();
    TailDiag dg{n_t, 0};
    int path = 1;
    bool done = false;
    if (!list_tried && !overflow) {
        MemSrc<NT, false, BF16> src{lst, nullptr, nlist, 0ull, 0.0f};
        done = finish_row<NT>(P, row, md, src, nlist, (int64_t)f32_key(__float_as_uint(tc)) - 1, kmax, rest, tc,
                              t, sh, rb, dg);
    }
    if (!done) {
        path = 2;
        const uint32_t ns = ns_h ? ns_h : (uint32_t)min(V, kSampleN);
        const float r0 = md.K_t > 0 ? ceilf(lambda + 5.0f * sqrtf(lambda) + 5.0f) : 64.0f;
        float prev = tc;
#pragma unroll 1
        for (int attempt = 1; attempt <= 8 && !done; ++attempt) {
            const float rr = r0 * (float)(1u << (2 * attempt));
            float tr;
            if (rr < (float)ns)
                tr = sample_rank_value<NT, BF16>(rowp, V, (uint32_t)rr, sh, rb);
            else if (prev > -kInf)
                tr = -kInf;
            else
                break;
            if (!(tr < prev)) continue;
            prev = tr;
            uint64_t rest2 = 0;
            uint32_t kmax2 = 0;
            bool ovf = false;
            const uint32_t cnt =
                collect_row<NT, BF16>(P, row, tr, md.topp && !md.topk, sh, rb, rest2, kmax2, ovf);
            if (ovf) break;
            MemSrc<NT, false, BF16> src{lst, nullptr, cnt, 0ull, 0.0f};
            done = finish_row<NT>(P, row, md, src, cnt, (int64_t)f32_key(__float_as_uint(tr)) - 1, kmax2, rest2,
                                  tr, t, sh, rb, dg);
            if (tr == -kInf) break;
        }
    }
    if (!done) {
        path = 3;
        uint32_t kr = 0, d0 = 0, d1 = 0;
        uint64_t d2 = 0;
        for (int64_t e = threadIdx.x; e < V; e += NT) {
            const uint32_t key = f32_key(__float_as_uint(load_value<BF16>(rowp, e)));
            kr = key > kr ? key : kr;
        }
        block_sum_min_max<NT>(d0, d1, kr, d2, sh, rb);
        MemSrc<NT, true, BF16> src{nullptr, rowp, (uint32_t)V, 0ull, 0.0f};
        done = finish_row<NT>(P, row, md, src, (uint32_t)V, -1, kr, 0ull, 0.0f, t, sh, rb, dg);
    }
    return TailOut{done ? 1 : 0, path, dg.n_t, dg.iters, rb};
}

// Tail: one workgroup per row, after pass 1 has completed for every row. A
// row list of up to 2048 candidates is searched by one wave with the
// candidates in its registers, a longer one of up to tail_cap by the whole
// workgroup the same way; everything else takes tail_fallback.
template <int NT, bool BF16>
__global__ __launch_bounds__(NT) void tail_kernel(Params P) {
    __shared__ Shared sh;
    int rb = 0;
    const int64_t row = blockIdx.x;
    if (row >= P.batch) return;
    const int32_t V = P.vocab;
    uint32_t* hdr = P.hdr + row * H_WORDS;
    const uint64_t* lst = P.glist + row * (int64_t)P.list_stride;
    // wave 0 reads the head of the row list before the header tells how much
    // of it is filled (entries past the fill are ignored)
    uint64_t pre[kWaveR];
    if (threadIdx.x < (uint32_t)kWave) {
        const uint32_t lim = min((uint32_t)P.list_stride, (uint32_t)(kWave * kWaveR));
#pragma unroll
        for (int r = 0; r < kWaveR; ++r) {
            const uint32_t i = (uint32_t)r * kWave + threadIdx.x;
            pre[r] = i < lim ? lst[i] : 0ull;
        }
    }
    const RowMode md = row_mode(P, row);
    const float t = __uint_as_float(hdr[H_T]);
    const float tc = __uint_as_float(hdr[H_TC]);
    const uint32_t nlist = hdr[H_LIST];
    const uint32_t kmax = hdr[H_KMAX];
    const bool overflow = hdr[H_FLAGS] != 0 || nlist > (uint32_t)P.list_cap;
    const uint64_t rest = (uint64_t)hdr[H_REST] | ((uint64_t)hdr[H_REST + 1] << 32);
    const bool predicted = hdr[H_PRED] != 0;

    TailDiag dg{-1, 0};
    int path = 0;
    bool done = false;
    if (!md.need_cand) {
        if (P.out_count && threadIdx.x == 0) P.out_count[row] = V;
        done = true;
    } else {
        const bool in_regs = !overflow && nlist <= (uint32_t)P.tail_cap;
        if (in_regs) {
            // every candidate has z >= tc, so its key exceeds key(tc) - 1
            const int64_t key_lo = (int64_t)f32_key(__float_as_uint(tc)) - 1;
            if (nlist <= (uint32_t)(kWave * kWaveR)) {
                // a small set is searched by one wave alone, without barriers
                if (threadIdx.x < (uint32_t)kWave) {
                    if (threadIdx.x == 0) sh.u32[5] = 0u;
                    RegSet<kWave, kWaveR> src;
                    src.lows = (uint32_t*)(lds_cands() + P.tail_alloc);
                    src.em = (float*)lds_cands();
                    src.load_from(pre, nlist);
                    const bool ok =
                        finish_row<kWave>(P, row, md, src, nlist, key_lo, kmax, rest, tc, t, sh, rb, dg);
                    if (threadIdx.x == 0) sh.u32[7] = ok ? 1u : 0u;
                }
                __syncthreads();
                done = sh.u32[7] != 0;
                // kept sets above 128 were gathered by the wave and are sorted here
                if (done && sh.u32[5]) sort_emit<NT>(sh.u32[4], P.out_idx + row * (int64_t)P.idx_cap);
            } else {
                RegSet<NT, kTailR> src;
                src.lows = (uint32_t*)(lds_cands() + P.tail_alloc);
                src.em = (float*)lds_cands();  // the sort buffer is free until the indices are emitted
                src.load(lst, nlist);
                RowState st;
                const bool hit = finish_head<NT>(P, row, md, src, nlist, key_lo, kmax, rest, tc, t, sh, rb, dg, st);
                if (hit && src.nslots <= (uint32_t)(kWave * kWaveR)) {
                    // the top-k set is small: one wave carries on without barriers
                    uint32_t* kb = (uint32_t*)lds_cands();
                    src.store_keys(kb);
                    __syncthreads();
                    if (threadIdx.x < (uint32_t)kWave) {
                        if (threadIdx.x == 0) sh.u32[5] = 0u;
                        RegSet<kWave, kWaveR> s1;
                        s1.lows = src.lows;
                        s1.em = src.em;
                        s1.load_keys(kb, src.nslots);
                        const bool ok = finish_rest<kWave>(P, row, md, s1, st, sh, rb, dg);
                        if (threadIdx.x == 0) sh.u32[7] = ok ? 1u : 0u;
                    }
                    __syncthreads();
                    done = sh.u32[7] != 0;
                    if (done && sh.u32[5]) sort_emit<NT>(sh.u32[4], P.out_idx + row * (int64_t)P.idx_cap);
                } else if (hit) {
                    done = finish_rest<NT>(P, row, md, src, st, sh, rb, dg);
                }
            }
        }
        if (!done) {
            const TailOut o = tail_fallback<NT, BF16>(P, row, md, t, tc, nlist, kmax, rest, overflow, in_regs,
                                                      __uint_as_float(hdr[H_LAMBDA]), hdr[H_NS], dg.n_t, sh, rb);
            done = o.done != 0;
            path = o.path;
            dg.n_t = o.n_t;
            dg.iters += o.iters;
            rb = o.rb;
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
