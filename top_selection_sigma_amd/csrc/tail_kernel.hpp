// The tail of the path (steps a4-a7): one workgroup of four waves per row,
// launched after the streaming pass has completed for every row.
//
// The row's candidates (the slices' sub-lists) are loaded once into LDS as
// keys. Every pivot evaluation of the quaternary search is one loop over the
// candidates still in play followed by one combination across the four waves.
// After an evaluation each wave moves its candidates inside the new search
// range to a segment of LDS of its own (no barrier: a wave only ever reads its
// own segment), so later evaluations visit a quarter of the keys or fewer.
// Rows whose candidates do not fit LDS are searched from the lists in global
// memory the same way; a truncation miss re-collects the row or, last, searches
// the whole row ("Metodología" §1).
//
// All visits are loops, so the code of one search step stays small enough to
// remain in the instruction cache while the step repeats.
#pragma once

namespace qrita {

// ---------------------------------------------------------------------------
// Tiers of the tail (the summary's tiered block sizes, "Autotuning"): the
// light tier fits two workgroups per CU (rows of large batches overlap their
// latencies), the heavy one holds twice the candidates and sorts kept sets of
// up to 8704 (8192 and their boundary duplicates) in one piece.
// ---------------------------------------------------------------------------
template <int CFULL_, int SEG_, int CSORT_, int NB_>
struct TailTier {
    static constexpr int NT = 256;         // threads per row
    static constexpr int NW = NT / kWave;  // waves
    static constexpr int CFULL = CFULL_;   // candidate keys held in LDS
    static constexpr int SEG = SEG_;       // 8-byte entries of one wave's search segment
    static constexpr int CSORT = CSORT_;   // largest set sorted in one piece
    static constexpr int NB = NB_;         // bucket-sort bins
    static constexpr int WAVES_PER_SIMD = CFULL_ <= 12288 ? 2 : 1;  // rows resident per CU
    // LDS layout (bytes). Search phase: keys, then the wave segments. Emit
    // phase (after the search): the words to sort; then a region that holds
    // either the words again in bin order (the bucket sort's usual case) or,
    // when bins get sized in proportion to the codes, the positions in bin
    // order, each word's bin (16 bits each) and the code starts; then the
    // bin counts. After the sort, everything past the words holds the mask
    // bitmap; the bitonic fallback sorts in everything from the words on.
    static constexpr size_t A_OFF = 0;
    static constexpr size_t W_OFF = A_OFF + (size_t)CFULL * 4;
    static constexpr size_t SEARCH_END = W_OFF + (size_t)NW * SEG * 8;
    static constexpr size_t SA_OFF = 0;
    static constexpr size_t SB_OFF = SA_OFF + (size_t)(CSORT + 8) * 8;
    static constexpr size_t BO_OFF = SB_OFF + ((size_t)CSORT * 2 + 15) / 16 * 16;
    static constexpr size_t HC_OFF = BO_OFF + ((size_t)CSORT * 2 + 15) / 16 * 16;
    static constexpr size_t BINS_OFF = SB_OFF + (size_t)CSORT * 8;
    static constexpr size_t EMIT_END = BINS_OFF + (size_t)(NB + 4) * 4;
    static constexpr size_t LDS = SEARCH_END > EMIT_END ? SEARCH_END : EMIT_END;
    static constexpr uint32_t BITMAP_BITS = (uint32_t)((LDS - SB_OFF) * 8);
    static_assert(CSORT <= 65536, "16-bit positions");
    static_assert(HC_OFF + (size_t)(NB + 4) * 4 <= BINS_OFF, "positions, bins of words and code starts in the words' region");
    static_assert(LDS - SA_OFF >= (size_t)2 * CSORT * 8, "bitonic fallback region");
    static_assert(SEARCH_END % 16 == 0 && SB_OFF % 16 == 0 && BINS_OFF % 16 == 0, "alignment");
};
using TierLight = TailTier<12288, 768, 4096, 2048>;
using TierHeavy = TailTier<24576, 1536, 8704, 4096>;

extern __shared__ uint64_t qrita_dyn_lds[];
QRITA_DEV char* dyn_lds() { return (char*)qrita_dyn_lds; }

// ---------------------------------------------------------------------------
// Block combination. Every wave reduces its lanes with DPP; lane 0 stores the
// wave's record in LDS; after one barrier every lane reads all records and
// combines them, so every thread holds the block's values without a second
// barrier (two record buffers alternate).
// ---------------------------------------------------------------------------

// Values read back from LDS are the same in every lane; readfirstlane makes
// that known to the compiler, so what depends on them (search bounds, pivots,
// branch decisions) stays in scalar registers.
QRITA_DEV uint32_t uni(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
QRITA_DEV uint64_t uni(uint64_t x) {
    return ((uint64_t)uni((uint32_t)(x >> 32)) << 32) | uni((uint32_t)x);
}

// Records of N32 u32 sums, N64 u64 sums and NMIN u32 minima (wave totals on
// entry, block totals on return).
template <int NT, int N32, int N64, int NMIN>
QRITA_DEV void comb_record(uint32_t* s32, uint64_t* s64, uint32_t* mn, Shared& sh, int& rb) {
    constexpr int NW = NT / kWave;
    constexpr int NR = N32 + 2 * N64 + NMIN;
    constexpr int NQ = (NR + 3) / 4;
    static_assert(NW <= 8 && NR <= 32, "record layout");
    if constexpr (NW > 1) {
        uint32_t* base = &sh.slot[rb][0][0];
        const uint32_t lane = tid_here() & (kWave - 1), wave = wave_base_here() / kWave;
        uint32_t w[NQ * 4];
#pragma unroll
        for (int i = 0; i < N32; ++i) w[i] = s32[i];
#pragma unroll
        for (int i = 0; i < N64; ++i) {
            w[N32 + 2 * i] = (uint32_t)s64[i];
            w[N32 + 2 * i + 1] = (uint32_t)(s64[i] >> 32);
        }
#pragma unroll
        for (int i = 0; i < NMIN; ++i) w[N32 + 2 * N64 + i] = mn[i];
#pragma unroll
        for (int i = NR; i < NQ * 4; ++i) w[i] = 0u;
        if (lane == 0) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                *(uint4*)(base + wave * 32 + 4 * q) = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
        }
        lds_sync();
#pragma unroll
        for (int i = 0; i < N32; ++i) s32[i] = 0u;
#pragma unroll
        for (int i = 0; i < N64; ++i) s64[i] = 0ull;
#pragma unroll
        for (int i = 0; i < NMIN; ++i) mn[i] = 0xFFFFFFFFu;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            uint32_t r[NQ * 4];
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const uint4 x = *(const uint4*)(base + v * 32 + 4 * q);
                r[4 * q] = x.x;
                r[4 * q + 1] = x.y;
                r[4 * q + 2] = x.z;
                r[4 * q + 3] = x.w;
            }
#pragma unroll
            for (int i = 0; i < N32; ++i) s32[i] += r[i];
#pragma unroll
            for (int i = 0; i < N64; ++i) s64[i] += (uint64_t)r[N32 + 2 * i] | ((uint64_t)r[N32 + 2 * i + 1] << 32);
#pragma unroll
            for (int i = 0; i < NMIN; ++i) mn[i] = r[N32 + 2 * N64 + i] < mn[i] ? r[N32 + 2 * N64 + i] : mn[i];
        }
        rb ^= 1;
#pragma unroll
        for (int i = 0; i < N32; ++i) s32[i] = uni(s32[i]);
#pragma unroll
        for (int i = 0; i < N64; ++i) s64[i] = uni(s64[i]);
#pragma unroll
        for (int i = 0; i < NMIN; ++i) mn[i] = uni(mn[i]);
    }
}

// Exclusive prefix over the waves of per-wave counts c (wave uniform):
// returns the sum over the lower waves and sets total to the sum over all.
template <int NT>
QRITA_DEV uint32_t wave_prefix(uint32_t c, uint32_t& total, Shared& sh, int& rb) {
    constexpr int NW = NT / kWave;
    const uint32_t lane = tid_here() & (kWave - 1), wave = wave_base_here() / kWave;
    if (lane == 0) sh.slot[rb][wave][0] = c;
    lds_sync();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t q = sh.slot[rb][w][0];
        before += (uint32_t)w < wave ? q : 0u;
        all += q;
    }
    rb ^= 1;
    total = uni(all);
    return uni(before);
}

template <int NT>
QRITA_DEV uint32_t comb_sum32(uint32_t v, Shared& sh, int& rb) {
    uint32_t s[1] = {wave_sum_u32(v)};
    comb_record<NT, 1, 0, 0>(s, nullptr, nullptr, sh, rb);
    return s[0];
}

// ---------------------------------------------------------------------------
// Candidate sources. A source hands every candidate to a visitor f(key, low):
// key 0 marks an empty slot (every real key is nonzero); low is the
// complemented vocabulary index (sources with kLows only). Visits are
// wave-uniform loops: every lane calls f the same number of times, so
// visitors may use ballots.
// ---------------------------------------------------------------------------

// The row's candidate keys in LDS, interleaved over the block's threads in
// 16-byte groups (zero padded to a multiple of four keys).
template <int NT>
struct SrcLds {
    static constexpr bool kLows = false;
    const uint32_t* a;
    uint32_t n;
    template <class F>
    QRITA_DEV void visit(F&& f) const {
        const uint32_t n4 = (n + 3u) / 4u;
        const uint32_t lane = tid_here() & (kWave - 1);
        const uint4* a4 = (const uint4*)a;
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        // two 16-byte reads per step, both issued before use (indices
        // clamped, values masked: no branch waits for a read)
        for (uint32_t v0 = wave_base_here(); v0 < n4; v0 += 2 * NT) {
            const uint32_t v = v0 + lane, w = v + NT;
            const uint4 qa = a4[v < n4 ? v : n4 - 1u], qb = a4[w < n4 ? w : n4 - 1u];
            const uint4 q = v < n4 ? qa : z, r = w < n4 ? qb : z;
            f(q.x, 0u);
            f(q.y, 0u);
            f(q.z, 0u);
            f(q.w, 0u);
            f(r.x, 0u);
            f(r.y, 0u);
            f(r.z, 0u);
            f(r.w, 0u);
        }
    }
    // this wave's share of the candidates (for sizing decisions)
    QRITA_DEV uint32_t wave_share() const { return (n + (uint32_t)(NT / kWave) - 1u) / (uint32_t)(NT / kWave); }
};

// The row's candidate lists in global memory: S sub-lists, sub-list s holding
// cnt[s] (LDS) entries at base + s * stride. Sub-list s is read by a group of
// NT >> gshift threads; two batches of eight loads per thread alternate.
template <int NT>
struct SrcList {
    static constexpr bool kLows = true;
    const uint64_t* base;
    uint32_t stride;
    uint32_t S;
    uint32_t gshift;       // log2(threads per sub-list group)
    const uint32_t* cnt;   // LDS
    uint32_t n;            // total
    template <class F>
    QRITA_DEV void visit(F&& f) const {
        constexpr int U = 8;  // entries per thread per batch; the next batch is in flight meanwhile
        const uint32_t t = tid_here();
        const uint32_t tps = 1u << gshift;
        const uint32_t s0 = t >> gshift, g = t & (tps - 1u);
        const uint32_t s = s0 < S ? s0 : 0u;  // groups past the last sub-list read sub-list 0, masked
        const uint32_t cs = s0 < S ? cnt[s] : 0u;
        const uint64_t* p = base + (size_t)s * stride;
        const uint32_t jmax = cs ? cs - 1u : 0u;
        // wave-uniform trip count: the longest group of this wave
        const uint32_t trips = wave_max_u32((cs + tps * U - 1u) / (tps * U));
        // indices clamped, values masked: the loads never become branches
        // that wait for each load in turn
        auto load = [&](uint32_t it, uint64_t (&c)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t j = g + (it * U + (uint32_t)u) * tps;
                const uint64_t x = p[j < cs ? j : jmax];
                c[u] = j < cs ? x : 0ull;
            }
        };
        auto use = [&](const uint64_t (&c)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) f(cand_key(c[u]), cand_low(c[u]));
        };
        uint64_t ca[U], cb[U];
        if (trips) load(0, ca);
        for (uint32_t it = 0; it < trips; it += 2) {
            if (it + 1 < trips) load(it + 1, cb);
            use(ca);
            if (it + 2 < trips) load(it + 2, ca);
            if (it + 1 < trips) use(cb);
        }
    }
    QRITA_DEV uint32_t wave_share() const { return (n + (uint32_t)(NT / kWave) - 1u) / (uint32_t)(NT / kWave); }
};

// The row's logits themselves (the full-row fallback).
template <int NT>
struct SrcRow {
    static constexpr bool kLows = true;
    const void* row;
    uint32_t V;
    int dtype;
    uint32_t n;
    template <class F>
    QRITA_DEV void visit(F&& f) const {
        constexpr int U = 16;  // logits per thread per batch; the next batch is in flight meanwhile
        const uint32_t lane = tid_here() & (kWave - 1);
        const uint32_t wb = wave_base_here();
        // indices clamped, values masked (unconditional loads stay in flight together)
        auto load = [&](uint32_t i0, uint32_t (&b)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = i0 + (uint32_t)u * NT + lane;
                const uint32_t ic = i < V ? i : V - 1u;
                uint32_t x;
                if (dtype == 0) {
                    x = ((const uint32_t*)row)[ic];
                } else {
                    const uint32_t h = ((const uint16_t*)row)[ic];
                    x = __float_as_uint(dtype == 1 ? lo16<1>(h) : lo16<2>(h));
                }
                b[u] = i < V ? x : 0u;
            }
        };
        auto use = [&](uint32_t i0, const uint32_t (&b)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = i0 + (uint32_t)u * NT + lane;
                f(i < V ? f32_key(b[u]) : 0u, ~i);
            }
        };
        const uint32_t step = NT * U;
        uint32_t ba[U], bb[U];
        if (wb < V) load(wb, ba);
        for (uint32_t i0 = wb; i0 < V; i0 += 2 * step) {
            if (i0 + step < V) load(i0 + step, bb);
            use(i0, ba);
            if (i0 + 2 * step < V) load(i0 + 2 * step, ba);
            if (i0 + step < V) use(i0 + step, bb);
        }
    }
    QRITA_DEV uint32_t wave_share() const { return (n + (uint32_t)(NT / kWave) - 1u) / (uint32_t)(NT / kWave); }
};

// ---------------------------------------------------------------------------
// Per-wave search state. A wave visits either its share of the base source or
// its own LDS segment, which holds the wave's candidates inside the range of
// the last compaction (keys, or keys with their softmax masses). Candidates
// above that range were dropped and are added back as counts (and masses).
// ---------------------------------------------------------------------------
struct WaveSet {
    uint32_t on_seg;  // 1: the wave visits its segment
    uint32_t n;       // entries in the segment
    uint32_t above;   // this wave's dropped candidates above the segment's range
    uint64_t above_m; // and their fixed-point mass
};

QRITA_DEV WaveSet wave_set_base() { return WaveSet{0u, 0u, 0u, 0ull}; }

// Visit the wave's current set: f(key, low, mass). Segment entries are keys
// (MASS false, four per 16 bytes) or (key, mass) pairs (two per 16 bytes);
// base entries carry no mass (mass = -1: compute it).
template <bool MASS, class S, class F>
QRITA_DEV void visit_set(const S& src, const WaveSet& ws, const uint32_t* seg, F&& f) {
    if (ws.on_seg) {
        const uint32_t lane = tid_here() & (kWave - 1);
        const uint32_t nv = MASS ? (ws.n + 1u) / 2u : (ws.n + 3u) / 4u;
        for (uint32_t v0 = 0; v0 < nv; v0 += kWave) {
            const uint32_t v = v0 + lane;
            const uint4 qr = ((const uint4*)seg)[v < nv ? v : nv - 1u];  // clamped: no branch
            const uint4 q = v < nv ? qr : make_uint4(0u, 0u, 0u, 0u);
            if (MASS) {
                f(q.x, 0u, __uint_as_float(q.y));
                f(q.z, 0u, __uint_as_float(q.w));
            } else {
                f(q.x, 0u, -1.0f);
                f(q.y, 0u, -1.0f);
                f(q.z, 0u, -1.0f);
                f(q.w, 0u, -1.0f);
            }
        }
    } else {
        src.visit([&](uint32_t key, uint32_t low) { f(key, low, -1.0f); });
    }
}

// ---------------------------------------------------------------------------
// One pivot evaluation of the quaternary search (§2), in one pass over the
// wave sets and one block combination. With t_0 the current lower end and
// t_1 <= t_2 <= t_3 the pivots it returns G_i = #{f > t_i} (and for the mass
// search M_i, the fixed-point mass above t_i), and for each pivot the smallest
// value above it (the z_mn of §2) and the largest value at or below it. The
// minima come from wrap-around differences: f - (p + 1) is small exactly for
// values above p, p - f exactly for values at or below it, so no lane masks
// are needed. NP = 1 evaluates a single pivot (a binary search step); its
// results are copied to all three pivot slots.
//
// FIELD 1 searches the complemented indices of the candidates whose key is
// v_eq (duplicate resolution); FIELD 0 searches keys.
//
// With MASS, a candidate's mass exp(z - m) is taken from the segment or
// computed (only for keys above t_0). With FILL (a mass search's first
// evaluation on the base source), the wave also writes its candidates above
// t_0 with their masses into its segment, as far as they fit.
// ---------------------------------------------------------------------------
struct Eval4 {
    uint32_t G[4];
    uint64_t M[4];
    uint32_t mn[3];  // smallest value above pivot i
    uint32_t mx[3];  // largest value at or below pivot i (0: none)
    uint32_t Gw[4];  // this wave's counts
    uint32_t filled; // FILL: candidates the wave wrote to its segment (may exceed the segment)
};

template <int FIELD>
QRITA_DEV uint32_t field_of(uint32_t key, uint32_t low, uint32_t v_eq) {
    if (FIELD == 0) return key;
    return key == v_eq ? low : 0u;
}

template <int NT, int NP, bool MASS, bool FILL, int FIELD, class S>
QRITA_DEV Eval4 evaluate(const S& src, const WaveSet& ws, uint32_t* seg, uint32_t segcap, uint32_t v_eq, uint32_t t0,
                         uint32_t p0, uint32_t p1, uint32_t p2, float m, Shared& sh, int rb) {
    uint32_t g0 = 0, g1 = 0, g2 = 0, g3 = 0;
    uint32_t a0 = 0xFFFFFFFFu, a1 = 0xFFFFFFFFu, a2 = 0xFFFFFFFFu;
    uint32_t c0 = 0xFFFFFFFFu, c1 = 0xFFFFFFFFu, c2 = 0xFFFFFFFFu;
    uint64_t q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    uint32_t run = 0;
    const uint32_t s0 = p0 + 1u, s1 = p1 + 1u, s2 = p2 + 1u;
    visit_set<MASS>(src, ws, seg, [&](uint32_t key, uint32_t low, float ec) {
        const uint32_t f = field_of<FIELD>(key, low, v_eq);
        const uint32_t b0 = gt01(f, t0), b1 = gt01(f, p0);
        g0 += b0;
        g1 += b1;
        const uint32_t u0 = f - s0;
        a0 = u0 < a0 ? u0 : a0;
        const uint32_t w0 = p0 - f;
        c0 = w0 < c0 ? w0 : c0;
        uint32_t b2 = 0, b3 = 0;
        if constexpr (NP == 3) {
            b2 = gt01(f, p1);
            b3 = gt01(f, p2);
            g2 += b2;
            g3 += b3;
            const uint32_t u1 = f - s1, u2 = f - s2;
            a1 = u1 < a1 ? u1 : a1;
            a2 = u2 < a2 ? u2 : a2;
            const uint32_t w1 = p1 - f, w2 = p2 - f;
            c1 = w1 < c1 ? w1 : c1;
            c2 = w2 < c2 ? w2 : c2;
        }
        if constexpr (MASS) {
            float e = ec;
            if (e < 0.0f) e = b0 ? mass_f32(key, m) : 0.0f;
            const uint64_t x = fx_from_unit_f32(e);
            q0 += b0 ? x : 0ull;
            q1 += b1 ? x : 0ull;
            if constexpr (NP == 3) {
                q2 += b2 ? x : 0ull;
                q3 += b3 ? x : 0ull;
            }
            if constexpr (FILL) {
                const uint64_t bb = __ballot(b0 != 0u);
                const uint32_t pos = run + lanes_below(bb);
                if (b0 && pos < segcap) *(uint2*)(seg + 2 * pos) = make_uint2(key, __float_as_uint(e));
                run += (uint32_t)__popcll(bb);
            }
        }
    });
    uint32_t s32[4] = {wave_sum_u32(g0) + ws.above, wave_sum_u32(g1) + ws.above, 0u, 0u};
    uint32_t mn[6] = {wave_min_u32(a0), 0xFFFFFFFFu, 0xFFFFFFFFu, wave_min_u32(c0), 0xFFFFFFFFu, 0xFFFFFFFFu};
    if constexpr (NP == 3) {
        s32[2] = wave_sum_u32(g2) + ws.above;
        s32[3] = wave_sum_u32(g3) + ws.above;
        mn[1] = wave_min_u32(a1);
        mn[2] = wave_min_u32(a2);
        mn[4] = wave_min_u32(c1);
        mn[5] = wave_min_u32(c2);
    }
    Eval4 E;
#pragma unroll
    for (int i = 0; i < 4; ++i) E.Gw[i] = s32[i];
    E.filled = run;
    if constexpr (MASS) {
        uint64_t s64[4] = {wave_sum_u64(q0) + ws.above_m, wave_sum_u64(q1) + ws.above_m, 0ull, 0ull};
        if constexpr (NP == 3) {
            s64[2] = wave_sum_u64(q2) + ws.above_m;
            s64[3] = wave_sum_u64(q3) + ws.above_m;
        }
        comb_record<NT, 4, 4, 6>(s32, s64, mn, sh, rb);
#pragma unroll
        for (int i = 0; i < 4; ++i) E.M[i] = s64[i];
    } else {
        comb_record<NT, 4, 0, 6>(s32, nullptr, mn, sh, rb);
#pragma unroll
        for (int i = 0; i < 4; ++i) E.M[i] = 0ull;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) E.G[i] = s32[i];
    E.mn[0] = mn[0] + s0;
    E.mn[1] = mn[1] + s1;
    E.mn[2] = mn[2] + s2;
    E.mx[0] = mn[3] <= p0 ? p0 - mn[3] : 0u;
    E.mx[1] = mn[4] <= p1 ? p1 - mn[4] : 0u;
    E.mx[2] = mn[5] <= p2 ? p2 - mn[5] : 0u;
    if constexpr (NP == 1) {
        E.G[2] = E.G[3] = E.G[1];
        E.Gw[2] = E.Gw[3] = E.Gw[1];
        E.M[2] = E.M[3] = E.M[1];
        E.mn[1] = E.mn[2] = E.mn[0];
        E.mx[1] = E.mx[2] = E.mx[0];
    }
    return E;
}

// Move the wave's candidates with lo < f <= hi into its segment (in place
// when the wave already visits its segment: entries only move down, and a
// wave reads each group of entries before it writes any of them); the
// candidates above hi are dropped and counted. With MASS the entries carry
// their masses (computed here for base entries). Returns false, changing
// nothing, when the candidates do not fit the segment.
template <bool MASS, class S>
QRITA_DEV bool compact_wave(const S& src, WaveSet& ws, uint32_t* seg, uint32_t segcap, uint32_t lo, uint32_t hi,
                            float m) {
    uint32_t run = 0, above = 0;
    uint64_t above_m = 0;
    visit_set<MASS>(src, ws, seg, [&](uint32_t key, uint32_t, float ec) {
        const bool keep = key > lo && key <= hi;
        const bool up = key > hi;
        float e = ec;
        if (MASS && e < 0.0f && (keep || up)) e = mass_f32(key, m);
        if (MASS && up) above_m += fx_from_unit_f32(e);
        above += up ? 1u : 0u;
        const uint64_t bb = __ballot(keep);
        const uint32_t pos = run + lanes_below(bb);
        if (keep && pos < segcap) {
            if (MASS)
                *(uint2*)(seg + 2 * pos) = make_uint2(key, __float_as_uint(e));
            else
                seg[pos] = key;
        }
        run += (uint32_t)__popcll(bb);
    });
    if (run > segcap) return false;  // only a base source can overflow (nothing of the segment was overwritten)
    // zero padding after the last entry, up to the next 16-byte group
    const uint32_t lane = tid_here() & (kWave - 1);
    if (MASS) {
        if (lane == 0 && (run & 1u) && run < segcap) *(uint2*)(seg + 2 * run) = make_uint2(0u, 0u);
    } else {
        if (lane < 3 && run + lane < ((run + 3u) & ~3u) && run + lane < segcap) seg[run + lane] = 0u;
    }
    ws.on_seg = 1u;
    ws.n = run;
    ws.above += wave_sum_u32(above);
    if (MASS) ws.above_m += wave_sum_u64(above_m);
    return true;
}

// Three pivots at 25/50/75 % of the open range (lo, hi) of field values
// (hi - lo >= 2): of the key range (mode 0), or of the value range (mode 1,
// keys only, finite ends). Pivots lie strictly inside and do not descend.
// Mode 2 is the binary search's single pivot at 50 % of the key range.
QRITA_DEV void make_pivots(uint32_t lo, uint32_t hi, int mode, int field, uint32_t piv[3]) {
    const uint32_t span = hi - lo;
    if (mode == 2) {
        uint32_t pm = lo + (span >> 1);
        pm = pm <= lo ? lo + 1 : pm;
        pm = pm >= hi ? hi - 1 : pm;
        piv[0] = piv[1] = piv[2] = pm;
        return;
    }
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

// A wave compacts its set only when it holds at least this many candidates
// (four per lane): below that an evaluation costs little more than the
// compaction pass itself.
constexpr uint32_t kCompactMin = 256;

template <class T>
QRITA_DEV T pick4(int j, T a, T b, T c, T d) {
    return j == 3 ? d : (j == 2 ? c : (j == 1 ? b : a));
}

// The search context of one row: its candidate source and LDS regions.
template <class T, class S>
struct Ctx {
    S src;
    uint32_t* seg;     // this wave's segment
    uint32_t segcap;   // entries of 8 bytes
    int mode;          // pivot placement
    Shared* sh;
    int rb;
    int iters;
};

template <class T>
QRITA_DEV uint32_t* wave_segment() {
    return (uint32_t*)(dyn_lds() + T::W_OFF + (size_t)(wave_base_here() / kWave) * T::SEG * 8);
}

struct CountOut {
    uint32_t v, n_gt, N;
};

// Dispatch of the evaluation: one pivot for mode 2, three otherwise.
template <int NT, bool MASS, bool FILL, int FIELD, class C>
QRITA_DEV Eval4 eval_step(C& c, const WaveSet& ws, uint32_t segcap, uint32_t v_eq, uint32_t t0, const uint32_t piv[3],
                          float m) {
    Eval4 E;
    if (c.mode == 2)
        E = evaluate<NT, 1, MASS, FILL, FIELD>(c.src, ws, c.seg, segcap, v_eq, t0, piv[0], piv[1], piv[2], m, *c.sh,
                                               c.rb);
    else
        E = evaluate<NT, 3, MASS, FILL, FIELD>(c.src, ws, c.seg, segcap, v_eq, t0, piv[0], piv[1], piv[2], m, *c.sh,
                                               c.rb);
    c.rb ^= 1;
    ++c.iters;
    return E;
}

// Quaternary pivot search for the K-th largest field value (K >= 1) among
// the source's candidates, with duplicates (§2): returns v, n_gt = #{> v} and
// N = #{== v}, so #{> v} < K <= #{>= v}. Invariant: G(lo) >= K > G(hi) with
// G(x) = #{field > x}; hi is 0xFFFFFFFF or a value present.
//
// Each iteration evaluates pivots at 25/50/75 % of (lo, hi). Let j* be the
// highest pivot with G >= K (none: the lower end). The K-th value lies in
// (t_j*, t_j*+1]: the range jumps to [z_mn, z_mx], the smallest value above
// t_j* and the largest at or below t_j*+1. When the two coincide the
// interval holds one distinct value and the search ends there. Otherwise z_mn
// becomes the lower end, and its multiplicity N_zmn = G(t_j*) - G(z_mn) comes
// from the next evaluation, which counts above the lower end as well: if then
// G(z_mn) < K, the search ends at v = z_mn (the termination test of §2,
// #{> z_mn} < K <= #{>= z_mn}). After each step every wave keeps only its
// candidates inside the new range (FIELD 0).
template <int NT, int FIELD, class C>
QRITA_DEV CountOut search_count(C& c, uint32_t v_eq, uint32_t K, int64_t lo_in, uint32_t G_lo, int64_t hi_in,
                                uint32_t G_hi) {
    // every field value is nonzero, so a lower end below 0 is the same as 0
    uint32_t lo = lo_in > 0 ? (uint32_t)lo_in : 0u;
    uint32_t hi = (uint32_t)hi_in;
    bool conf = true;   // G(lo) = G_lo is known (then G_lo >= K)
    uint32_t G_up = 0;  // lo not confirmed: G at the pivot below lo
    WaveSet ws = wave_set_base();
    const uint32_t kcap = 2u * c.segcap;  // keys fit two per 8-byte entry
    uint32_t share = c.src.wave_share();
#pragma unroll 1
    for (int guard = 0; guard < 80; ++guard) {
        if (conf && hi - lo <= 1) return CountOut{hi, G_hi, G_lo - G_hi};
        uint32_t piv[3] = {hi, hi, hi};
        if (hi - lo >= 2) make_pivots(lo, hi, c.mode, FIELD, piv);
        const Eval4 E = eval_step<NT, false, false, FIELD>(c, ws, kcap, v_eq, lo, piv, 0.0f);
        if (!conf) {
            if (E.G[0] < K) return CountOut{lo, E.G[0], G_up - E.G[0]};
            conf = true;
            G_lo = E.G[0];
        }
        const int js = E.G[3] >= K ? 3 : (E.G[2] >= K ? 2 : (E.G[1] >= K ? 1 : 0));
        const uint32_t up = js < 3 ? pick4(js, E.mx[0], E.mx[1], E.mx[2], 0u) : hi;
        const uint32_t G_n = js < 3 ? pick4(js, E.G[1], E.G[2], E.G[3], 0u) : G_hi;
        if (js >= 1) {
            const uint32_t mn = pick4(js - 1, E.mn[0], E.mn[1], E.mn[2], 0u);
            const uint32_t Gj = pick4(js - 1, E.G[1], E.G[2], E.G[3], 0u);
            if (mn == up) return CountOut{mn, G_n, Gj - G_n};
            lo = mn;
            conf = false;
            G_up = Gj;
        }
        if (js < 3) {
            hi = up;
            G_hi = G_n;
        }
        if constexpr (FIELD == 0) {
            // this wave's candidates in the new range (lo, hi] are among those
            // in (t_js, t_js+1]
            const uint32_t bound = pick4(js, E.Gw[0], E.Gw[1], E.Gw[2], E.Gw[3]) -
                                   pick4(js, E.Gw[1], E.Gw[2], E.Gw[3], ws.above);
            if (share >= kCompactMin && bound <= kcap && bound * 4u <= share * 3u) {
                if (compact_wave<false>(c.src, ws, c.seg, kcap, lo, hi, 0.0f)) share = ws.n;
            }
        }
    }
    return CountOut{hi, G_hi, G_lo - G_hi};  // not reached for consistent inputs
}

struct MassOut {
    uint32_t v, n_gt, N;
    uint64_t M_gt;
};

// What the mass search works on: the source's candidates above lo, except
// that of the dN + (kept) candidates with value vx only the kept ones count
// (the top-k set's boundary duplicates; dN = 0 when top-k is off). The
// candidates of value vx are the lowest of the set, so the correction applies
// exactly to thresholds below vx, which only the lower end can be.
struct MassSet {
    double p;       // target fraction
    double rest;    // mass outside the source (top-p-only rows), relative to m
    bool need_all;  // the source must hold mass p itself (else a miss)
    uint32_t vx, dN;
};

// The quaternary search over softmax mass (top-p): finds the key v with
// M(> v) < T <= M(>= v), T = p * (M(set) + rest). The masses are integers, so
// M >= T is tested as M >= Tq = ceil(T). The first evaluation computes every
// candidate's mass, the set's total and, where they fit, writes the
// candidates with their masses to the wave segments. Returns false on a miss
// (need_all and the source holds less than T).
template <int NT, class C>
QRITA_DEV bool search_mass(C& c, const MassSet& ms, float m, int64_t lo_in, int64_t hi_in, MassOut& out,
                           uint64_t& Tq, double* Stot = nullptr) {
    uint32_t lo = lo_in > 0 ? (uint32_t)lo_in : 0u;
    uint32_t hi = (uint32_t)hi_in;
    const uint64_t ex = ms.dN ? (uint64_t)ms.dN * mass_fx(ms.vx, m) : 0ull;
    uint64_t M_hi = 0;
    uint32_t G_hi = 0, G_lo = 0, G_up = 0;
    bool conf = true;
    WaveSet ws = wave_set_base();
    uint32_t share = c.src.wave_share();
#pragma unroll 1
    for (int guard = 0; guard < 80; ++guard) {
        if (guard > 0 && conf && hi - lo <= 1) {
            out = MassOut{hi, G_hi, G_lo - G_hi, M_hi};
            return true;
        }
        uint32_t piv[3] = {hi, hi, hi};
        if (hi - lo >= 2) make_pivots(lo, hi, c.mode, 0, piv);
        Eval4 E;
        if (guard == 0) {
            E = eval_step<NT, true, true, 0>(c, ws, c.segcap, 0u, lo, piv, m);
            // the candidates above lo now sit in the wave's segment, if they fit
            if (E.filled <= c.segcap) {
                if ((tid_here() & (kWave - 1)) == 0 && (E.filled & 1u) && E.filled < c.segcap)
                    *(uint2*)(c.seg + 2 * E.filled) = make_uint2(0u, 0u);
                ws.on_seg = 1u;
                ws.n = E.filled;
                share = E.filled;
            }
        } else {
            E = eval_step<NT, true, false, 0>(c, ws, c.segcap, 0u, lo, piv, m);
        }
        if (lo < ms.vx) {
            E.G[0] -= ms.dN;
            E.M[0] -= ex;
        }
        if (guard == 0) {
            const double tot = (double)E.M[0] + ms.rest;
            if (Stot) *Stot = tot;
            Tq = (uint64_t)ceil(ms.p * tot);
            Tq = Tq ? Tq : 1u;  // at least one unit of mass: the first token with mass
            if (ms.need_all && E.M[0] < Tq) return false;
        }
        if (!conf) {
            if (E.M[0] < Tq) {
                out = MassOut{lo, E.G[0], G_up - E.G[0], E.M[0]};
                return true;
            }
            conf = true;
        }
        G_lo = E.G[0];
        const int js = E.M[3] >= Tq ? 3 : (E.M[2] >= Tq ? 2 : (E.M[1] >= Tq ? 1 : 0));
        const uint32_t up = js < 3 ? pick4(js, E.mx[0], E.mx[1], E.mx[2], 0u) : hi;
        const uint32_t G_n = js < 3 ? pick4(js, E.G[1], E.G[2], E.G[3], 0u) : G_hi;
        const uint64_t M_n = js < 3 ? pick4<uint64_t>(js, E.M[1], E.M[2], E.M[3], 0) : M_hi;
        if (js >= 1) {
            const uint32_t mn = pick4(js - 1, E.mn[0], E.mn[1], E.mn[2], 0u);
            const uint32_t Gj = pick4(js - 1, E.G[1], E.G[2], E.G[3], 0u);
            if (mn == up) {
                out = MassOut{mn, G_n, Gj - G_n, M_n};
                return true;
            }
            lo = mn;
            conf = false;
            G_up = Gj;
        }
        if (js < 3) {
            hi = up;
            G_hi = G_n;
            M_hi = M_n;
        }
        // keep the wave's candidates in (lo, hi] (with masses); the
        // correction for the duplicates at vx stays valid: it applies only
        // while lo < vx, and until then the candidates at vx are kept
        const uint32_t bound = pick4(js, E.Gw[0], E.Gw[1], E.Gw[2], E.Gw[3]) -
                                   pick4(js, E.Gw[1], E.Gw[2], E.Gw[3], ws.above);
        if (share >= kCompactMin && bound <= c.segcap && bound * 4u <= share * 3u) {
            if (compact_wave<true>(c.src, ws, c.seg, c.segcap, lo, hi, m)) share = ws.n;
        }
    }
    out = MassOut{hi, G_hi, G_lo - G_hi, M_hi};  // not reached for consistent inputs
    return true;
}

// ---------------------------------------------------------------------------
// Rank order of a set of distinct words (key << 32 | ~index): descending
// words are descending values with ties by ascending index, a total order.
// ---------------------------------------------------------------------------
QRITA_DEV uint32_t next_pow2(uint32_t x) {
    uint32_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

QRITA_DEV uint32_t bits_for(uint64_t x) { return x ? 64u - (uint32_t)__builtin_clzll(x) : 0u; }

// Exclusive prefix sum, in place, of the n counts v[0 .. n) (n <= NB); v[n]
// becomes the total. Returns the largest count (uniform). One block round.
template <int NT, int NB>
QRITA_DEV uint32_t scan_counts(uint32_t* v, uint32_t n, Shared& sh, int& rb) {
    constexpr int PER = NB / NT;
    const uint32_t t = threadIdx.x;
    const uint32_t per = (n + NT - 1) / NT;
    uint32_t c[PER];
    uint32_t sum = 0, big = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const uint32_t i = t * per + (uint32_t)j;
        c[j] = ((uint32_t)j < per && i < n) ? v[i] : 0u;
        sum += c[j];
        big = c[j] > big ? c[j] : big;
    }
    uint32_t incl = sum;
    {
        uint32_t x = incl;
        QRITA_WAVE_STEPS(op_add, 0u)  // inclusive prefix over the wave
        incl = x;
    }
    const uint32_t wtot = readlane(incl, 63), wbig = wave_max_u32(big);
    uint32_t run = incl - sum;
    uint32_t total = 0;
    {
        constexpr int NW = NT / kWave;
        const uint32_t lane = t & (kWave - 1), wave = t / kWave;
        uint32_t* rec = &sh.slot[rb][0][0];
        if (lane == 0) *(uint2*)(rec + wave * 2) = make_uint2(wtot, wbig);
        lds_sync();
        uint32_t mm = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint2 q = *(const uint2*)(rec + w * 2);
            run += (uint32_t)w < wave ? q.x : 0u;
            total += q.x;
            mm = q.y > mm ? q.y : mm;
        }
        rb ^= 1;
        big = uni(mm);
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const uint32_t i = t * per + (uint32_t)j;
        if ((uint32_t)j < per && i < n) v[i] = run;
        run += c[j];
    }
    if (t == 0) v[n] = uni(total);
    lds_sync();
    return big;
}

// Where a sort puts the word w of rank r: index r of the index output
// (r < lout); the mask byte when r < lmask (scattered bytes, mrow); and, with
// `last`, the word of rank lmask - 1 (the kept set's boundary word, for a
// bitmap mask afterwards).
struct RankOut {
    int32_t* out;
    uint32_t lout;
    uint8_t* mrow;   // scattered mask bytes (null: none)
    uint32_t lmask;
    uint64_t* last;  // LDS word (null: none)
    float* prob;     // probabilities beside the indices (null: none)
    float mref;      // the row maximum the masses are taken against
    double inv_s;    // 1 / the kept set's fixed-point mass
    uint64_t* sorted;  // LDS: word of rank r to sorted[r] (null: none)
    QRITA_DEV void put(uint32_t r, uint64_t w) const {
        if (sorted) sorted[r] = w;
        if (r < lout) {
            out[r] = (int32_t)cand_idx(w);
            if (prob) prob[r] = (float)((double)mass_fx(cand_key(w), mref) * inv_s);
        }
        if (mrow && r < lmask) mrow[cand_idx(w)] = 1;
        if (last && r + 1 == lmask) *last = w;
    }
};

// Up to NT words: each word's rank is the number of larger words, counted by
// NT / next_pow2(cnt) threads per word over a share of the words each, the
// shares added in LDS.
template <int NT>
QRITA_DEV void rank_sort(uint64_t* a, uint32_t cnt, const RankOut& ro, uint32_t* acc) {
    const uint32_t P = (uint32_t)NT / next_pow2(cnt);
    const uint32_t t = threadIdx.x, e = t / P, q = t % P;
    const uint32_t span = (((cnt + P - 1) / P) + 7u) & ~7u;
    if (t < 8u) a[cnt + t] = 0ull;
    if (q == 0 && e < cnt) acc[e] = 0u;
    lds_sync();
    uint64_t x = 0;
    if (e < cnt) {
        x = a[e];
        const uint32_t j0 = q * span, j1 = min(j0 + span, (cnt + 7u) & ~7u);
        uint32_t above = 0;
        for (uint32_t j = j0; j < j1; j += 8) {
            const uint4* v = (const uint4*)(a + j);
            const uint4 v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
            const uint64_t y[8] = {((uint64_t)v0.y << 32) | v0.x, ((uint64_t)v0.w << 32) | v0.z,
                                   ((uint64_t)v1.y << 32) | v1.x, ((uint64_t)v1.w << 32) | v1.z,
                                   ((uint64_t)v2.y << 32) | v2.x, ((uint64_t)v2.w << 32) | v2.z,
                                   ((uint64_t)v3.y << 32) | v3.x, ((uint64_t)v3.w << 32) | v3.z};
#pragma unroll
            for (int u = 0; u < 8; ++u) above += y[u] > x ? 1u : 0u;
        }
        if (above) atomicAdd(&acc[e], above);
    }
    lds_sync();
    if (q == 0 && e < cnt) ro.put(acc[e], x);
    lds_sync();
}

// Bitonic sort, descending, of the np (a power of two, at most twice the
// set) words a[0 .. np) in LDS, one barrier per stage; then the rank of
// position g is g. For sets the bucket sort cannot split.
template <int NT>
QRITA_DEV void bitonic_lds(uint64_t* a, uint32_t np, uint32_t cnt, const RankOut& ro) {
    const uint32_t t = threadIdx.x;
    for (uint32_t k = 2; k <= np; k <<= 1) {
        for (uint32_t j = k >> 1; j >= 1; j >>= 1) {
            for (uint32_t i = t; i < np / 2; i += NT) {
                // the i-th pair of this stage: lower position x, partner x | j
                const uint32_t x = ((i & ~(j - 1u)) << 1) | (i & (j - 1u));
                const uint32_t y = x | j;
                const uint64_t u = a[x], v = a[y];
                const bool desc = (x & k) == 0;
                if ((u < v) == desc) {
                    a[x] = v;
                    a[y] = u;
                }
            }
            lds_sync();
        }
    }
    for (uint32_t g = t; g < cnt; g += NT) ro.put(g, a[g]);
    lds_sync();
}

// Bucket sort, descending, of the cnt distinct words a[0 .. cnt) (LDS).
// Bins ascend as words descend. Keys are coded exactly as (kmax - key) >> z,
// z the number of low bits all keys share (16 for bf16 logits), coarsened by
// dropping low code bits if the codes outnumber the bins. Within a code,
// words spread by a sub-coordinate: the dropped code bits, then the index
// (lmax - low), so tie groups spread too. First every code gets the same
// number of bins; if a bin then holds more than kMaxBin words, each code
// instead gets a run of bins in proportion to how many words it holds (code
// starts in hc). The words (equal runs; bw) or their positions (proportional
// runs; pos) are scattered into bins; a word's rank is its bin's start plus
// the number of larger words in its bin, counted directly, so the result does
// not depend on the order of the LDS atomics that fill the bins. Returns
// false, having written nothing, when a bin still holds more than kMaxBin
// words.
constexpr uint32_t kMaxBin = 96;

// Extents of a set of words, gathered with it (block-uniform): key and
// complemented-index ranges, and the number of low key bits all keys share.
struct SortExt {
    uint32_t kmn, kmx, lmn, lmx, tz;
};

template <int NT, int NB>
QRITA_DEV bool bucket_sort(const uint64_t* a, uint32_t cnt, const SortExt& ex, const RankOut& ro, uint64_t* bw,
                           uint16_t* pos, uint16_t* binof, uint32_t* bins, uint32_t* hc, Shared& sh, int& rb,
                           bool* ordered) {
    const uint32_t t = threadIdx.x;
    const uint32_t kmn = ex.kmn, kmx = ex.kmx, lmn = ex.lmn, lmx = ex.lmx;
    const uint32_t nb = min((uint32_t)NB, 2u * next_pow2(cnt));
    for (uint32_t i = t; i <= nb; i += NT) bins[i] = 0u;
    const uint32_t kz = min(ex.tz, 31u);
    const uint32_t nbits = 31u - (uint32_t)__builtin_clz(nb);
    const uint32_t fine_max = (kmx - kmn) >> kz;
    const uint32_t cbits = bits_for((uint64_t)fine_max);
    const uint32_t kdrop = cbits > nbits ? cbits - nbits : 0u;
    const uint32_t ncodes = (fine_max >> kdrop) + 1u;
    const uint32_t lbits = bits_for((uint64_t)(lmx - lmn));
    // sub-coordinate: dropped code bits, then the index, within 48 bits
    const uint32_t sfull = kdrop + lbits;
    const uint32_t scut = sfull > 48u ? sfull - 48u : 0u;
    const uint32_t sbits = sfull - scut;
    auto code_of = [&](uint64_t w) { return ((kmx - cand_key(w)) >> kz) >> kdrop; };
    auto sub_of = [&](uint64_t w) {
        const uint32_t fine = (kmx - cand_key(w)) >> kz;
        const uint64_t dropped = kdrop ? (uint64_t)(fine & ((1u << kdrop) - 1u)) : 0ull;
        return ((dropped << lbits) | (uint64_t)(lmx - cand_low(w))) >> scut;
    };
    // every code the same run of bins: code bits, then the top sub bits
    const uint32_t lkeep = nbits - (cbits - kdrop);
    const uint32_t sshift = sbits > lkeep ? sbits - lkeep : 0u;
    auto bin_eq = [&](uint64_t w) {
        const uint32_t sc = lkeep ? (uint32_t)(sub_of(w) >> sshift) : 0u;
        return (code_of(w) << lkeep) | sc;
    };
    lds_sync();
    for (uint32_t i = t; i < cnt; i += 2 * NT) {
        const uint32_t i1 = i + NT;
        const uint32_t b0 = bin_eq(a[i]);
        const uint32_t b1 = i1 < cnt ? bin_eq(a[i1]) : 0u;
        atomicAdd(&bins[b0], 1u);
        if (i1 < cnt) atomicAdd(&bins[b1], 1u);
    }
    lds_sync();
    uint32_t big = scan_counts<NT, NB>(bins, nb, sh, rb);
    if (big <= kMaxBin) {
        // the usual case: the words themselves go to their bins (bw), so
        // that ranking reads each bin's words side by side; a word's bin is
        // recomputed from the word
        for (uint32_t i0 = t; i0 < cnt; i0 += 4 * NT) {
            uint64_t w[4];
            uint32_t q[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t i = i0 + (uint32_t)u * NT;
                w[u] = a[i < cnt ? i : i0];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t i = i0 + (uint32_t)u * NT;
                q[u] = i < cnt ? atomicAdd(&bins[bin_eq(w[u])], 1u) : 0u;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (i0 + (uint32_t)u * NT < cnt) bw[q[u]] = w[u];
        }
        lds_sync();
        // afterwards bins[i] is the end of bin i: a word's rank is its bin's
        // start plus the number of larger words in its bin
        for (uint32_t p0 = t; p0 < cnt; p0 += 4 * NT) {
            uint64_t w[4];
            uint32_t s0[4], e0[4], r[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t p = p0 + (uint32_t)u * NT;
                w[u] = bw[p < cnt ? p : p0];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t bi = bin_eq(w[u]);
                s0[u] = bi ? bins[bi - 1] : 0u;
                e0[u] = bins[bi];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                r[u] = s0[u];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint32_t q = s0[u] + (uint32_t)m;
                    const uint64_t y = bw[q < e0[u] ? q : s0[u]];
                    r[u] += (q < e0[u] && y > w[u]) ? 1u : 0u;
                }
                for (uint32_t q = s0[u] + 4; q < e0[u]; ++q) r[u] += bw[q] > w[u] ? 1u : 0u;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (p0 + (uint32_t)u * NT < cnt) ro.put(r[u], w[u]);
        }
        lds_sync();
        return true;
    }
    // below, ranking reads the words in place: no sorted copy over them
    const bool keep_sorted = ro.sorted != a;
    if (!keep_sorted) *ordered = false;
    {
        // runs of bins in proportion to the codes' sizes
        for (uint32_t i = t; i <= ncodes; i += NT) hc[i] = 0u;
        lds_sync();
        for (uint32_t i = t; i < cnt; i += NT) atomicAdd(&hc[code_of(a[i])], 1u);
        lds_sync();
        scan_counts<NT, NB>(hc, ncodes, sh, rb);
        const float ratio = (float)nb / (float)cnt;
        auto first = [&](uint32_t cc) {
            if (cc >= ncodes) return nb;
            const uint32_t f = (uint32_t)((float)hc[cc] * ratio);
            return f < nb - 1u ? f : nb - 1u;
        };
        for (uint32_t i = t; i <= nb; i += NT) bins[i] = 0u;
        lds_sync();
        for (uint32_t i = t; i < cnt; i += NT) {
            const uint64_t w = a[i];
            const uint32_t cc = code_of(w);
            const uint32_t f0 = first(cc), nsub = first(cc + 1u) - f0;
            const uint32_t off = sbits ? (uint32_t)((sub_of(w) * nsub) >> sbits) : 0u;
            binof[i] = (uint16_t)(f0 + off);
            atomicAdd(&bins[f0 + off], 1u);
        }
        lds_sync();
        big = scan_counts<NT, NB>(bins, nb, sh, rb);
        if (big > kMaxBin) return false;
    }
    // scatter the positions, four words per thread and step so that their
    // LDS round trips overlap; afterwards bins[i] is the end of bin i
    for (uint32_t i0 = t; i0 < cnt; i0 += 4 * NT) {
        uint32_t b[4], q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t i = i0 + (uint32_t)u * NT;
            b[u] = binof[i < cnt ? i : i0];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t i = i0 + (uint32_t)u * NT;
            q[u] = i < cnt ? atomicAdd(&bins[b[u]], 1u) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t i = i0 + (uint32_t)u * NT;
            if (i < cnt) pos[q[u]] = (uint16_t)i;
        }
    }
    lds_sync();
    // ranks, by position in the binned order: a word's rank is its bin's
    // start plus the number of larger bin mates. Four positions per thread
    // and step, each with its first four bin mates (the word itself stands in
    // past the bin's end), so that the chains of LDS reads overlap; longer
    // bins continue four mates at a time.
    for (uint32_t p0 = t; p0 < cnt; p0 += 4 * NT) {
        uint32_t i[4], s0[4], e0[4], r[4];
        uint64_t w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t p = p0 + (uint32_t)u * NT;
            i[u] = pos[p < cnt ? p : p0];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            w[u] = a[i[u]];
            const uint32_t bi = binof[i[u]];
            s0[u] = bi ? bins[bi - 1] : 0u;
            e0[u] = bins[bi];
        }
        uint32_t j[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int m = 0; m < 4; ++m) j[u][m] = s0[u] + m < e0[u] ? pos[s0[u] + m] : i[u];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            r[u] = s0[u];
#pragma unroll
            for (int m = 0; m < 4; ++m) r[u] += a[j[u][m]] > w[u] ? 1u : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            for (uint32_t q = s0[u] + 4; q < e0[u]; q += 4) {
                const uint32_t j0 = pos[q];
                const uint32_t j1 = q + 1 < e0[u] ? pos[q + 1] : i[u];
                const uint32_t j2 = q + 2 < e0[u] ? pos[q + 2] : i[u];
                const uint32_t j3 = q + 3 < e0[u] ? pos[q + 3] : i[u];
                r[u] += (a[j0] > w[u] ? 1u : 0u) + (a[j1] > w[u] ? 1u : 0u) + (a[j2] > w[u] ? 1u : 0u) +
                        (a[j3] > w[u] ? 1u : 0u);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (p0 + (uint32_t)u * NT < cnt) {
                if (keep_sorted)
                    ro.put(r[u], w[u]);
                else
                    RankOut{ro.out, ro.lout, ro.mrow, ro.lmask, ro.last, ro.prob, ro.mref, ro.inv_s, nullptr}.put(r[u], w[u]);
            }
    }
    lds_sync();
    return true;
}

// Rank order of the cnt <= CSORT words at the start of the sort region: a
// handful by ranking, more by the bucket sort, sets it cannot split by the
// bitonic sort. The words stay in the first region (the bitonic sort permutes
// them). Returns whether ro.sorted received the words in rank order (not when
// it is the sort region itself and the bucket sort sized its bins in
// proportion to the codes, which ranks the words in place).
template <class T>
QRITA_DEV bool sort_words(uint32_t cnt, const SortExt& ex, RankOut ro, Shared& sh, int& rb) {
    constexpr int NT = T::NT;
    uint64_t* a = (uint64_t*)(dyn_lds() + T::SA_OFF);
    uint16_t* pos = (uint16_t*)(dyn_lds() + T::SB_OFF);
    uint16_t* binof = (uint16_t*)(dyn_lds() + T::BO_OFF);
    uint32_t* bins = (uint32_t*)(dyn_lds() + T::BINS_OFF);
    uint32_t* hc = (uint32_t*)(dyn_lds() + T::HC_OFF);
    cnt = min(uni(cnt), (uint32_t)T::CSORT);  // more only for inputs outside the contract (NaN logits)
    if (cnt == 0) return true;
    if (cnt <= (uint32_t)NT) {
        rank_sort<NT>(a, cnt, ro, bins);
        return true;
    }
    uint64_t* bw = (uint64_t*)(dyn_lds() + T::SB_OFF);
    bool ordered = true;
    if (bucket_sort<NT, T::NB>(a, cnt, ex, ro, bw, pos, binof, bins, hc, sh, rb, &ordered)) return ordered;
    const uint32_t np = next_pow2(cnt);  // < 2 cnt: inside the fallback region
    for (uint32_t i = cnt + threadIdx.x; i < np; i += NT) a[i] = 0ull;
    lds_sync();
    bitonic_lds<NT>(a, np, cnt, ro);
    return true;
}

// ---------------------------------------------------------------------------
// Gathering words from a source into the sort region, and the mask.
// ---------------------------------------------------------------------------

// Words c with lo_w <= c < hi_w from the source (with indices) into
// a[0 .. ), reserved per wave in LDS; returns the count (uniform; at most
// cap are written) and the set's extents for the sort. The key of lo_w must
// be one of the set's keys (the reference for the shared low bits).
template <int NT, class L>
QRITA_DEV uint32_t gather_words(const L& lsrc, uint64_t* a, uint32_t cap, uint64_t lo_w, uint64_t hi_w, SortExt& ex,
                                Shared& sh, int& rb, uint32_t key_ref = 0u) {
    block_sync<NT>();
    if (threadIdx.x == 0) sh.gather_n = 0;
    lds_sync();
    const uint32_t lane = tid_here() & (kWave - 1);
    const uint32_t key0 = key_ref ? key_ref : cand_key(lo_w);
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u, lmn = 0xFFFFFFFFu, lmx = 0u, tz = 32u;
    lsrc.visit([&](uint32_t key, uint32_t low) {
        const uint64_t w = ((uint64_t)key << 32) | low;
        const bool take = key != 0 && w >= lo_w && w < hi_w;
        const uint64_t b = __ballot(take);
        if (b) {
            uint32_t r0 = 0;
            if (lane == 0) r0 = atomicAdd(&sh.gather_n, (uint32_t)__popcll(b));
            const uint32_t pos = readlane(r0, 0) + lanes_below(b);
            if (take && pos < cap) a[pos] = w;
            if (take) {
                kmn = key < kmn ? key : kmn;
                kmx = key > kmx ? key : kmx;
                lmn = low < lmn ? low : lmn;
                lmx = low > lmx ? low : lmx;
                const uint32_t d = key ^ key0;
                const uint32_t z = d ? (uint32_t)__builtin_ctz(d) : 32u;
                tz = z < tz ? z : tz;
            }
        }
    });
    uint32_t e[5] = {wave_min_u32(kmn), ~wave_max_u32(kmx), wave_min_u32(lmn), ~wave_max_u32(lmx), wave_min_u32(tz)};
    comb_record<NT, 0, 0, 5>(nullptr, nullptr, e, sh, rb);  // its barrier also completes the gather
    ex = SortExt{e[0], ~e[1], e[2], ~e[3], e[4]};
    return uni(sh.gather_n);
}

// Write the mask row from an LDS bitmap of the kept indices (whole row,
// 16-byte stores; one byte per logit, 1 = kept).
template <int NT>
QRITA_DEV void write_mask_row(uint8_t* mrow, const uint32_t* bm, uint32_t V) {
    const uint32_t t = threadIdx.x;
    const uint32_t head = (uint32_t)((16u - ((uintptr_t)mrow & 15u)) & 15u);
    const uint32_t h = head < V ? head : V;
    for (uint32_t i = t; i < h; i += NT) mrow[i] = (uint8_t)((bm[i >> 5] >> (i & 31u)) & 1u);
    const uint32_t nv = (V - h) / 16u;
    for (uint32_t v = t; v < nv; v += NT) {
        const uint32_t i = h + v * 16u;
        // the 16 bits of logits i .. i+15 (i need not be a multiple of 32;
        // the word after the last one lies inside the bitmap's region)
        const uint64_t two = ((uint64_t)bm[(i >> 5) + 1] << 32) | bm[i >> 5];
        const uint32_t bits = (uint32_t)(two >> (i & 31u)) & 0xFFFFu;
        uint32_t wd[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t nib = (bits >> (4 * q)) & 15u;
            wd[q] = (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
        }
        const u32x4_t wv = {wd[0], wd[1], wd[2], wd[3]};
        __builtin_nontemporal_store(wv, (u32x4_t*)(mrow + i));
    }
    for (uint32_t i = h + nv * 16u + t; i < V; i += NT) mrow[i] = (uint8_t)((bm[i >> 5] >> (i & 31u)) & 1u);
}

// A whole mask row of ones (keep-all rows).
template <int NT>
QRITA_DEV void fill_mask_row(uint8_t* mrow, uint32_t V, uint8_t val) {
    const uint32_t t = threadIdx.x;
    const uint32_t head = (uint32_t)((16u - ((uintptr_t)mrow & 15u)) & 15u);
    const uint32_t h = head < V ? head : V;
    for (uint32_t i = t; i < h; i += NT) mrow[i] = val;
    const uint32_t nv = (V - h) / 16u;
    const uint32_t w = 0x01010101u * val;
    const u32x4_t wv = {w, w, w, w};
    for (uint32_t v = t; v < nv; v += NT) __builtin_nontemporal_store(wv, (u32x4_t*)(mrow + h + v * 16u));
    for (uint32_t i = h + nv * 16u + t; i < V; i += NT) mrow[i] = val;
}

QRITA_DEV void clear_words(uint32_t* p, uint32_t n, uint32_t NT) {
    for (uint32_t i = threadIdx.x; i < n; i += NT) p[i] = 0u;
}

struct TailDiag {
    int32_t n_t;
    int32_t iters;
};

// Boundary word B of "the `need` lowest-index candidates with key v, plus
// everything above v" (so the kept set is {c >= B}). A small tie group is
// ranked directly in LDS; a large one by a quaternary search over the tied
// candidates' indices.
template <class T, class L>
QRITA_DEV uint64_t tie_boundary(const L& lsrc, uint32_t v, uint32_t need, uint32_t N, uint32_t V, int mode,
                                Shared& sh, int& rb, int& iters, bool exact = false) {
    constexpr int NT = T::NT;
    uint64_t b = (uint64_t)v << 32;
    if (need >= N && !exact) return b;  // all duplicates: the bound needs no index
    need = need < N ? need : N;
    if (N <= kTieDirect) {
        const uint32_t lane = tid_here() & (kWave - 1);
        block_sync<NT>();
        if (threadIdx.x == 0) sh.gather_n = 0;
        // zeros after the ties (below every complemented index) round the
        // list up to whole uint4 reads
        if (threadIdx.x < 4u && N + threadIdx.x < (uint32_t)kTieDirect + 4u) sh.ties[N + threadIdx.x] = 0u;
        lds_sync();
        lsrc.visit([&](uint32_t key, uint32_t low) {
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
        lds_sync();
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
        lds_sync();
        return b | uni(sh.u32[6]);
    }
    // complemented indices of a row lie in [~(V - 1), 0xFFFFFFFF]
    Ctx<T, L> c{lsrc, wave_segment<T>(), (uint32_t)T::SEG, mode == 2 ? 2 : 0, &sh, rb, 0};
    const int64_t lo = (int64_t)(0xFFFFFFFFu - (V - 1u)) - 1;
    const CountOut t = search_count<NT, 1>(c, v, need, lo, N, (int64_t)0xFFFFFFFFu, 0u);
    rb = c.rb;
    iters += c.iters;
    return b | t.v;
}

// Where the outputs of a row go.
struct RowOut {
    int32_t* idx;    // out_idx row or null
    uint32_t idx_cap;
    uint8_t* mrow;   // mask row or null (keep-all rows: filled elsewhere)
    bool bitmap;     // mask written whole from an LDS bitmap
    uint32_t V;
    float* prob;     // probabilities beside idx, or null
    float mref;
    double inv_s;
    const void* rowp;  // the row's logits (index-ordered probabilities)
    int dtype;
};

// Mask of the kept set {c >= B} from a pass over the candidates: bitmap, or
// bytes scattered into the row that pass 1 zero-filled.
template <class T, class L>
QRITA_DEV void mask_from_boundary(const L& lsrc, uint64_t B, const RowOut& o) {
    constexpr int NT = T::NT;
    if (!o.mrow) return;
    if (o.bitmap) {
        uint32_t* bm = (uint32_t*)(dyn_lds() + T::SB_OFF);
        lds_sync();
        clear_words(bm, (o.V + 31u) / 32u, NT);
        lds_sync();
        lsrc.visit([&](uint32_t key, uint32_t low) {
            const uint64_t w = ((uint64_t)key << 32) | low;
            if (key != 0 && w >= B) atomicOr(&bm[(~low) >> 5], 1u << ((~low) & 31u));
        });
        lds_sync();
        write_mask_row<NT>(o.mrow, bm, o.V);
    } else {
        lsrc.visit([&](uint32_t key, uint32_t low) {
            const uint64_t w = ((uint64_t)key << 32) | low;
            if (key != 0 && w >= B) o.mrow[~low] = 1;
        });
    }
}

// Bitmap mask of the sorted words at or above the boundary word B (the words
// are still in the first sort region; the bitmap follows it).
template <class T>
QRITA_DEV void mask_from_sorted(uint32_t cnt, uint64_t B, const RowOut& o) {
    constexpr int NT = T::NT;
    if (!o.mrow || !o.bitmap) return;
    const uint64_t* a = (const uint64_t*)(dyn_lds() + T::SA_OFF);
    uint32_t* bm = (uint32_t*)(dyn_lds() + T::SB_OFF);
    lds_sync();
    clear_words(bm, (o.V + 31u) / 32u, NT);
    lds_sync();
    for (uint32_t p = threadIdx.x; p < cnt; p += NT) {
        const uint64_t w = a[p];
        if (w >= B) {
            const uint32_t i = cand_idx(w);
            atomicOr(&bm[i >> 5], 1u << (i & 31u));
        }
    }
    lds_sync();
    write_mask_row<NT>(o.mrow, bm, o.V);
}

template <int NT>
QRITA_DEV void bitmap_outputs(const uint32_t* bm, const RowOut& o, uint32_t Lout, Shared& sh, int& rb);

// Probability of vocabulary entry i (index-ordered output reads its logit).
QRITA_DEV float prob_at(const RowOut& o, uint32_t i) {
    uint32_t x;
    if (o.dtype == 0) {
        x = ((const uint32_t*)o.rowp)[i];
    } else {
        const uint32_t h = ((const uint16_t*)o.rowp)[i];
        x = __float_as_uint(o.dtype == 1 ? lo16<1>(h) : lo16<2>(h));
    }
    return (float)((double)mass_fx(f32_key(x), o.mref) * o.inv_s);
}

// The outputs of a row in ascending index order (the kept set as in
// emit_row): the kept set {c >= B} becomes an LDS bitmap, which also gives
// the mask; each thread then takes a run of bitmap words, and an exclusive
// prefix of their bit counts over the block places its indices.
template <class T, class C, class L>
QRITA_DEV void emit_row_by_index(C& c, const L& lsrc, const RowOut& o, bool all, uint32_t vf, uint32_t needf,
                                 uint32_t Nf, uint32_t L_, TailDiag& dg) {
    constexpr int NT = T::NT;
    Shared& sh = *c.sh;
    const uint32_t V = o.V;
    const uint32_t Lout = o.idx ? (L_ < o.idx_cap ? L_ : o.idx_cap) : 0u;
    if (all) {  // every index is kept: 0, 1, ..., Lout - 1
        for (uint32_t r = threadIdx.x; r < Lout; r += NT) {
            o.idx[r] = (int32_t)r;
            if (o.prob) o.prob[r] = prob_at(o, r);
        }
        return;
    }
    if (!o.mrow && Lout == 0) return;
    const uint64_t B = tie_boundary<T>(lsrc, vf, needf, Nf, V, c.mode, sh, c.rb, dg.iters);
    uint32_t* bm = (uint32_t*)(dyn_lds() + T::SB_OFF);
    const uint32_t nw = (V + 31u) / 32u;
    lds_sync();
    clear_words(bm, nw + 1u, NT);  // one word past the row: write_mask_row reads it
    lds_sync();
    lsrc.visit([&](uint32_t key, uint32_t low) {
        const uint64_t w = ((uint64_t)key << 32) | low;
        if (key != 0 && w >= B) atomicOr(&bm[(~low) >> 5], 1u << ((~low) & 31u));
    });
    lds_sync();
    bitmap_outputs<NT>(bm, o, Lout, sh, c.rb);
}

// The mask (whole row, or bytes into the zero-filled row) and the first Lout
// kept indices in ascending order, from the kept set's bitmap bm in LDS:
// each thread takes a run of bitmap words, and an exclusive prefix of their
// bit counts over the block places its indices.
template <int NT>
QRITA_DEV void bitmap_outputs(const uint32_t* bm, const RowOut& o, uint32_t Lout, Shared& sh, int& rb) {
    const uint32_t nw = (o.V + 31u) / 32u;
    if (o.mrow) {
        if (o.bitmap) {
            write_mask_row<NT>(o.mrow, bm, o.V);
        } else {
            for (uint32_t i = threadIdx.x; i < nw; i += NT) {
                uint32_t bits = bm[i];
                while (bits) {
                    const uint32_t b = (uint32_t)__builtin_ctz(bits);
                    bits &= bits - 1u;
                    o.mrow[i * 32u + b] = 1;
                }
            }
        }
    }
    if (Lout == 0) return;
    const uint32_t per = (nw + NT - 1u) / NT;
    const uint32_t w0 = threadIdx.x * per < nw ? threadIdx.x * per : nw;
    const uint32_t w1 = w0 + per < nw ? w0 + per : nw;
    uint32_t cnt = 0;
    for (uint32_t i = w0; i < w1; ++i) cnt += (uint32_t)__builtin_popcount(bm[i]);
    // exclusive prefix of cnt over the block: lanes, then waves
    uint32_t x = cnt;
    QRITA_WAVE_STEPS(op_add, 0u)
    const uint32_t wave_tot = readlane(x, kWave - 1);
    uint32_t total = 0;
    const uint32_t before = wave_prefix<NT>(wave_tot, total, sh, rb);
    uint32_t r = before + x - cnt;
    for (uint32_t i = w0; i < w1 && r < Lout; ++i) {
        uint32_t bits = bm[i];
        while (bits && r < Lout) {
            const uint32_t b = (uint32_t)__builtin_ctz(bits);
            bits &= bits - 1u;
            const uint32_t ix = i * 32u + b;
            o.idx[r] = (int32_t)ix;
            if (o.prob) o.prob[r] = prob_at(o, ix);
            ++r;
        }
    }
}

// The outputs (a7) of a row whose kept set is {> vf} and the needf
// lowest-index of its Nf duplicates at vf (L = ngt + needf tokens), with
// `all` for rows that keep everything. The first Lout = min(L, idx_cap)
// ranks go to the index output. When every candidate at or above the value
// that bounds the index output fits one sort, the sort's rank order resolves
// the duplicates and writes the outputs; otherwise the duplicates are
// resolved by tie_boundary and the indices sorted in windows. With
// keep_sorted, returns whether the one sort also left the kept set's words in
// rank order at the start of the sort region.
template <class T, class C, class L>
QRITA_DEV bool emit_row(C& c, const L& lsrc, const RowOut& o, bool all, uint32_t vf, uint32_t ngt, uint32_t needf,
                        uint32_t Nf, uint32_t L_, int64_t key_lo, uint32_t n, uint32_t kmax, TailDiag& dg,
                        bool keep_sorted = false) {
    constexpr int NT = T::NT;
    Shared& sh = *c.sh;
    const uint32_t Lout = o.idx ? (L_ < o.idx_cap ? L_ : o.idx_cap) : 0u;
    const bool mask = o.mrow != nullptr && !all;
    if (!mask && Lout == 0) return false;
    // the boundary of the index output's last rank
    uint32_t vo = vf, ngo = ngt, needo = needf, No = Nf;
    if (Lout > 0 && (all || Lout < L_)) {
        // every candidate >= vf counts above vf - 1, the unkept duplicates too
        const CountOut r = search_count<NT, 0>(c, 0u, Lout, all ? key_lo : (int64_t)vf - 1, all ? n : ngt + Nf,
                                               (int64_t)kmax, 0u);
        vo = r.v;
        ngo = r.n_gt;
        needo = Lout - r.n_gt;
        No = r.N;
    }
    uint64_t* a = (uint64_t*)(dyn_lds() + T::SA_OFF);
    const uint32_t Gi = Lout > 0 ? ngo + No : ngt + Nf;
    const bool same = Lout == 0 || (!all && Lout == L_);  // the index boundary is the kept set's boundary
    if (Gi <= (uint32_t)T::CSORT && same) {
        // one sort over every candidate at or above the boundary value
        SortExt ex;
        const uint32_t cnt =
            gather_words<NT>(lsrc, a, T::CSORT, (uint64_t)(Lout > 0 ? vo : vf) << 32, ~0ull, ex, sh, c.rb);
        RankOut ro{o.idx, Lout, (mask && !o.bitmap) ? o.mrow : nullptr, mask ? L_ : 0u,
                   (mask && o.bitmap) ? (uint64_t*)&sh.u32[0] : nullptr, o.prob, o.mref, o.inv_s,
                   keep_sorted ? a : nullptr};
        const bool ord = sort_words<T>(cnt, ex, ro, sh, c.rb);
        if (mask && o.bitmap) {
            lds_sync();
            const uint64_t B = uni(*(const uint64_t*)&sh.u32[0]);
            mask_from_sorted<T>(min(cnt, (uint32_t)T::CSORT), B, o);
        }
        return keep_sorted && ord;  // then the kept set is a[0 .. L) in rank order
    }
    // the kept set's boundary word, for the mask
    if (mask) {
        const uint64_t B = tie_boundary<T>(lsrc, vf, needf, Nf, o.V, c.mode, sh, c.rb, dg.iters);
        mask_from_boundary<T>(lsrc, B, o);
    }
    if (Lout == 0) return false;
    if (Gi <= (uint32_t)T::CSORT) {
        SortExt ex;
        const uint32_t cnt = gather_words<NT>(lsrc, a, T::CSORT, (uint64_t)vo << 32, ~0ull, ex, sh, c.rb);
        sort_words<T>(cnt, ex, RankOut{o.idx, Lout, nullptr, 0u, nullptr, o.prob, o.mref, o.inv_s}, sh, c.rb);
        return false;
    }
    // windows of CSORT ranks, each bounded by its own boundary word. The
    // gathers and sorts reuse the LDS that may hold the search source's
    // keys, so each window's boundary is searched over the candidate list in
    // memory (lsrc), which nothing overwrites.
    const uint64_t Bo = tie_boundary<T>(lsrc, vo, needo, No, o.V, c.mode, sh, c.rb, dg.iters);
    Ctx<T, L> cl{lsrc, c.seg, c.segcap, c.mode, c.sh, c.rb, 0};
    uint64_t prev = ~0ull;
    for (uint32_t done = 0; done < Lout;) {
        const uint32_t cnt = min((uint32_t)T::CSORT, Lout - done);
        uint64_t Bn = Bo;
        if (done + cnt < Lout) {
            cl.rb = c.rb;
            const CountOut r = search_count<NT, 0>(cl, 0u, done + cnt, (int64_t)vo - 1, ngo + No, (int64_t)kmax, 0u);
            c.rb = cl.rb;
            dg.iters += cl.iters;
            cl.iters = 0;
            Bn = tie_boundary<T>(lsrc, r.v, done + cnt - r.n_gt, r.N, o.V, c.mode, sh, c.rb, dg.iters);
        }
        SortExt ex;
        const uint32_t got = gather_words<NT>(lsrc, a, T::CSORT, Bn, prev, ex, sh, c.rb);
        sort_words<T>(got, ex,
                      RankOut{o.idx + done, cnt, nullptr, 0u, nullptr, o.prob ? o.prob + done : nullptr, o.mref, o.inv_s},
                      sh, c.rb);
        prev = Bn;
        done += cnt;
    }
    return false;
}

// Exclusive prefix over the block of per-thread 64-bit values v (thread
// order); total is the block's sum (uniform).
template <int NT>
QRITA_DEV uint64_t block_scan_u64(uint64_t v, uint64_t& total, Shared& sh, int& rb) {
    constexpr int NW = NT / kWave;
    const uint32_t lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    uint64_t x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)x, o, kWave);
        const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(x >> 32), o, kWave);
        if (lane >= (uint32_t)o) x += ((uint64_t)hi << 32) | lo;
    }
    const uint64_t wtot = ((uint64_t)readlane((uint32_t)(x >> 32), kWave - 1) << 32) | readlane((uint32_t)x, kWave - 1);
    if (lane == 0) *(uint2*)&sh.slot[rb][wave][0] = make_uint2((uint32_t)wtot, (uint32_t)(wtot >> 32));
    lds_sync();
    uint64_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint2 q = *(const uint2*)&sh.slot[rb][w][0];
        const uint64_t t = ((uint64_t)q.y << 32) | q.x;
        before += (uint32_t)w < wave ? t : 0ull;
        all += t;
    }
    rb ^= 1;
    total = uni(all);
    return before + x - v;
}

// Smallest rank r < R whose running mass P_r (rank-order prefix of
// mass_fx over s[0 .. R), starting from the thread's exclusive prefix) is at
// least T, or R. Each thread walks its own run of ranks [r0, r1).
template <int NT>
QRITA_DEV uint32_t first_reaching(const uint64_t* s, uint32_t r0, uint32_t r1, uint64_t before, uint64_t T,
                                  float m, uint32_t R, Shared& sh, int& rb) {
    uint32_t hit = 0xFFFFFFFFu;
    uint64_t run = before;
    for (uint32_t r = r0; r < r1; ++r) {
        run += mass_fx(cand_key(s[r]), m);
        if (run >= T) {
            hit = r;
            break;
        }
    }
    uint32_t mn[1] = {wave_min_u32(hit)};
    comb_record<NT, 0, 0, 1>(nullptr, nullptr, mn, sh, rb);
    return mn[0] < R ? mn[0] : R;
}

// Logit of vocabulary entry i of a row, as a key.
QRITA_DEV uint32_t key_at(const void* rowp, int dtype, uint32_t i) {
    uint32_t x;
    if (dtype == 0) {
        x = ((const uint32_t*)rowp)[i];
    } else {
        const uint32_t h = ((const uint16_t*)rowp)[i];
        x = __float_as_uint(dtype == 1 ? lo16<1>(h) : lo16<2>(h));
    }
    return f32_key(x);
}

// The draw (and the probabilities) for a row whose kept set of L ranks the
// index output already holds in rank order (idx[0 .. L)): the masses of the
// kept logits in rank order go to LDS (free once the outputs are written;
// coalesced index reads, eight gathers in flight per thread), then their
// block prefix gives the first rank whose running mass reaches u * S. The
// same integers as the mass search over the kept set. Returns the drawn index.
template <int NT>
QRITA_DEV int32_t draw_from_ranks(const int32_t* idx, float* prob, uint32_t L, uint32_t lprob, const void* rowp,
                                  int dtype, float m, double u, Shared& sh, int& rb) {
    // the index output is this workgroup's own global stores: a full
    // workgroup barrier (release and acquire at workgroup scope) orders them
    __syncthreads();
    uint64_t* em = (uint64_t*)dyn_lds();
    constexpr int U = 8;
    for (uint32_t r0 = threadIdx.x; r0 < L; r0 += U * NT) {
        uint32_t ix[U], key[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const uint32_t r = r0 + (uint32_t)j * NT;
            ix[j] = (uint32_t)idx[r < L ? r : r0];
        }
#pragma unroll
        for (int j = 0; j < U; ++j) key[j] = key_at(rowp, dtype, ix[j]);
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const uint32_t r = r0 + (uint32_t)j * NT;
            if (r < L) em[r] = mass_fx(key[j], m);
        }
    }
    lds_sync();
    const uint32_t per = (L + NT - 1u) / NT;
    const uint32_t r0 = threadIdx.x * per < L ? threadIdx.x * per : L;
    const uint32_t r1 = r0 + per < L ? r0 + per : L;
    uint64_t loc = 0;
    for (uint32_t r = r0; r < r1; ++r) loc += em[r];
    uint64_t total = 0;
    const uint64_t before = block_scan_u64<NT>(loc, total, sh, rb);
    uint64_t T = (uint64_t)ceil(u * (double)total);
    T = T ? T : 1u;
    uint32_t hit = 0xFFFFFFFFu;
    uint64_t run = before;
    for (uint32_t r = r0; r < r1; ++r) {
        run += em[r];
        if (run >= T) {
            hit = r;
            break;
        }
    }
    uint32_t mn[1] = {wave_min_u32(hit)};
    comb_record<NT, 0, 0, 1>(nullptr, nullptr, mn, sh, rb);
    if (prob) {
        const double inv = total ? 1.0 / (double)total : 0.0;
        for (uint32_t r = threadIdx.x; r < lprob; r += NT) prob[r] = (float)((double)em[r] * inv);
    }
    const uint32_t rt = mn[0] < L ? mn[0] : L - 1u;
    const int32_t tok = idx[rt];
    lds_sync();
    return tok;
}

// The draw (and the probabilities) from the kept set's words in rank order
// in LDS (s[0 .. L)): the block prefix of their masses and the first rank
// whose running mass reaches u * S, as in the sort-and-scan path.
template <int NT>
QRITA_DEV int32_t draw_from_sorted(const uint64_t* s, float* prob, uint32_t L, float m, double u, Shared& sh,
                                   int& rb) {
    const uint32_t per = (L + NT - 1u) / NT;
    const uint32_t r0 = threadIdx.x * per < L ? threadIdx.x * per : L;
    const uint32_t r1 = r0 + per < L ? r0 + per : L;
    uint64_t loc = 0;
    for (uint32_t r = r0; r < r1; ++r) loc += mass_fx(cand_key(s[r]), m);
    uint64_t total = 0;
    const uint64_t before = block_scan_u64<NT>(loc, total, sh, rb);
    uint64_t T = (uint64_t)ceil(u * (double)total);
    T = T ? T : 1u;
    const uint32_t rt = first_reaching<NT>(s, r0, r1, before, T, m, L, sh, rb);
    if (prob) {
        const double inv = total ? 1.0 / (double)total : 0.0;
        for (uint32_t r = threadIdx.x; r < L; r += NT) prob[r] = (float)((double)mass_fx(cand_key(s[r]), m) * inv);
    }
    const int32_t tok = (int32_t)cand_idx(s[rt < L ? rt : L - 1u]);
    lds_sync();
    return tok;
}

// Steps a4-a7 on one candidate source holding n candidates, all with keys in
// (key_lo, kmax]; lsrc is the same candidates with their indices. rest_fx is
// the fixed-point mass, relative to rest_ref, of the logits left out of the
// source (top-p-only rows). Returns false when the source does not contain
// the answer (a truncation miss); then nothing has been written.
//
// Duplicates are resolved once, at the end: the top-k search gives the K-th
// value v with n_gt above it and need = K - n_gt of its N duplicates kept;
// the top-p search then runs over the candidates >= v, counting only `need`
// of those at v (their masses are equal, so which ones does not matter for
// the mass); the final boundary value and count then pick the lowest
// indices among its duplicates.
template <class T, class S, class L>
QRITA_DEV bool finish_row(const Params& P, int64_t row, const RowMode& md, const S& src, const L& lsrc, uint32_t n,
                          int64_t key_lo, uint32_t kmax, uint64_t rest_fx, float rest_ref, float t_gauss, Shared& sh,
                          int& rb, TailDiag& dg) {
    constexpr int NT = T::NT;
    const uint32_t V = (uint32_t)P.vocab;
    if (P.diag) {  // #{z >= Gaussian t} among the candidates, for diagnostics
        const uint32_t key_t = f32_key(__float_as_uint(t_gauss));
        uint32_t cc = 0;
        src.visit([&](uint32_t key, uint32_t) { cc += key >= key_t ? 1u : 0u; });
        dg.n_t = (int32_t)comb_sum32<NT>(cc, sh, rb);
    }
    bool topk = md.topk, topp = md.topp;
    uint32_t K = md.K;
    // a4: truncation hit test
    if (md.K_t > 0 && n < md.K_t) return false;
    if ((topp || md.sample_all) && n == 0) return false;
    const float m = key_value(kmax);
    if (topp && m == -__builtin_inff()) {  // all -inf: keep one token
        topp = false;
        topk = true;
        K = 1;
    }
    Ctx<T, S> c{src, wave_segment<T>(), (uint32_t)T::SEG, P.pivot_mode, &sh, rb, 0};
    // kept set: {> vf} and the needf lowest-index of the Nf candidates at vf
    bool all = true;
    uint32_t vf = 0, ngt = 0, needf = 0, Nf = 0;
    // a5: top-k
    if (topk) {
        const CountOut r = search_count<NT, 0>(c, 0u, K, key_lo, n, (int64_t)kmax, 0u);
        all = false;
        vf = r.v;
        ngt = r.n_gt;
        needf = K - r.n_gt;
        Nf = r.N;
    }
    // a6: top-p over the renormalised top-k set
    if (topp) {
        MassSet ms{md.p, 0.0, !topk, 0u, 0u};
        int64_t lo = key_lo;
        if (topk) {
            ms.vx = vf;
            ms.dN = Nf - needf;
            lo = (int64_t)vf - 1;
        } else if (rest_fx) {
            // the dropped logits' mass was taken relative to rest_ref <= m
            ms.rest = (double)rest_fx * (double)mass_f32(f32_key(__float_as_uint(rest_ref)), m);
        }
        MassOut mo;
        uint64_t Tq = 0;
        if (!search_mass<NT>(c, ms, m, lo, (int64_t)kmax, mo, Tq)) {
            rb = c.rb;
            dg.iters += c.iters;
            return false;
        }
        // smallest number of duplicates at v that reaches T: ceil((Tq - M_gt) / e)
        // (M_gt < Tq <= M_gt + N e), clamped to [1, N]
        const uint64_t e = mass_fx(mo.v, m);
        uint32_t need = mo.N;
        if (e > 0) {
            const uint64_t d = Tq - mo.M_gt;
            uint64_t j = d / e + (d % e ? 1u : 0u);
            if (j > mo.N) j = mo.N;
            if (j < 1) j = 1;
            need = (uint32_t)j;
        }
        // at the top-k boundary value all of its duplicates are in the source
        Nf = (topk && mo.v == vf) ? Nf : mo.N;
        all = false;
        vf = mo.v;
        ngt = mo.n_gt;
        needf = need;
    }
    const uint32_t Lk = all ? V : ngt + needf;
    // the draw from the kept set (sampling calls): with S the kept set's mass
    // (plus, for a keep-all row, the mass left out of the candidates) and u the
    // row's uniform, the drawn token has the smallest rank whose cumulative mass
    // reaches u * S: the mass search over the kept set with that target gives
    // its value and its position j among that value's duplicates
    double s_kept = 0.0;
    int32_t token = -1;
    // the kept set sorted in one piece for the index output: the draw reads
    // its words in rank order after the outputs are written (one pass instead
    // of a mass search over the candidates); if the sort ranked them in place,
    // from the index output
    const bool draw_after = P.out_token && m != -__builtin_inff() && !all && !P.idx_order && P.out_idx &&
                            Lk <= (uint32_t)P.idx_cap && ngt + Nf <= (uint32_t)T::CSORT;
    if (P.out_token && !draw_after) {
        if (m == -__builtin_inff()) {
            // no finite logit: rank 0, the lowest index of the maximum
            const CountOut r0 = search_count<NT, 0>(c, 0u, 1u, key_lo, n, (int64_t)kmax, 0u);
            token = (int32_t)cand_idx(tie_boundary<T>(lsrc, r0.v, 1u, r0.N, V, c.mode, sh, c.rb, dg.iters, true));
        } else {
            MassSet ms{row_uniform(P.seed, P.offset, (uint64_t)(P.row0 + row)), 0.0, all, 0u, 0u};
            int64_t lo = key_lo;
            if (all) {
                if (rest_fx) ms.rest = (double)rest_fx * (double)mass_f32(f32_key(__float_as_uint(rest_ref)), m);
            } else {
                ms.vx = vf;
                ms.dN = Nf - needf;
                lo = (int64_t)vf - 1;
            }
            MassOut mo;
            uint64_t Tq = 0;
            if (!search_mass<NT>(c, ms, m, lo, (int64_t)kmax, mo, Tq, &s_kept)) {
                rb = c.rb;
                dg.iters += c.iters;
                return false;  // a keep-all row whose candidates miss the draw
            }
            const uint64_t e = mass_fx(mo.v, m);
            uint32_t j = mo.N;
            if (e > 0) {
                const uint64_t d = Tq - mo.M_gt;
                uint64_t jj = d / e + (d % e ? 1u : 0u);
                jj = jj > mo.N ? mo.N : (jj < 1 ? 1 : jj);
                j = (uint32_t)jj;
            }
            const uint32_t Nv = (!all && mo.v == vf) ? Nf : mo.N;
            token = (int32_t)cand_idx(tie_boundary<T>(lsrc, mo.v, j, Nv, V, c.mode, sh, c.rb, dg.iters, true));
        }
    }
    const void* rowp = P.dtype != 0 ? (const void*)((const uint16_t*)P.logits + row * (int64_t)V)
                                    : (const void*)((const float*)P.logits + row * (int64_t)V);
    float* prow = (P.out_prob && P.idx_cap > 0) ? P.out_prob + row * (int64_t)P.idx_cap : nullptr;
    RowOut o{(P.out_idx && P.idx_cap > 0) ? P.out_idx + row * (int64_t)P.idx_cap : nullptr, (uint32_t)P.idx_cap,
             (P.mask && !md.keep_all) ? P.mask + row * (int64_t)V : nullptr, P.bitmap != 0, V,
             draw_after ? nullptr : prow, m, s_kept > 0.0 ? 1.0 / s_kept : 0.0, rowp, (int)P.dtype};
    bool sorted_kept = false;
    if (P.idx_order)
        emit_row_by_index<T>(c, lsrc, o, all, vf, needf, Nf, Lk, dg);
    else
        sorted_kept = emit_row<T>(c, lsrc, o, all, vf, ngt, needf, Nf, Lk, key_lo, n, kmax, dg, draw_after);
    if (draw_after) {
        const double u = row_uniform(P.seed, P.offset, (uint64_t)(P.row0 + row));
        // (Lk <= CSORT: its masses fit the dynamic LDS for draw_from_ranks)
        token = sorted_kept
                    ? draw_from_sorted<NT>((const uint64_t*)(dyn_lds() + T::SA_OFF), prow, Lk, m, u, sh, c.rb)
                    : draw_from_ranks<NT>(o.idx, prow, Lk, Lk, rowp, (int)P.dtype, m, u, sh, c.rb);
    }
    if (P.out_count && threadIdx.x == 0) P.out_count[row] = (int32_t)Lk;
    if (P.out_token && threadIdx.x == 0) P.out_token[row] = token;
    rb = c.rb;
    dg.iters += c.iters;
    return true;
}

// Steps a4-a7 for a row with few candidates (n <= CSORT / 2, all in the list
// lsrc): every candidate is gathered and sorted once, after which the rank
// order answers top-k (the first K ranks), top-p (the first rank whose
// running fixed-point mass reaches T = p * S) and the draw (the first rank
// reaching u * S) directly. The quantities are those of finish_row's pivot
// searches, rank for rank: the searches exist to avoid ordering a large
// candidate set, and once the set is small enough to sort in one piece the
// order needed for the index output answers them as well. Returns false on a
// truncation miss (nothing written).
template <class T, class L>
QRITA_DEV bool finish_small(const Params& P, int64_t row, const RowMode& md, const L& lsrc, uint32_t n,
                            uint32_t kmax, uint64_t rest_fx, float rest_ref, float t_gauss, Shared& sh, int& rb,
                            TailDiag& dg) {
    constexpr int NT = T::NT;
    const uint32_t V = (uint32_t)P.vocab;
    if (P.diag) {  // #{z >= Gaussian t} among the candidates, for diagnostics
        const uint32_t key_t = f32_key(__float_as_uint(t_gauss));
        uint32_t cc = 0;
        lsrc.visit([&](uint32_t key, uint32_t) { cc += key >= key_t ? 1u : 0u; });
        dg.n_t = (int32_t)comb_sum32<NT>(cc, sh, rb);
    }
    bool topk = md.topk, topp = md.topp;
    uint32_t K = md.K;
    if (md.K_t > 0 && n < md.K_t) return false;
    if ((topp || md.sample_all) && n == 0) return false;
    const float m = key_value(kmax);
    if (topp && m == -__builtin_inff()) {  // all -inf: keep one token
        topp = false;
        topk = true;
        K = 1;
    }
    const bool all = !topk && !topp;
    // every candidate (a: the first half of the sort region), then in rank
    // order (s: its second half, which no sort path reads for sets of at most
    // half the region): s[r] is the word of rank r
    uint64_t* a = (uint64_t*)(dyn_lds() + T::SA_OFF);
    uint64_t* s = a + T::CSORT / 2;
    SortExt ex;
    const uint32_t cnt = gather_words<NT>(lsrc, a, (uint32_t)T::CSORT / 2, 1ull, ~0ull, ex, sh, rb, kmax);
    RankOut so{nullptr, 0u, nullptr, 0u, nullptr, nullptr, 0.0f, 0.0, s};
    sort_words<T>(cnt, ex, so, sh, rb);
    // ranks the masses run over: the top-k set, or every candidate
    const uint32_t R = topk ? (K < cnt ? K : cnt) : cnt;
    const uint32_t per = (R + NT - 1u) / NT;
    const uint32_t r0 = threadIdx.x * per < R ? threadIdx.x * per : R;
    const uint32_t r1 = r0 + per < R ? r0 + per : R;
    const bool masses = topp || P.out_token || P.out_prob;
    uint64_t before = 0, total = 0;
    if (masses && m != -__builtin_inff()) {
        uint64_t loc = 0;
        for (uint32_t r = r0; r < r1; ++r) loc += mass_fx(cand_key(s[r]), m);
        before = block_scan_u64<NT>(loc, total, sh, rb);
    }
    // the logits outside the candidates (top-p-only and keep-all rows), in
    // the same fixed point
    const double rest =
        (!topk && rest_fx) ? (double)rest_fx * (double)mass_f32(f32_key(__float_as_uint(rest_ref)), m) : 0.0;
    uint32_t Lk = topk ? K : V;
    if (topp) {
        uint64_t Tq = (uint64_t)ceil((double)md.p * ((double)total + rest));
        Tq = Tq ? Tq : 1u;
        if (!topk && total < Tq) return false;  // the candidates hold less than p of the mass
        const uint32_t cut = first_reaching<NT>(s, r0, r1, before, Tq, m, R, sh, rb);
        Lk = cut < R ? cut + 1u : R;
    }
    // the kept set's mass: the prefix through rank Lk - 1 (plus the outside
    // mass for keep-all rows)
    double s_kept = 0.0;
    int32_t token = -1;
    if (masses && m != -__builtin_inff()) {
        const uint32_t lastr = (all ? R : (Lk < R ? Lk : R)) - 1u;
        uint64_t mine = 0;
        if (lastr >= r0 && lastr < r1) {
            uint64_t run = before;
            for (uint32_t r = r0; r <= lastr; ++r) run += mass_fx(cand_key(s[r]), m);
            mine = run;
        }
        uint64_t got[1] = {wave_sum_u64(mine)};
        comb_record<NT, 0, 1, 0>(nullptr, got, nullptr, sh, rb);
        s_kept = (double)got[0] + (all ? rest : 0.0);
        if (P.out_token) {
            uint64_t Tu = (uint64_t)ceil(row_uniform(P.seed, P.offset, (uint64_t)(P.row0 + row)) * s_kept);
            Tu = Tu ? Tu : 1u;
            if (all && (double)Tu > (double)got[0]) return false;  // the draw falls outside the candidates
            const uint32_t rt = first_reaching<NT>(s, r0, r1, before, Tu, m, R, sh, rb);
            token = (int32_t)cand_idx(s[rt < R ? rt : R - 1u]);
        }
    } else if (P.out_token) {
        token = (int32_t)cand_idx(s[0]);  // no finite logit: rank 0
    }
    const uint32_t L_ = all ? V : Lk;
    const void* rowp = P.dtype != 0 ? (const void*)((const uint16_t*)P.logits + row * (int64_t)V)
                                    : (const void*)((const float*)P.logits + row * (int64_t)V);
    RowOut o{(P.out_idx && P.idx_cap > 0) ? P.out_idx + row * (int64_t)P.idx_cap : nullptr, (uint32_t)P.idx_cap,
             (P.mask && !md.keep_all) ? P.mask + row * (int64_t)V : nullptr, P.bitmap != 0, V,
             (P.out_prob && P.idx_cap > 0) ? P.out_prob + row * (int64_t)P.idx_cap : nullptr, m,
             s_kept > 0.0 ? 1.0 / s_kept : 0.0, rowp, (int)P.dtype};
    const uint32_t Lout = o.idx ? (L_ < o.idx_cap ? L_ : o.idx_cap) : 0u;
    if (P.idx_order && !all) {
        uint32_t* bm = (uint32_t*)(dyn_lds() + T::SB_OFF);
        const uint32_t nw = (V + 31u) / 32u;
        clear_words(bm, nw + 1u, NT);  // one word past the row: write_mask_row reads it
        lds_sync();
        for (uint32_t r = threadIdx.x; r < Lk; r += NT) {
            const uint32_t i = cand_idx(s[r]);
            atomicOr(&bm[i >> 5], 1u << (i & 31u));
        }
        lds_sync();
        bitmap_outputs<NT>(bm, o, Lout, sh, rb);
    } else if (P.idx_order) {  // keep-all row: 0, 1, ..., Lout - 1
        for (uint32_t r = threadIdx.x; r < Lout; r += NT) {
            o.idx[r] = (int32_t)r;
            if (o.prob) o.prob[r] = prob_at(o, r);
        }
    } else {
        for (uint32_t r = threadIdx.x; r < Lout; r += NT) {
            const uint64_t w = s[r];
            o.idx[r] = (int32_t)cand_idx(w);
            if (o.prob) o.prob[r] = (float)((double)mass_fx(cand_key(w), m) * o.inv_s);
        }
        if (o.mrow && !all) {
            if (o.bitmap) {
                uint32_t* bm = (uint32_t*)(dyn_lds() + T::SB_OFF);
                clear_words(bm, (V + 31u) / 32u + 1u, NT);
                lds_sync();
                for (uint32_t r = threadIdx.x; r < Lk; r += NT) {
                    const uint32_t i = cand_idx(s[r]);
                    atomicOr(&bm[i >> 5], 1u << (i & 31u));
                }
                lds_sync();
                write_mask_row<NT>(o.mrow, bm, V);
            } else {
                for (uint32_t r = threadIdx.x; r < Lk; r += NT) o.mrow[cand_idx(s[r])] = 1;
            }
        }
    }
    if (P.out_count && threadIdx.x == 0) P.out_count[row] = (int32_t)L_;
    if (P.out_token && threadIdx.x == 0) P.out_token[row] = token;
    lds_sync();
    return true;
}

// r-th largest key of the sample (1 <= r <= number of sample entries), by the
// same quaternary search over the sample's keys in LDS.
template <class T>
QRITA_DEV float sample_rank_value(const Params& P, const void* rowp, uint32_t r, Shared& sh, int& rb) {
    constexpr int NT = T::NT;
    const int32_t V = P.vocab;
    float x[8];
    bool in[8];
    if (P.dtype == 1)
        load_sample<1>(rowp, V, x, in);
    else if (P.dtype == 2)
        load_sample<2>(rowp, V, x, in);
    else
        load_sample<0>(rowp, V, x, in);
    uint32_t* a = (uint32_t*)(dyn_lds() + T::A_OFF);
    lds_sync();
#pragma unroll
    for (int i = 0; i < 8; ++i) a[threadIdx.x * 8 + i] = in[i] ? f32_key(__float_as_uint(x[i])) : 0u;
    lds_sync();
    const uint32_t ns = (uint32_t)min(V, kSampleN);
    Ctx<T, SrcLds<NT>> c{SrcLds<NT>{a, 8u * NT}, wave_segment<T>(), (uint32_t)T::SEG, 0, &sh, rb, 0};
    const CountOut o = search_count<NT, 0>(c, 0u, r, (int64_t)0, ns, (int64_t)0xFFFFFFFFu, 0u);
    rb = c.rb;
    lds_sync();
    return key_value(o.v);
}

struct TailOut {
    int32_t done, path, n_t, iters, rb;
};

// The row's list (S sub-lists) as a source; gshift from the slice count.
template <int NT>
QRITA_DEV SrcList<NT> list_source(const Params& P, int64_t row, uint32_t S, uint32_t stride, const uint32_t* cnt,
                                  uint32_t n) {
    const uint32_t s2 = next_pow2(S);
    const uint32_t gshift = 31u - (uint32_t)__builtin_clz((uint32_t)NT / s2);
    return SrcList<NT>{P.glist + row * (int64_t)P.list_stride, stride, S, gshift, cnt, n};
}

// The tail's slow paths: a candidate list too long for LDS (searched in
// memory), and after a truncation miss the re-collection of the row with
// thresholds lowered to sample order statistics and, as the last resort, the
// search of the full row (§1). Inlined: as a separate function its LDS and
// global pointers would arrive as generic ones, and flat memory operations
// serialise the loops.
template <class T>
QRITA_DEV TailOut tail_fallback(const Params& P, int64_t row, RowMode md, float t, float tc, uint32_t nlist,
                                uint32_t kmax, uint64_t rest, bool overflow, bool lds_tried, float lambda,
                                uint32_t ns_h, int32_t n_t, Shared& sh, int rb) {
    constexpr int NT = T::NT;
    const int32_t V = P.vocab;
    const void* rowp = P.dtype != 0 ? (const void*)((const uint16_t*)P.logits + row * (int64_t)V)
                                    : (const void*)((const float*)P.logits + row * (int64_t)V);
    const float kInf = __builtin_inff();
    TailDiag dg{n_t, 0};
    int path = 1;
    bool done = false;
    if (!lds_tried && !overflow) {
        const SrcList<NT> src = list_source<NT>(P, row, (uint32_t)P.slices, (uint32_t)P.sub_cap, sh.cnt, nlist);
        done = finish_row<T>(P, row, md, src, src, nlist, (int64_t)f32_key(__float_as_uint(tc)) - 1, kmax, rest, tc,
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
                tr = sample_rank_value<T>(P, rowp, (uint32_t)rr, sh, rb);
            else if (prev > -kInf)
                tr = -kInf;
            else
                break;
            if (!(tr < prev)) continue;
            prev = tr;
            uint64_t rest2 = 0;
            uint32_t kmax2 = 0;
            bool ovf = false;
            uint32_t cnt;
            // the whole dynamic LDS stages the survivors (nothing in it is live here)
            uint64_t* stage = (uint64_t*)dyn_lds();
            const uint32_t scap = (uint32_t)(T::LDS / 8);
            if (P.dtype == 1)
                cnt = collect_row<NT, 1>(P, row, tr, md.rest_on(), stage, scap, sh, rb, rest2, kmax2, ovf);
            else if (P.dtype == 2)
                cnt = collect_row<NT, 2>(P, row, tr, md.rest_on(), stage, scap, sh, rb, rest2, kmax2, ovf);
            else
                cnt = collect_row<NT, 0>(P, row, tr, md.rest_on(), stage, scap, sh, rb, rest2, kmax2, ovf);
            if (ovf) break;
            if (threadIdx.x == 0) sh.cnt[0] = cnt;
            lds_sync();
            const SrcList<NT> src = list_source<NT>(P, row, 1u, (uint32_t)P.list_stride, sh.cnt, cnt);
            done = finish_row<T>(P, row, md, src, src, cnt, (int64_t)f32_key(__float_as_uint(tr)) - 1, kmax2, rest2,
                                 tr, t, sh, rb, dg);
            if (tr == -kInf) break;
        }
    }
    if (!done) {
        path = 3;
        uint32_t kr = 0;
        const SrcRow<NT> src{rowp, (uint32_t)V, (int)P.dtype, (uint32_t)V};
        src.visit([&](uint32_t key, uint32_t) { kr = key > kr ? key : kr; });
        uint32_t mn[1] = {~wave_max_u32(kr)};
        comb_record<NT, 0, 0, 1>(nullptr, nullptr, mn, sh, rb);
        kr = ~mn[0];
        done = finish_row<T>(P, row, md, src, src, (uint32_t)V, -1, kr, 0ull, 0.0f, t, sh, rb, dg);
    }
    return TailOut{done ? 1 : 0, path, dg.n_t, dg.iters, rb};
}

// Tail: one workgroup per row. When the rows take about two rounds of the
// workgroups resident at once, a workgroup takes its row from a counter
// (zeroed by pass 1) when it starts, rather than row = workgroup index. Rows
// are then handed out in the order the workgroups start, wherever they run,
// instead of by the fixed placement of workgroup indices on XCDs and CUs,
// which can put the expensive rows of a periodic pattern (a per-row k that
// cycles) on the same XCDs; the rows of the second round then also go to
// whichever workgroups start first. The grid has one workgroup per row, so
// each takes one ticket below the row count. The row's sub-lists are loaded
// into LDS when they fit and did not overflow; everything else takes
// tail_fallback.
template <class T>
__global__ __launch_bounds__(T::NT, T::WAVES_PER_SIMD) void tail_kernel(Params P) {
    constexpr int NT = T::NT;
    __shared__ Shared sh;
    int rb = 0;
    int64_t row = blockIdx.x;
    if (P.queue) {
        if (threadIdx.x == 0) sh.row = atomicAdd(P.queue, 1u);
        __syncthreads();
        row = uni(sh.row);
    }
    if (row >= P.batch) return;
    if (P.fused) {
        // one launch: this workgroup first streams the whole row as pass 1's
        // only slice, leaving the row and slice records and the list that
        // the rest reads back
        if (P.dtype == 1)
            pass1_slice<NT, 1>(P, row, 0u, sh, rb);
        else if (P.dtype == 2)
            pass1_slice<NT, 2>(P, row, 0u, sh, rb);
        else
            pass1_slice<NT, 0>(P, row, 0u, sh, rb);
        __threadfence_block();
        __syncthreads();
    }
    const int32_t V = P.vocab;
    const uint32_t S = (uint32_t)P.slices;
    const RowMode md = row_mode(P, row);
    const uint32_t* rr = P.rowrec + row * R_WORDS;
    const uint4 r4 = *(const uint4*)rr;
    const float t = __uint_as_float(uni(r4.x));
    const float tc = __uint_as_float(uni(r4.y));
    const bool predicted = uni(r4.z) != 0;
    const float lambda = __uint_as_float(uni(r4.w));
    const uint32_t ns_h = uni(rr[R_NS]);
    // the slice records: every wave combines them (lane s reads slice s)
    const uint32_t lane = threadIdx.x & (kWave - 1);
    uint4 q = make_uint4(0u, 0u, 0u, 0u);
    if (lane < S) q = *(const uint4*)(P.slrec + (row * kMaxSlices + lane) * S_WORDS);
    const uint32_t cnt_s = q.x;
    const uint32_t nlist = uni(wave_sum_u32(cnt_s));
    const uint32_t kmax = uni(wave_max_u32(q.y));
    const uint64_t rest = uni(wave_sum_u64((uint64_t)q.z | ((uint64_t)q.w << 32)));
    const bool overflow = uni(wave_max_u32(cnt_s)) > (uint32_t)P.sub_cap;
    if (threadIdx.x < S) sh.cnt[threadIdx.x] = cnt_s;
    if (threadIdx.x < kWave) {
        // exclusive prefix of the counts over the slices (lanes)
        uint32_t x = cnt_s;
        QRITA_WAVE_STEPS(op_add, 0u)
        if (lane < S) sh.pre[lane] = x - cnt_s;
    }
    lds_sync();

    TailDiag dg{-1, 0};
    int path = 0;
    bool done = false;
    uint8_t* mrow = P.mask ? P.mask + row * (int64_t)V : nullptr;
    if (!md.need_cand) {
        if (P.out_count && threadIdx.x == 0) P.out_count[row] = V;
        if (P.idx_order && P.out_idx) {  // keep-all row in index order
            const uint32_t lo = (uint32_t)P.idx_cap < (uint32_t)V ? (uint32_t)P.idx_cap : (uint32_t)V;
            int32_t* orow = P.out_idx + row * (int64_t)P.idx_cap;
            for (uint32_t r = threadIdx.x; r < lo; r += NT) orow[r] = (int32_t)r;
        }
        done = true;
    } else {
        const bool small = !overflow && nlist <= (uint32_t)P.small_max;
        const bool in_lds = !small && !overflow && nlist <= (uint32_t)P.tail_cap;
        if (small) {
            const SrcList<NT> lsrc = list_source<NT>(P, row, S, (uint32_t)P.sub_cap, sh.cnt, nlist);
            done = finish_small<T>(P, row, md, lsrc, nlist, kmax, rest, tc, t, sh, rb, dg);
        } else if (in_lds) {
            // every candidate has z >= tc, so its key exceeds key(tc) - 1
            const int64_t key_lo = (int64_t)f32_key(__float_as_uint(tc)) - 1;
            uint32_t* a = (uint32_t*)(dyn_lds() + T::A_OFF);
            // sub-list s is copied by a group of NT / next_pow2(S) threads to
            // a[pre[s] ..]; 32 loads per thread in flight
            {
                const uint32_t s2 = next_pow2(S);
                const uint32_t gshift = 31u - (uint32_t)__builtin_clz((uint32_t)NT / s2);
                const uint32_t tps = 1u << gshift;
                const uint32_t s = threadIdx.x >> gshift, g = threadIdx.x & (tps - 1u);
                const uint32_t cs = s < S ? sh.cnt[s] : 0u, ps = s < S ? sh.pre[s] : 0u;
                const uint64_t* p = P.glist + row * (int64_t)P.list_stride + (int64_t)s * P.sub_cap;
                constexpr int U = 32;
                // only the keys (the high words of the entries) are needed here
                const uint32_t* pk = (const uint32_t*)p + 1;
                for (uint32_t j0 = g; j0 < cs; j0 += tps * U) {
                    uint32_t kv[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        // clamped index: unconditional loads, all in flight together
                        const uint32_t j = j0 + (uint32_t)u * tps;
                        kv[u] = pk[2 * (size_t)(j < cs ? j : cs - 1u)];
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const uint32_t j = j0 + (uint32_t)u * tps;
                        if (j < cs) a[ps + j] = kv[u];
                    }
                }
                if (threadIdx.x < 4u && nlist + threadIdx.x < ((nlist + 3u) & ~3u)) a[nlist + threadIdx.x] = 0u;
            }
            lds_sync();
            const SrcLds<NT> src{a, nlist};
            const SrcList<NT> lsrc = list_source<NT>(P, row, S, (uint32_t)P.sub_cap, sh.cnt, nlist);
            done = finish_row<T>(P, row, md, src, lsrc, nlist, key_lo, kmax, rest, tc, t, sh, rb, dg);
        }
        if (!done) {
            const TailOut o = tail_fallback<T>(P, row, md, t, tc, nlist, kmax, rest, overflow, in_lds || small,
                                               lambda, ns_h, dg.n_t, sh, rb);
            done = o.done != 0;
            path = o.path;
            dg.n_t = o.n_t;
            dg.iters += o.iters;
            rb = o.rb;
        }
    }
    // keep-all rows: the whole mask row is ones (pass 1 wrote it unless the
    // tail writes masks)
    if (md.keep_all && mrow && P.bitmap) fill_mask_row<NT>(mrow, (uint32_t)V, 1);
    if (threadIdx.x == 0 && P.diag) {
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

}  // namespace qrita
