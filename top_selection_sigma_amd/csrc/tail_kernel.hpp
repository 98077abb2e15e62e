// The tail of the path (steps a4-a7): one workgroup of four waves per row,
// launched after pass 1 has completed for every row.
//
// No thread of a tail workgroup reads global memory that another one wrote
// (outside the re-collection of the fallback, which synchronises fully), so
// its barriers order LDS only and never wait for the mask and index stores.
//
// The row's candidate list is held in registers (RegSet: up to 64 keys per
// thread, 16384 per row) and every pivot evaluation of the quaternary search
// is one pass over those registers followed by one combination across the
// four waves. Longer lists, overflowed lists and truncation misses take the
// out-of-line fallback, which streams the candidates from memory (MemSrc).
#pragma once

namespace qrita {

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

// Exclusive prefix over the waves of per-wave counts c (wave uniform):
// returns the sum over the lower waves and sets total to the sum over all.
template <int NT>
QRITA_DEV uint32_t wave_prefix(uint32_t c, uint32_t& total, Shared& sh, int& rb) {
    constexpr int NW = NT / kWave;
    if (NW == 1) {
        total = c;
        return 0u;
    }
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
    uint32_t total = 0;
    wave_prefix<NT>(wave_sum_u32(v), total, sh, rb);
    return total;
}

template <int NT>
QRITA_DEV uint32_t comb_max32(uint32_t v, Shared& sh, int& rb) {
    uint32_t mn[1] = {~wave_max_u32(v)};
    comb_record<NT, 0, 0, 1>(nullptr, nullptr, mn, sh, rb);
    return ~mn[0];
}

// Records of N32 u32 sums, N64 u64 sums and NMIN u32 minima (wave totals on
// entry, block totals on return). A record takes at most 32 words and a
// workgroup at most 8 waves: the records of one buffer fill slot[rb].
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

// Calls f(std::integral_constant<int, C>) for C = B .. E-1 (compile-time
// register indices).
template <int B, int E, class F>
QRITA_DEV void unroll_rows(F& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        unroll_rows<B + 1, E>(f);
    }
}

// ---------------------------------------------------------------------------
// Candidate sources. A source hands every candidate to a visitor as
// (key, low, e, r): key 0 marks an empty slot or a candidate outside the
// current set (every real key is nonzero); low is the complemented vocabulary
// index (passed only to visits that ask for it); e is the candidate's cached
// softmax mass (register sets, visits that ask for it); r is the register row.
//
// RegSet keeps up to NT * R candidate keys in registers, slot (r, thread t)
// holding candidate r * NT + t; the complemented indices and the softmax
// masses wait in LDS under the same slot numbering. Each wave skips the
// register rows past its last candidate, four rows per uniform branch.
// ---------------------------------------------------------------------------
template <int NT, int R>
struct RegSet {
    static constexpr int kChunk = 4;
    static_assert(R % kChunk == 0, "register rows come in chunks");
    uint32_t key[R];
    uint32_t* lows;   // LDS, [R * NT]
    float* em;        // LDS, [R * NT]: exp(z - m) once a mass search has started
    uint32_t nslots;  // slots r * NT + t < nslots may hold candidates

    // number of register rows holding candidates of this thread's wave
    QRITA_DEV int rows_here() const {
        const uint32_t wb = wave_base_here();
        const uint32_t ns = __builtin_amdgcn_readfirstlane(nslots);
        return wb < ns ? (int)((ns - wb + NT - 1) / NT) : 0;
    }
    template <int C, class F>
    QRITA_DEV void chunks_from(F& f, int nr) const {
        if constexpr (C < R) {
            if (C < nr) {
                unroll_rows<C, C + kChunk>(f);
                chunks_from<C + kChunk>(f, nr);
            }
        }
    }
    // f(row) for the rows of every chunk holding this wave's candidates; rows
    // past the last candidate inside the last chunk hold key 0
    template <class F>
    QRITA_DEV void for_rows(F&& f) const {
        chunks_from<0>(f, rows_here());
    }

    // f(key, low, e, r); the indices (LOWS) and masses (EM) of the visited
    // rows are read from LDS in one batch first
    template <bool LOWS, bool EM, class F>
    QRITA_DEV void visit(F&& f) const {
        const uint32_t t = tid_here();
        uint32_t lw[R];
        float ev[R];
        if constexpr (LOWS || EM) {
            for_rows([&](auto rc) {
                constexpr int r = decltype(rc)::value;
                if (LOWS) lw[r] = lows[t + r * NT];
                if (EM) ev[r] = em[t + r * NT];
            });
        }
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            f(key[r], LOWS ? lw[r] : 0u, EM ? ev[r] : 0.0f, r);
        });
    }
    QRITA_DEV void put_mass(int r, float e) const { em[tid_here() + r * NT] = e; }

    // The n candidates of a row list in list order; the first PR rows were
    // read already (pre). Every load is issued before the first index is
    // stored.
    template <int PR>
    QRITA_DEV void load(const uint64_t* lst, uint32_t n, const uint64_t (&pre)[PR]) {
        nslots = n;
        const uint32_t t = tid_here();
        uint32_t lw[R];
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const uint32_t i = (uint32_t)r * NT + t;
            uint64_t c;
            if constexpr (r < PR)
                c = pre[r];
            else
                c = lst[i < n ? i : n - 1];
            key[r] = i < n ? cand_key(c) : 0u;
            lw[r] = cand_low(c);
        });
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            lows[t + r * NT] = lw[r];
        });
        block_sync<NT>();
    }
    // drop the candidates with key below v
    QRITA_DEV void restrict_ge(uint32_t v) {
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            key[r] = key[r] >= v ? key[r] : 0u;
        });
    }
    // drop the candidates c < B
    QRITA_DEV void restrict_to(uint64_t B) {
        const uint32_t bk = cand_key(B), bl = cand_low(B);
        visit<true, false>([&](uint32_t, uint32_t lw, float, int r) {
            const uint32_t k = key[r];
            key[r] = (k > bk || (k == bk && lw >= bl)) ? k : 0u;
        });
    }
    // Move the candidates still in the set (key != 0) to the first slots, in
    // slot order, through the mass buffer (which holds no masses yet); later
    // visits skip the emptied rows.
    QRITA_DEV void compact(Shared& sh, int& rb) {
        uint32_t c = 0;
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            c += (uint32_t)__popcll(__ballot(key[r] != 0u));
        });
        uint32_t total = 0;
        uint32_t run = wave_prefix<NT>(c, total, sh, rb);
        const uint32_t t = tid_here();
        uint32_t lw[R];
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            lw[r] = lows[t + r * NT];
        });
        block_sync<NT>();  // every index is read before any slot is rewritten
        uint32_t* kb = (uint32_t*)em;
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const uint32_t k = key[r];
            const uint64_t b = __ballot(k != 0u);
            if (k != 0u) {
                const uint32_t pos = run + lanes_below(b);
                kb[pos] = k;
                lows[pos] = lw[r];
            }
            run += (uint32_t)__popcll(b);
        });
        block_sync<NT>();
        nslots = total;
        for_rows([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const uint32_t i = (uint32_t)r * NT + t;
            const uint32_t k = kb[i];  // inside the buffer for every visited row
            key[r] = i < total ? k : 0u;
        });
        block_sync<NT>();  // the staged keys are read before the buffer is reused
    }
    // chunks of rows that a set of n candidates occupies in the busiest wave
    QRITA_DEV static uint32_t chunks_for(uint32_t n) {
        return (n + (uint32_t)(NT * kChunk) - 1) / (uint32_t)(NT * kChunk);
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

    QRITA_DEV uint64_t get(uint32_t i) const {
        if (ROW) return make_cand(f32_key(__float_as_uint(load_value<BF16>(row, i))), i);
        return p[i];
    }
    template <bool LOWS, bool EM, class F>
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
                f(ok ? cand_key(c[u]) : 0u, cand_low(c[u]), 0.0f, 0);
            }
        }
    }
    QRITA_DEV void put_mass(int, float) const {}
    QRITA_DEV void restrict_ge(uint32_t v) {
        const uint64_t b = (uint64_t)v << 32;
        filter = b > filter ? b : filter;
    }
    QRITA_DEV void restrict_to(uint64_t B) { filter = B > filter ? B : filter; }
    QRITA_DEV void compact(Shared&, int&) {}
    QRITA_DEV static uint32_t chunks_for(uint32_t) { return 0u; }
    static constexpr bool kRegs = false;
};

// Three pivots at 25/50/75 % of the open range (lo, hi) of field values
// (hi - lo >= 2): of the key range (mode 0), or of the value range (mode 1,
// keys only, finite ends). Pivots lie strictly inside and do not descend.
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

// Field 0 searches keys; field 1 searches the complemented indices of the
// candidates whose key is v_eq (duplicate resolution).
template <int FIELD>
QRITA_DEV uint32_t field_of(uint32_t key, uint32_t low, uint32_t v_eq) {
    if (FIELD == 0) return key;
    return key == v_eq ? low : 0u;
}

// One pivot evaluation of the quaternary search, in one pass over the source
// and one block combination. With t_0 the current lower end and t_1 < t_2 <
// t_3 the three pivots, it returns G_i = #{f > t_i} (and for the mass search
// M_i, the fixed-point mass above t_i), and for each pivot the smallest value
// above it (the z_mn of §2) and the largest value at or below it. The minima
// come from wrap-around differences: f - (p + 1) is small exactly for values
// above p, p - f exactly for values at or below it, so no lane masks are
// needed.
//
// MM = 0 counts only; MM = 1 computes each candidate's mass exp(z - m) and
// caches it; MM = 2 reads the cached masses.
struct Eval4 {
    uint32_t G[4];
    uint64_t M[4];
    uint32_t mn[3];  // smallest value above pivot i
    uint32_t mx[3];  // largest value at or below pivot i (0: none)
};

template <int NT, int FIELD, int MM, class S>
QRITA_DEV Eval4 eval4(const S& src, uint32_t v_eq, uint32_t t0, const uint32_t piv[3], float m, Shared& sh,
                      int& rb) {
    constexpr bool MASS = MM != 0;
    constexpr bool CACHED = MM == 2 && S::kRegs;
    uint32_t g0 = 0, g1 = 0, g2 = 0, g3 = 0;
    uint32_t a0 = 0xFFFFFFFFu, a1 = 0xFFFFFFFFu, a2 = 0xFFFFFFFFu;
    uint32_t c0 = 0xFFFFFFFFu, c1 = 0xFFFFFFFFu, c2 = 0xFFFFFFFFu;
    // register sets: 32-bit halves of the fixed-point masses; streamed
    // sources: 64-bit sums (any number of candidates per lane)
    uint32_t h0 = 0, h1 = 0, h2 = 0, h3 = 0, l0 = 0, l1 = 0, l2 = 0, l3 = 0;
    uint64_t q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    const uint32_t p0 = piv[0], p1 = piv[1], p2 = piv[2];
    const uint32_t s0 = p0 + 1u, s1 = p1 + 1u, s2 = p2 + 1u;
    src.template visit<FIELD == 1, CACHED>([&](uint32_t key, uint32_t low, float ec, int r) {
        const uint32_t f = field_of<FIELD>(key, low, v_eq);
        const uint32_t b0 = gt01(f, t0), b1 = gt01(f, p0), b2 = gt01(f, p1), b3 = gt01(f, p2);
        g0 += b0;
        g1 += b1;
        g2 += b2;
        g3 += b3;
        const uint32_t u0 = f - s0, u1 = f - s1, u2 = f - s2;
        a0 = u0 < a0 ? u0 : a0;
        a1 = u1 < a1 ? u1 : a1;
        a2 = u2 < a2 ? u2 : a2;
        const uint32_t w0 = p0 - f, w1 = p1 - f, w2 = p2 - f;
        c0 = w0 < c0 ? w0 : c0;
        c1 = w1 < c1 ? w1 : c1;
        c2 = w2 < c2 ? w2 : c2;
        if constexpr (MASS) {
            float e = ec;
            if constexpr (!CACHED) {
                // computed where the visit runs: hoisted out of the row-chunk
                // branches it would be paid for every register row
                uint32_t kk = key;
                asm volatile("" : "+v"(kk));
                e = kk ? mass_f32(kk, m) : 0.0f;
            }
            if constexpr (MM == 1) src.put_mass(r, e);
            if constexpr (S::kRegs) {
                uint32_t eh, el;
                fx_split(e, eh, el);
                h0 += __umul24(b0, eh);
                l0 += __umul24(b0, el);
                h1 += __umul24(b1, eh);
                l1 += __umul24(b1, el);
                h2 += __umul24(b2, eh);
                l2 += __umul24(b2, el);
                h3 += __umul24(b3, eh);
                l3 += __umul24(b3, el);
            } else {
                const uint64_t x = fx_from_unit_f32(e);
                q0 += b0 ? x : 0ull;
                q1 += b1 ? x : 0ull;
                q2 += b2 ? x : 0ull;
                q3 += b3 ? x : 0ull;
            }
        }
    });
    uint32_t s32[4] = {wave_sum_u32(g0), wave_sum_u32(g1), wave_sum_u32(g2), wave_sum_u32(g3)};
    uint32_t mn[6] = {wave_min_u32(a0), wave_min_u32(a1), wave_min_u32(a2),
                      wave_min_u32(c0), wave_min_u32(c1), wave_min_u32(c2)};
    Eval4 E;
    if constexpr (MASS) {
        uint64_t s64[4];
        if constexpr (S::kRegs) {
            s64[0] = wave_sum_split(h0, l0);
            s64[1] = wave_sum_split(h1, l1);
            s64[2] = wave_sum_split(h2, l2);
            s64[3] = wave_sum_split(h3, l3);
        } else {
            s64[0] = wave_sum_u64(q0);
            s64[1] = wave_sum_u64(q1);
            s64[2] = wave_sum_u64(q2);
            s64[3] = wave_sum_u64(q3);
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
    return E;
}

template <class T>
QRITA_DEV T pick4(int j, T a, T b, T c, T d) {
    return j == 3 ? d : (j == 2 ? c : (j == 1 ? b : a));
}

struct CountOut {
    uint32_t v, n_gt, N;
};

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
// #{> z_mn} < K <= #{>= z_mn}).
template <int NT, int FIELD, class S>
QRITA_DEV CountOut qsearch_count(const S& src, uint32_t v_eq, uint32_t K, int64_t lo_in, uint32_t G_lo,
                                 int64_t hi_in, uint32_t G_hi, int mode, Shared& sh, int& rb, int& iters) {
    // every field value is nonzero, so a lower end below 0 is the same as 0
    uint32_t lo = lo_in > 0 ? (uint32_t)lo_in : 0u;
    uint32_t hi = (uint32_t)hi_in;
    bool conf = true;   // G(lo) = G_lo is known (then G_lo >= K)
    uint32_t G_up = 0;  // lo not confirmed: G at the pivot below lo
#pragma unroll 1
    for (int guard = 0; guard < 80; ++guard) {
        if (conf && hi - lo <= 1) return CountOut{hi, G_hi, G_lo - G_hi};
        uint32_t piv[3] = {hi, hi, hi};
        if (hi - lo >= 2) make_pivots(lo, hi, mode, FIELD, piv);
        const Eval4 E = eval4<NT, FIELD, 0>(src, v_eq, lo, piv, 0.0f, sh, rb);
        ++iters;
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
    float p;        // target fraction
    double rest;    // mass outside the source (top-p-only rows), relative to m
    bool need_all;  // the source must hold mass p itself (else a miss)
    uint32_t vx, dN;
};

// The quaternary search over softmax mass (top-p): finds the key v with
// M(> v) < T <= M(>= v), T = p * (M(set) + rest). The masses are integers, so
// M >= T is tested as M >= Tq = ceil(T). The first evaluation also computes
// and caches every candidate's mass and the set's total. Returns false on a
// miss (need_all and the source holds less than T).
template <int NT, class S>
QRITA_DEV bool qsearch_mass(const S& src, const MassSet& ms, float m, int64_t lo_in, int64_t hi_in, int mode,
                            Shared& sh, int& rb, int& iters, MassOut& out, uint64_t& Tq) {
    uint32_t lo = lo_in > 0 ? (uint32_t)lo_in : 0u;
    uint32_t hi = (uint32_t)hi_in;
    const uint64_t ex = ms.dN ? (uint64_t)ms.dN * mass_fx(ms.vx, m) : 0ull;
    uint64_t M_hi = 0;
    uint32_t G_hi = 0, G_lo = 0, G_up = 0;
    bool conf = true;
#pragma unroll 1
    for (int guard = 0; guard < 80; ++guard) {
        if (guard > 0 && conf && hi - lo <= 1) {
            out = MassOut{hi, G_hi, G_lo - G_hi, M_hi};
            return true;
        }
        uint32_t piv[3] = {hi, hi, hi};
        if (hi - lo >= 2) make_pivots(lo, hi, mode, 0, piv);
        Eval4 E;
        if (guard == 0)
            E = eval4<NT, 0, 1>(src, 0u, lo, piv, m, sh, rb);
        else
            E = eval4<NT, 0, 2>(src, 0u, lo, piv, m, sh, rb);
        ++iters;
        if (lo < ms.vx) {
            E.G[0] -= ms.dN;
            E.M[0] -= ex;
        }
        if (guard == 0) {
            Tq = (uint64_t)ceil((double)ms.p * ((double)E.M[0] + ms.rest));
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
    }
    out = MassOut{hi, G_hi, G_lo - G_hi, M_hi};  // not reached for consistent inputs
    return true;
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
                src.template visit<false, false>(
                    [&](uint32_t key, uint32_t, float, int) { c += (uint32_t)__popcll(__ballot(key == v)); });
                uint32_t total = 0;
                uint32_t run = wave_prefix<NT>(c, total, sh, rb);
                src.template visit<true, false>([&](uint32_t key, uint32_t low, float, int) {
                    const bool tie = key == v;
                    const uint64_t bb = __ballot(tie);
                    const uint32_t pos = run + lanes_below(bb);
                    if (tie && pos < (uint32_t)kTieDirect) sh.ties[pos] = low;
                    run += (uint32_t)__popcll(bb);
                });
            } else {
                block_sync<NT>();
                src.template visit<true, false>([&](uint32_t key, uint32_t low, float, int) {
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
            b |= uni(sh.u32[6]);
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

// ---------------------------------------------------------------------------
// Rank order of the kept set (a7). The candidates to order sit in LDS as
// (key << 32 | ~index), so descending words are descending values with ties
// by ascending index, a total order.
// ---------------------------------------------------------------------------
QRITA_DEV uint32_t next_pow2(uint32_t x) {
    uint32_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

// Where a sort puts the candidate of rank r: index r of the index output
// (r < lout) and, for r < lmask, its mask byte.
struct RankOut {
    int32_t* out;
    uint32_t lout;
    uint8_t* mrow;
    uint32_t lmask;
    QRITA_DEV void put(uint32_t r, uint32_t idx) const {
        if (r < lout) out[r] = (int32_t)idx;
        if (r < lmask) mrow[idx] = 1;
    }
};

// Up to NT entries: each entry's rank is the number of larger entries,
// counted by NT / next_pow2(cnt) threads per entry over a share of the
// entries each, the shares added in LDS. The entries are read eight at a time
// (zero padding after the last one is below every entry).
template <int NT>
QRITA_DEV void rank_sort(uint64_t* a, uint32_t cnt, const RankOut& ro, Shared& sh) {
    const uint32_t P = (uint32_t)NT / next_pow2(cnt);
    const uint32_t t = threadIdx.x, e = t / P, q = t % P;
    const uint32_t span = (((cnt + P - 1) / P) + 7u) & ~7u;
    if (t < 8u) a[cnt + t] = 0ull;
    if (q == 0 && e < cnt) sh.ties[e] = 0u;
    lds_sync();
    uint64_t x = 0;
    if (e < cnt) {
        x = a[e];
        const uint32_t j0 = q * span, j1 = min(j0 + span, (cnt + 7u) & ~7u);
        uint32_t above = 0;
#pragma unroll 4
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
        if (above) atomicAdd(&sh.ties[e], above);
    }
    lds_sync();
    if (q == 0 && e < cnt) ro.put(sh.ties[e], cand_idx(x));
}

// Bitonic sort, descending, of the NT * E entries a[0 .. NT*E) (any order),
// then out[g] = index of rank g for g < cnt. Thread t holds the logical
// elements g = t * E + e in registers. By partner distance j a stage runs in
// the thread's registers (j < E), across lanes of the wave with shuffles
// (E <= j < 64 E) or across waves through LDS (j >= 64 E; element (t, e) at
// a[e * NT + t], so the accesses of a wave are consecutive).
template <int NT, int E>
QRITA_DEV void bitonic_sort(uint64_t* a, const RankOut& ro, uint32_t cnt) {
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
        if (g < cnt) ro.put(g, cand_idx(x[e]));
    }
}

// Exclusive prefix sum, in place, of the n <= kSortBins counts v[0 .. n)
// (thread t owns entries [t * per, (t + 1) * per)); v[n] becomes the total.
// Returns the largest count (uniform). One block round.
constexpr uint32_t kSortBins = 4096;

template <int NT>
QRITA_DEV uint32_t scan_counts(uint32_t* v, uint32_t n, Shared& sh, int& rb) {
    constexpr int PER = (int)(kSortBins / NT);
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
        uint32_t m = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint2 q = *(const uint2*)(rec + w * 2);
            run += (uint32_t)w < wave ? q.x : 0u;
            total += q.x;
            m = q.y > m ? q.y : m;
        }
        rb ^= 1;
        big = uni(m);
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

// Bucket sort, descending, of the cnt <= E * NT distinct words a[0 .. cnt)
// into out[rank] = index. Thread t holds words e * NT + t in registers.
//
// Bins ascend as words descend. Keys are coded exactly as (kmax - key) >> z,
// z the number of low bits all keys share (16 for bf16 logits), coarsened by
// dropping low code bits if the codes outnumber the bins. Within a code,
// words spread by a sub-coordinate: the dropped code bits, then the index
// (lmax - low), so tie groups spread too. First every code gets the same
// number of bins; if a bin then holds more than kMaxBin words, each code
// instead gets a run of bins in proportion to how many words it holds (from
// a histogram over the codes). A word's rank is its bin's start plus the
// number of larger words in its bin, counted directly, so the result does
// not depend on the order of the LDS atomics that fill the bins. Returns
// false, having written nothing, when a bin still holds more than kMaxBin
// words.
constexpr uint32_t kMaxBin = 96;

QRITA_DEV uint32_t bits_for(uint64_t x) { return x ? 64u - (uint32_t)__builtin_clzll(x) : 0u; }

template <int NT, int E>
QRITA_DEV bool bucket_sort(uint64_t* a, uint32_t cnt, const RankOut& ro, uint64_t* b, uint32_t* bins, Shared& sh,
                           int& rb) {
    const uint32_t t = threadIdx.x;
    uint64_t x[E];
    const uint32_t key0 = uni(cand_key(a[0]));
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u, lmn = 0xFFFFFFFFu, lmx = 0u, tz = 32u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t i = (uint32_t)e * NT + t;
        x[e] = i < cnt ? a[i] : 0ull;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t i = (uint32_t)e * NT + t;
        if (i < cnt) {
            const uint32_t k = cand_key(x[e]), l = cand_low(x[e]);
            kmn = k < kmn ? k : kmn;
            kmx = k > kmx ? k : kmx;
            lmn = l < lmn ? l : lmn;
            lmx = l > lmx ? l : lmx;
            const uint32_t d = k ^ key0;
            const uint32_t z = d ? (uint32_t)__builtin_ctz(d) : 32u;
            tz = z < tz ? z : tz;
        }
    }
    uint32_t ext[5] = {wave_min_u32(kmn), ~wave_max_u32(kmx), wave_min_u32(lmn), ~wave_max_u32(lmx),
                       wave_min_u32(tz)};
    // the bin counts are cleared before the combination's barrier, which
    // orders them before the first count
    const uint32_t nb = min(kSortBins, 2u * next_pow2(cnt));
    for (uint32_t i = t; i <= nb; i += NT) bins[i] = 0u;
    comb_record<NT, 0, 0, 5>(nullptr, nullptr, ext, sh, rb);
    kmn = uni(ext[0]);
    kmx = ~uni(ext[1]);
    lmn = uni(ext[2]);
    lmx = ~uni(ext[3]);
    const uint32_t kz = min(uni(ext[4]), 31u);
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
    // a word's code and sub-coordinate, recomputed where needed (fewer
    // registers held across the phases)
    auto code_of = [&](uint64_t w) { return ((kmx - cand_key(w)) >> kz) >> kdrop; };
    auto sub_of = [&](uint64_t w) {
        const uint32_t fine = (kmx - cand_key(w)) >> kz;
        const uint64_t dropped = kdrop ? (uint64_t)(fine & ((1u << kdrop) - 1u)) : 0ull;
        return ((dropped << lbits) | (uint64_t)(lmx - cand_low(w))) >> scut;
    };
    // every code the same run of bins: code bits, then the top sub bits
    const uint32_t lkeep = nbits - (cbits - kdrop);
    const uint32_t sshift = sbits > lkeep ? sbits - lkeep : 0u;
    uint32_t bin[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t sc = lkeep ? (uint32_t)(sub_of(x[e]) >> sshift) : 0u;
        bin[e] = (uint32_t)e * NT + t < cnt ? ((code_of(x[e]) << lkeep) | sc) : 0u;
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        if ((uint32_t)e * NT + t < cnt) atomicAdd(&bins[bin[e]], 1u);
    lds_sync();
    uint32_t big = scan_counts<NT>(bins, nb, sh, rb);
    if (big > kMaxBin) {
        // runs of bins in proportion to the codes' sizes; the code histogram
        // sits in the second buffer (free until the scatter)
        uint32_t* hc = (uint32_t*)b;
        for (uint32_t i = t; i <= ncodes; i += NT) hc[i] = 0u;
        lds_sync();
#pragma unroll
        for (int e = 0; e < E; ++e)
            if ((uint32_t)e * NT + t < cnt) atomicAdd(&hc[code_of(x[e])], 1u);
        lds_sync();
        scan_counts<NT>(hc, ncodes, sh, rb);
        const float ratio = (float)nb / (float)cnt;
        auto first = [&](uint32_t c) {
            if (c >= ncodes) return nb;
            const uint32_t f = (uint32_t)((float)hc[c] * ratio);
            return f < nb - 1u ? f : nb - 1u;
        };
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t c = code_of(x[e]);
            const uint32_t f0 = first(c), nsub = first(c + 1u) - f0;
            const uint32_t off = sbits ? (uint32_t)((sub_of(x[e]) * nsub) >> sbits) : 0u;
            bin[e] = (uint32_t)e * NT + t < cnt ? f0 + off : 0u;
        }
        for (uint32_t i = t; i <= nb; i += NT) bins[i] = 0u;
        lds_sync();  // the code starts are read before the scatter reuses the buffer
#pragma unroll
        for (int e = 0; e < E; ++e)
            if ((uint32_t)e * NT + t < cnt) atomicAdd(&bins[bin[e]], 1u);
        lds_sync();
        big = scan_counts<NT>(bins, nb, sh, rb);
        if (big > kMaxBin) return false;
    }
    // scatter, with each word's bin beside it (in the first buffer, whose
    // words are all in registers now); afterwards bins[i] is the end of bin i
    uint32_t* binp = (uint32_t*)a;
    uint32_t pos[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        pos[e] = (uint32_t)e * NT + t < cnt ? atomicAdd(&bins[bin[e]], 1u) : 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if ((uint32_t)e * NT + t < cnt) {
            b[pos[e]] = x[e];
            binp[pos[e]] = bin[e];
        }
    }
    lds_sync();
    // ranks, by position in the binned order: the lanes of a wave mostly
    // share a bin, so their scans take the same number of steps
    for (uint32_t p = t; p < cnt; p += NT) {
        const uint64_t w = b[p];
        const uint32_t bi = binp[p];
        const uint32_t s0 = bi ? bins[bi - 1] : 0u, e0 = bins[bi];
        uint32_t r = s0;
        if (e0 - s0 > 1) {
            // eight words per step from 16-byte reads; words outside the bin
            // (up to 7 past its end, still inside the LDS allocation) do not count
            for (uint32_t q = s0 & ~1u; q < e0; q += 8) {
                const uint4* v = (const uint4*)(b + q);
                const uint4 v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
                const uint64_t y[8] = {((uint64_t)v0.y << 32) | v0.x, ((uint64_t)v0.w << 32) | v0.z,
                                       ((uint64_t)v1.y << 32) | v1.x, ((uint64_t)v1.w << 32) | v1.z,
                                       ((uint64_t)v2.y << 32) | v2.x, ((uint64_t)v2.w << 32) | v2.z,
                                       ((uint64_t)v3.y << 32) | v3.x, ((uint64_t)v3.w << 32) | v3.z};
#pragma unroll
                for (int u = 0; u < 8; ++u) r += (q + u >= s0 && q + u < e0 && y[u] > w) ? 1u : 0u;
            }
        }
        ro.put(r, cand_idx(w));
    }
    lds_sync();
    return true;
}

// Largest kept set one sort handles; larger ones are sorted in windows.
template <int NT>
QRITA_DEV uint32_t sort_cap(const Params& P) {
    return min((uint32_t)P.tail_alloc, 32u * NT);
}

// Rank order of the cnt <= sort_cap<NT>() candidates in a[0 .. cnt): a
// handful by ranking, more by the bucket sort, and sets with heavy ties by
// the bitonic sort. The LDS past the candidates (the index store and the bin
// counts) is free by now. Kept out of line: the sort's registers are then
// allocated on their own instead of on top of everything live at its call
// sites.
template <int NT>
__device__ __attribute__((always_inline)) void sort_emit(uint32_t cnt, RankOut ro, uint32_t alloc, Shared& sh, int rb) {
    cnt = uni(cnt);
    alloc = uni(alloc);
    uint64_t* a = lds_cands();
    if (cnt <= (uint32_t)NT) {
        rank_sort<NT>(a, cnt, ro, sh);
        return;
    }
    uint64_t* b = a + alloc;
    uint32_t* bins = (uint32_t*)(a + 2 * alloc);
    bool done;
    if (cnt <= 2u * NT)
        done = bucket_sort<NT, 2>(a, cnt, ro, b, bins, sh, rb);
    else if (cnt <= 4u * NT)
        done = bucket_sort<NT, 4>(a, cnt, ro, b, bins, sh, rb);
    else if (cnt <= 8u * NT)
        done = bucket_sort<NT, 8>(a, cnt, ro, b, bins, sh, rb);
    else if (cnt <= 16u * NT)
        done = bucket_sort<NT, 16>(a, cnt, ro, b, bins, sh, rb);
    else
        done = bucket_sort<NT, 32>(a, cnt, ro, b, bins, sh, rb);
    if (done) return;
    uint32_t np = next_pow2(cnt);
    if (np < 2u * NT) np = 2u * NT;
    for (uint32_t i = cnt + threadIdx.x; i < np; i += NT) a[i] = 0ull;
    lds_sync();
    switch (np / NT) {
        case 2: bitonic_sort<NT, 2>(a, ro, cnt); break;
        case 4: bitonic_sort<NT, 4>(a, ro, cnt); break;
        case 8: bitonic_sort<NT, 8>(a, ro, cnt); break;
        case 16: bitonic_sort<NT, 16>(a, ro, cnt); break;
        default: bitonic_sort<NT, 32>(a, ro, cnt); break;
    }
    lds_sync();
}

// Mask bytes of the kept set {c >= B} (when mask is set) and, when cnt > 0,
// the indices of the cnt candidates c >= Bo (Bo >= B) in rank order at
// out_idx[row][off ...]: one visit counts them per wave, a second writes the
// mask and gathers them into LDS at prefix positions (no atomics).
template <int NT, class S>
QRITA_DEV void emit_out(const Params& P, int64_t row, const S& src, uint64_t B, bool mask, uint64_t Bo,
                        uint32_t cnt, uint32_t off, Shared& sh, int& rb) {
    uint8_t* mrow = P.mask + row * (int64_t)P.vocab;
    const uint32_t bk = cand_key(B), bl = cand_low(B);
    const uint32_t ok = cand_key(Bo), ol = cand_low(Bo);
    auto keeps = [&](uint32_t key, uint32_t lw) { return key != 0 && (key > bk || (key == bk && lw >= bl)); };
    auto takes = [&](uint32_t key, uint32_t lw) { return key != 0 && (key > ok || (key == ok && lw >= ol)); };
    if (cnt == 0) {
        if (mask)
            src.template visit<true, false>([&](uint32_t key, uint32_t lw, float, int) {
                if (keeps(key, lw)) mrow[~lw] = 1;
            });
        return;
    }
    uint64_t* a = lds_cands();
    const uint32_t cap = (uint32_t)P.tail_alloc;
    uint32_t run = 0;
    if constexpr (S::kRegs) {
        uint32_t c = 0;
        src.template visit<true, false>(
            [&](uint32_t key, uint32_t lw, float, int) { c += (uint32_t)__popcll(__ballot(takes(key, lw))); });
        uint32_t total = 0;
        run = wave_prefix<NT>(c, total, sh, rb);
    } else {
        block_sync<NT>();
        if (threadIdx.x == 0) sh.gather_n = 0;
    }
    block_sync<NT>();  // the masses in the gather buffer are no longer read
    const uint32_t lane = tid_here() & (kWave - 1);
    src.template visit<true, false>([&](uint32_t key, uint32_t lw, float, int) {
        if (mask && keeps(key, lw)) mrow[~lw] = 1;
        const bool take = takes(key, lw);
        const uint64_t b = __ballot(take);
        uint32_t base = run;
        if constexpr (!S::kRegs) {
            if (b) {
                uint32_t r0 = 0;
                if (lane == 0) r0 = atomicAdd(&sh.gather_n, (uint32_t)__popcll(b));
                base = readlane(r0, 0);
            }
        }
        const uint32_t pos = base + lanes_below(b);
        if (take && pos < cap) a[pos] = ((uint64_t)key << 32) | lw;
        if constexpr (S::kRegs) run += (uint32_t)__popcll(b);
    });
    block_sync<NT>();
    sort_emit<NT>(cnt, RankOut{P.out_idx + row * (int64_t)P.idx_cap + off, cnt, nullptr, 0u}, (uint32_t)P.tail_alloc,
                  sh, rb);
}

// The candidates c >= lo_w (every candidate at or above the final boundary
// value, so the kept set and its boundary duplicates) gathered into LDS and
// sorted; the sort then writes the mask bytes of ranks < lmask and the
// indices of ranks < lout directly, so the boundary duplicates are resolved
// by their rank order (lower index first) without a separate search. The
// caller guarantees at most sort_cap<NT>() such candidates.
template <int NT, class S>
QRITA_DEV void emit_ranked(const Params& P, int64_t row, const S& src, uint64_t lo_w, uint32_t lmask,
                           uint32_t lout, Shared& sh, int& rb) {
    const uint32_t lk = cand_key(lo_w), ll = cand_low(lo_w);
    auto takes = [&](uint32_t key, uint32_t lw) { return key != 0 && (key > lk || (key == lk && lw >= ll)); };
    uint64_t* a = lds_cands();
    const uint32_t cap = sort_cap<NT>(P);
    uint32_t run = 0, cnt = 0;
    if constexpr (S::kRegs) {
        uint32_t c = 0;
        src.template visit<true, false>(
            [&](uint32_t key, uint32_t lw, float, int) { c += (uint32_t)__popcll(__ballot(takes(key, lw))); });
        run = wave_prefix<NT>(c, cnt, sh, rb);
    } else {
        block_sync<NT>();
        if (threadIdx.x == 0) sh.gather_n = 0;
    }
    block_sync<NT>();  // the masses in the gather buffer are no longer read
    const uint32_t lane = tid_here() & (kWave - 1);
    src.template visit<true, false>([&](uint32_t key, uint32_t lw, float, int) {
        const bool take = takes(key, lw);
        const uint64_t b = __ballot(take);
        uint32_t base = run;
        if constexpr (!S::kRegs) {
            if (b) {
                uint32_t r0 = 0;
                if (lane == 0) r0 = atomicAdd(&sh.gather_n, (uint32_t)__popcll(b));
                base = readlane(r0, 0);
            }
        }
        const uint32_t pos = base + lanes_below(b);
        if (take && pos < cap) a[pos] = ((uint64_t)key << 32) | lw;
        if constexpr (S::kRegs) run += (uint32_t)__popcll(b);
    });
    block_sync<NT>();
    if constexpr (!S::kRegs) cnt = uni(sh.gather_n);
    cnt = min(cnt, cap);
    RankOut ro{P.out_idx ? P.out_idx + row * (int64_t)P.idx_cap : nullptr, lout,
               P.mask ? P.mask + row * (int64_t)P.vocab : nullptr, lmask};
    sort_emit<NT>(cnt, ro, (uint32_t)P.tail_alloc, sh, rb);
}

struct TailDiag {
    int32_t n_t;
    int32_t iters;
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
        // the window: Bn <= c < prev
        S w = src;
        w.restrict_to(Bn);
        const uint32_t ok = cand_key(prev), ol = cand_low(prev);
        uint64_t* a = lds_cands();
        const uint32_t lane = tid_here() & (kWave - 1);
        block_sync<NT>();
        if (threadIdx.x == 0) sh.gather_n = 0;
        block_sync<NT>();
        w.template visit<true, false>([&](uint32_t key, uint32_t lw, float, int) {
            const bool take = key != 0 && (key < ok || (key == ok && lw < ol));
            const uint64_t b = __ballot(take);
            if (b) {
                uint32_t r0 = 0;
                if (lane == 0) r0 = atomicAdd(&sh.gather_n, (uint32_t)__popcll(b));
                const uint32_t pos = readlane(r0, 0) + lanes_below(b);
                if (take && pos < cap) a[pos] = ((uint64_t)key << 32) | lw;
            }
        });
        block_sync<NT>();
        sort_emit<NT>(cnt, RankOut{P.out_idx + row * (int64_t)P.idx_cap + done, cnt, nullptr, 0u},
                      (uint32_t)P.tail_alloc, sh, rb);
        prev = Bn;
        done += cnt;
    }
}

// The same over the row's list in memory (the n candidates the register set
// was loaded from), for kept sets larger than one sort. Returns the
// iterations spent in iters and the record-buffer parity in n_t. (The
// out-of-line functions take the parameters by value: a reference would make
// the kernel keep its parameters in scratch memory and read them per lane.)
template <int NT>
__device__ __attribute__((noinline)) TailDiag emit_windows(const Params P, int64_t row, uint32_t n, uint64_t B,
                                                           uint32_t Lout, uint32_t setn, int64_t lo_b,
                                                           uint32_t kmax, Shared& sh, int rb) {
    MemSrc<NT, false, false> src{P.glist + row * (int64_t)P.list_stride, nullptr, n, B};
    TailDiag dg{0, 0};
    emit_windows_src<NT>(P, row, src, B, Lout, setn, lo_b, kmax, sh, rb, dg);
    dg.n_t = rb;
    return dg;
}

// Steps a4-a7 on one candidate source holding n candidates (list entries
// 0 .. n-1 of the row), all with keys in (key_lo, kmax]; rest_fx is the
// fixed-point mass, relative to rest_ref, of the logits left out of the
// source (top-p-only rows). Returns false when the source does not contain
// the answer (a truncation miss); then nothing has been written.
//
// Duplicates are resolved once, at the end: the top-k search gives the K-th
// value v with n_gt above it and need = K - n_gt of its N duplicates kept;
// the top-p search then runs over the candidates >= v, counting only `need`
// of those at v (their masses are equal, so which ones does not matter for
// the mass); the final boundary value and count then pick the lowest
// indices among its duplicates.
template <int NT, class S>
QRITA_DEV bool finish_row(const Params& P, int64_t row, const RowMode& md, S& src, uint32_t n, int64_t key_lo,
                          uint32_t kmax, uint64_t rest_fx, float rest_ref, float t_gauss, Shared& sh, int& rb,
                          TailDiag& dg) {
    const uint32_t V = (uint32_t)P.vocab;
    if (P.diag) {  // #{z >= Gaussian t} among the candidates, for diagnostics
        const uint32_t key_t = f32_key(__float_as_uint(t_gauss));
        uint32_t c = 0;
        src.template visit<false, false>([&](uint32_t key, uint32_t, float, int) { c += key >= key_t ? 1u : 0u; });
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
    // kept set: {> vf} and the needf lowest-index of the Nf candidates at vf
    bool all = true;
    uint32_t vf = 0, ngt = 0, needf = 0, Nf = 0;
    // a5: top-k
    if (topk) {
        const CountOut r = qsearch_count<NT, 0>(src, 0u, K, key_lo, n, (int64_t)kmax, 0u, P.pivot_mode, sh, rb,
                                                dg.iters);
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
            src.restrict_ge(vf);
            if constexpr (S::kRegs) {
                if (S::chunks_for(ngt + Nf) < S::chunks_for(src.nslots)) src.compact(sh, rb);
            }
            ms.vx = vf;
            ms.dN = Nf - needf;
            lo = (int64_t)vf - 1;
        } else if (rest_fx) {
            // the dropped logits' mass was taken relative to rest_ref <= m
            ms.rest = (double)rest_fx * (double)mass_f32(f32_key(__float_as_uint(rest_ref)), m);
        }
        MassOut mo;
        uint64_t Tq = 0;
        if (!qsearch_mass<NT>(src, ms, m, lo, (int64_t)kmax, P.pivot_mode, sh, rb, dg.iters, mo, Tq)) return false;
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
    const uint32_t L = all ? V : ngt + needf;
    const bool mask = P.mask && !md.keep_all;
    // a7: when every candidate at or above the final boundary value fits one
    // sort, the sort's rank order resolves the duplicates and writes the
    // outputs
    {
        const bool want_idx = P.out_idx && P.idx_cap > 0;
        const uint32_t Lout = want_idx ? (L < (uint32_t)P.idx_cap ? L : (uint32_t)P.idx_cap) : 0u;
        const uint32_t Gn = all ? n : ngt + Nf;
        if ((mask || Lout > 0) && Gn <= sort_cap<NT>(P)) {
            emit_ranked<NT>(P, row, src, all ? 0ull : (uint64_t)vf << 32, mask ? L : 0u, Lout, sh, rb);
            if (P.out_count && threadIdx.x == 0) P.out_count[row] = (int32_t)L;
            return true;
        }
    }
    // a7: duplicate resolution at the final boundary value
    const uint64_t B = all ? 0ull : tie_boundary<NT>(src, vf, needf, Nf, V, 0ull, sh, rb, dg.iters);
    // a7: mask (pass 1 zero-filled the row; keep-all rows were filled there)
    // and the indices in rank order
    if (P.out_idx && P.idx_cap > 0) {
        const uint32_t Lout = L < (uint32_t)P.idx_cap ? L : (uint32_t)P.idx_cap;
        const int64_t lo_b = B ? (int64_t)cand_key(B) - 1 : key_lo;
        const uint32_t setn = all ? n : L;
        if (Lout <= sort_cap<NT>(P)) {
            uint64_t Bo = B;
            if (Lout < L) {
                if (mask) emit_out<NT>(P, row, src, B, true, B, 0u, 0u, sh, rb);
                src.restrict_to(B);
                Bo = select_boundary<NT>(src, Lout, setn, lo_b, kmax, V, P.pivot_mode, B, sh, rb, dg.iters);
                emit_out<NT>(P, row, src, B, false, Bo, Lout, 0u, sh, rb);
            } else {
                emit_out<NT>(P, row, src, B, mask, Bo, Lout, 0u, sh, rb);
            }
        } else {
            if (mask) emit_out<NT>(P, row, src, B, true, B, 0u, 0u, sh, rb);
            if constexpr (S::kRegs) {
                // a kept set larger than one sort: windows over the row list
                const TailDiag w = emit_windows<NT>(P, row, n, B, Lout, setn, lo_b, kmax, sh, rb);
                dg.iters += w.iters;
                rb = w.n_t;
            } else {
                src.restrict_to(B);
                emit_windows_src<NT>(P, row, src, B, Lout, setn, lo_b, kmax, sh, rb, dg);
            }
        }
    } else if (mask) {
        emit_out<NT>(P, row, src, B, true, B, 0u, 0u, sh, rb);
    }
    if (P.out_count && threadIdx.x == 0) P.out_count[row] = (int32_t)L;
    return true;
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

struct TailOut {
    int32_t done, path, n_t, iters, rb;
};

// The tail's slow paths, kept out of line so their registers are allocated
// apart from the register-set path: a row list too long for registers
// (searched in memory), and after a truncation miss the re-collection of the
// row with thresholds lowered to sample order statistics and, as the last
// resort, the search of the full row (§1).
template <int NT, bool BF16>
__device__ __attribute__((noinline)) TailOut tail_fallback(const Params P, int64_t row, RowMode md, float t,
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
        MemSrc<NT, false, BF16> src{lst, nullptr, nlist, 0ull};
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
            MemSrc<NT, false, BF16> src{lst, nullptr, cnt, 0ull};
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
        MemSrc<NT, true, BF16> src{nullptr, rowp, (uint32_t)V, 0ull};
        done = finish_row<NT>(P, row, md, src, (uint32_t)V, -1, kr, 0ull, 0.0f, t, sh, rb, dg);
    }
    return TailOut{done ? 1 : 0, path, dg.n_t, dg.iters, rb};
}

// Tail: one workgroup per row. A row list of up to tail_cap candidates is
// searched with the candidates in registers; everything else takes
// tail_fallback.
template <int NT, bool BF16>
__global__ __launch_bounds__(NT) void tail_kernel(Params P) {
    __shared__ Shared sh;
    int rb = 0;
    const int64_t row = blockIdx.x;
    if (row >= P.batch) return;
    const int32_t V = P.vocab;
    uint32_t* hdr = P.hdr + row * H_WORDS;
    const uint64_t* lst = P.glist + row * (int64_t)P.list_stride;
    // the head of the row list is read before the header tells how much of
    // it is filled (entries past the fill are ignored)
    uint64_t pre[kTailPre];
    {
        const uint32_t lim = min((uint32_t)P.list_stride, (uint32_t)(kTailPre * NT));
#pragma unroll
        for (int r = 0; r < kTailPre; ++r) {
            const uint32_t i = (uint32_t)r * NT + threadIdx.x;
            pre[r] = i < lim ? lst[i] : 0ull;
        }
    }
    const RowMode md = row_mode(P, row);
    const float t = __uint_as_float(uni(hdr[H_T]));
    const float tc = __uint_as_float(uni(hdr[H_TC]));
    const uint32_t nlist = uni(hdr[H_LIST]);
    const uint32_t kmax = uni(hdr[H_KMAX]);
    const bool overflow = uni(hdr[H_FLAGS]) != 0 || nlist > (uint32_t)P.list_cap;
    const uint64_t rest = (uint64_t)uni(hdr[H_REST]) | ((uint64_t)uni(hdr[H_REST + 1]) << 32);
    const bool predicted = uni(hdr[H_PRED]) != 0;

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
            RegSet<NT, kTailR> src;
            src.em = (float*)lds_cands();  // shares the sort buffer: masses are dead by the sort
            src.lows = (uint32_t*)(lds_cands() + P.tail_alloc);
            src.load(lst, nlist, pre);
            done = finish_row<NT>(P, row, md, src, nlist, key_lo, kmax, rest, tc, t, sh, rb, dg);
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
    lds_sync();
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

}  // namespace qrita
