// Exact top-k / top-p candidate-set selection: the fused gfx950 kernel.
//
// One launch runs the whole path of the Qrita method (gist.science paper
// 2602.01518, "Metodología" and "Detalles de Implementación"):
//
//   pass 1 (every workgroup, one slice of one row):
//     a2  sampled mean / standard deviation and the normal-quantile delta
//         table give the truncation threshold t = mu + delta * sigma (§1);
//     a3  one coalesced read of the slice keeps the logits >= t (the
//         truncated set Z_t) as candidates, zero-fills the mask slice and,
//         for top-p-only rows, accumulates the softmax mass of the dropped
//         logits (§1, "Resultado": a single pass);
//   tail (the last workgroup of each row to finish pass 1):
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
//
// Rows run in parallel; small batches split each row over several
// workgroups ("slices"), combined by the last workgroup to arrive.
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
    int32_t slice_len;  // elements per slice (multiple of 16)
    int32_t stage_cap;  // pass 1: candidate capacity of the LDS stage (entries)
    int32_t tail_cap;   // tail: candidates held in LDS (entries)
    int32_t tail_alloc; // tail: LDS entries allocated (power of two >= max(tail_cap, 2048))
    int32_t list_cap;   // usable entries of the per-row list
    int32_t list_stride;
    int32_t force_miss;
    float delta_scale;
    int32_t pivot_mode;
};

// Per-row header words (zero between calls).
enum : int {
    H_LIST = 1,     // candidates in the row list (pass-1 atomics)
    H_FLAGS = 2,    // bit 0: list overflow
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

struct Shared {
    uint64_t red[2][kMaxWaves][8];
    float fred[kMaxWaves];
    uint32_t ncand;
    uint32_t flags;
    uint32_t last;
    uint32_t gather_n;
    uint32_t u32[4];
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
    int32_t kb = P.k ? P.k[row] : 0;
    float pb = P.p ? P.p[row] : 1.0f;
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
    uint32_t lcap = (P.out_idx && P.idx_cap > 0) ? (uint32_t)P.idx_cap : 0u;
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
        uint32_t u = ((const uint16_t*)rowp)[e];
        return __uint_as_float(u << 16);
    }
    return ((const float*)rowp)[e];
}

// ---------------------------------------------------------------------------
// Block reductions over a small record. Every thread ends with the combined
// value. Two slot buffers alternate, so one barrier per reduction suffices.
// ---------------------------------------------------------------------------
struct PStat {
    uint64_t M[3];
    uint32_t G[3];
    uint32_t mn[3];
    uint32_t N[3];
};

template <int THREADS>
QRITA_DEV void block_pstat(PStat& s, Shared& sh, int& rbuf, bool mass) {
    constexpr int NW = THREADS / kWave;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        uint32_t m = wave_min_u32(s.mn[j]);
        uint32_t c = (s.mn[j] == m) ? s.N[j] : 0u;
        s.N[j] = wave_sum_u32(c);
        s.mn[j] = m;
        if (mass) s.M[j] = wave_sum_u64(s.M[j]);
    }
    uint64_t* slot = sh.red[rbuf][wave];
    if (lane == 0) {
        slot[0] = (uint64_t)s.G[0] | ((uint64_t)s.G[1] << 32);
        slot[1] = (uint64_t)s.G[2] | ((uint64_t)s.mn[0] << 32);
        slot[2] = (uint64_t)s.mn[1] | ((uint64_t)s.mn[2] << 32);
        slot[3] = (uint64_t)s.N[0] | ((uint64_t)s.N[1] << 32);
        slot[4] = (uint64_t)s.N[2];
        slot[5] = s.M[0];
        slot[6] = s.M[1];
        slot[7] = s.M[2];
    }
    __syncthreads();
    PStat r;
    for (int j = 0; j < 3; ++j) {
        r.M[j] = 0;
        r.G[j] = 0;
        r.mn[j] = 0xFFFFFFFFu;
        r.N[j] = 0;
    }
    for (int w = 0; w < NW; ++w) {
        const uint64_t* q = sh.red[rbuf][w];
        uint32_t G[3] = {(uint32_t)q[0], (uint32_t)(q[0] >> 32), (uint32_t)q[1]};
        uint32_t mn[3] = {(uint32_t)(q[1] >> 32), (uint32_t)q[2], (uint32_t)(q[2] >> 32)};
        uint32_t N[3] = {(uint32_t)q[3], (uint32_t)(q[3] >> 32), (uint32_t)q[4]};
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            r.G[j] += G[j];
            r.M[j] += q[5 + j];
            if (mn[j] < r.mn[j]) {
                r.mn[j] = mn[j];
                r.N[j] = N[j];
            } else if (mn[j] == r.mn[j]) {
                r.N[j] += N[j];
            }
        }
    }
    s = r;
    rbuf ^= 1;
}

// (sum u32, min u32, max u32, sum u64) over the block.
struct Quad {
    uint32_t n, kmin, kmax;
    uint64_t sum;
};

template <int THREADS>
QRITA_DEV Quad block_quad(Quad q, Shared& sh, int& rbuf) {
    constexpr int NW = THREADS / kWave;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    q.n = wave_sum_u32(q.n);
    q.kmin = wave_min_u32(q.kmin);
    q.kmax = wave_max_u32(q.kmax);
    q.sum = wave_sum_u64(q.sum);
    uint64_t* slot = sh.red[rbuf][wave];
    if (lane == 0) {
        slot[0] = q.n;
        slot[1] = q.kmin;
        slot[2] = q.kmax;
        slot[3] = q.sum;
    }
    __syncthreads();
    Quad r{0u, 0xFFFFFFFFu, 0u, 0ull};
    for (int w = 0; w < NW; ++w) {
        const uint64_t* s = sh.red[rbuf][w];
        r.n += (uint32_t)s[0];
        r.kmin = min(r.kmin, (uint32_t)s[1]);
        r.kmax = max(r.kmax, (uint32_t)s[2]);
        r.sum += s[3];
    }
    rbuf ^= 1;
    return r;
}

// ---------------------------------------------------------------------------
// Candidate sources: the LDS array, the per-row list in global memory, or the
// row itself (the full-row fallback of §1).
// ---------------------------------------------------------------------------
struct SrcLds {
    uint32_t n;
    QRITA_DEV uint64_t get(uint32_t i) const { return lds_cands()[i]; }
    static constexpr bool kLds = true;
    static constexpr bool kRow = false;
};

struct SrcList {
    const uint64_t* ptr;
    uint32_t n;
    QRITA_DEV uint64_t get(uint32_t i) const { return ptr[i]; }
    static constexpr bool kLds = false;
    static constexpr bool kRow = false;
};

template <bool BF16>
struct SrcRow {
    const void* row;
    uint32_t n;
    QRITA_DEV uint64_t get(uint32_t i) const {
        return make_cand(f32_key(__float_as_uint(load_value<BF16>(row, i))), i);
    }
    static constexpr bool kLds = false;
    static constexpr bool kRow = true;
};

// One pass over the candidates for three pivots. field 0 tests keys of
// candidates c >= filter; field 1 tests the low words (complemented indices)
// of candidates with key == key_eq and c >= filter. With `mass`, also sums
// the fixed-point softmax mass of keys above each pivot.
template <int THREADS, class Src>
QRITA_DEV PStat pivot_pass(const Src& src, uint64_t filter, int field, uint32_t key_eq,
                           const uint32_t piv[3], bool mass, float m, Shared& sh, int& rbuf) {
    PStat s;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        s.M[j] = 0;
        s.G[j] = 0;
        s.mn[j] = 0xFFFFFFFFu;
        s.N[j] = 0;
    }
    const uint32_t n = src.n;
    for (uint32_t base = 0; base < n; base += THREADS) {
        const uint32_t i = base + threadIdx.x;
        bool ok = false;
        uint32_t f = 0;
        uint64_t e = 0;
        if (i < n) {
            uint64_t c = src.get(i);
            ok = c >= filter && (field == 0 || cand_key(c) == key_eq);
            f = field == 0 ? cand_key(c) : cand_low(c);
            if (ok && mass) e = mass_fx(f, m);
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            bool gt = ok && f > piv[j];
            s.G[j] += (uint32_t)__popcll(__ballot(gt));
            if (gt) {
                if (f < s.mn[j]) {
                    s.mn[j] = f;
                    s.N[j] = 1;
                } else if (f == s.mn[j]) {
                    s.N[j] += 1;
                }
                s.M[j] += e;
            }
        }
    }
    block_pstat<THREADS>(s, sh, rbuf, mass);
    return s;
}

QRITA_DEV void make_pivots(int64_t lo, int64_t hi, int mode, int field, uint32_t piv[3]) {
    const int64_t span = hi - lo;
    bool done = false;
    if (mode == 1 && field == 0 && lo >= 0) {
        float a = key_value((uint32_t)lo), b = key_value((uint32_t)hi);
        if (__builtin_isfinite(a) && __builtin_isfinite(b)) {
            int64_t prev = lo;
            for (int j = 1; j <= 3; ++j) {
                double v = (double)a + ((double)b - (double)a) * (0.25 * j);
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
            int64_t pj = lo + (span * j) / 4;
            if (pj <= lo) pj = lo + 1;
            if (pj >= hi) pj = hi - 1;
            piv[j - 1] = (uint32_t)pj;
        }
    }
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
template <int THREADS, class Src>
QRITA_DEV CountOut qsearch_count(const Src& src, uint64_t filter, int field, uint32_t key_eq,
                                 uint32_t K, int64_t lo, uint32_t G_lo, int64_t hi, uint32_t G_hi,
                                 int mode, Shared& sh, int& rbuf, int& iters) {
    for (int guard = 0; guard < 80; ++guard) {
        if (hi - lo <= 1) return CountOut{(uint32_t)hi, G_hi, G_lo - G_hi};
        uint32_t piv[3];
        make_pivots(lo, hi, mode, field, piv);
        PStat s = pivot_pass<THREADS>(src, filter, field, key_eq, piv, false, 0.0f, sh, rbuf);
        ++iters;
        int64_t nlo = lo, nhi = hi;
        uint32_t nGlo = G_lo, nGhi = G_hi;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            if (s.G[j] >= K) {
                if (s.G[j] - s.N[j] < K) return CountOut{s.mn[j], s.G[j] - s.N[j], s.N[j]};
                if ((int64_t)s.mn[j] > nlo) {
                    nlo = s.mn[j];
                    nGlo = s.G[j] - s.N[j];
                }
            } else if ((int64_t)piv[j] < nhi) {
                nhi = piv[j];
                nGhi = s.G[j];
            }
        }
        lo = nlo;
        hi = nhi;
        G_lo = nGlo;
        G_hi = nGhi;
    }
    return CountOut{(uint32_t)hi, G_hi, G_lo - G_hi};  // not reached for consistent inputs
}

struct MassOut {
    uint32_t v, n_gt, N;
    uint64_t M_gt;
};

// The same quaternary search over softmax mass: finds the key v with
// M(> v) < T <= M(>= v) among candidates c >= filter.
template <int THREADS, class Src>
QRITA_DEV MassOut qsearch_mass(const Src& src, uint64_t filter, double T, float m, int64_t lo,
                               uint64_t M_lo, uint32_t G_lo, int64_t hi, int mode, Shared& sh,
                               int& rbuf, int& iters) {
    uint64_t M_hi = 0;
    uint32_t G_hi = 0;
    for (int guard = 0; guard < 80; ++guard) {
        if (hi - lo <= 1) return MassOut{(uint32_t)hi, G_hi, G_lo - G_hi, M_hi};
        uint32_t piv[3];
        make_pivots(lo, hi, mode, 0, piv);
        PStat s = pivot_pass<THREADS>(src, filter, 0, 0u, piv, true, m, sh, rbuf);
        ++iters;
        int64_t nlo = lo, nhi = hi;
        uint64_t nMlo = M_lo, nMhi = M_hi;
        uint32_t nGlo = G_lo, nGhi = G_hi;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            if ((double)s.M[j] >= T) {
                uint64_t at = (uint64_t)s.N[j] * mass_fx(s.mn[j], m);
                uint64_t above = s.M[j] - at;
                if ((double)above < T) return MassOut{s.mn[j], s.G[j] - s.N[j], s.N[j], above};
                if ((int64_t)s.mn[j] > nlo) {
                    nlo = s.mn[j];
                    nMlo = above;
                    nGlo = s.G[j] - s.N[j];
                }
            } else if ((int64_t)piv[j] < nhi) {
                nhi = piv[j];
                nMhi = s.M[j];
                nGhi = s.G[j];
            }
        }
        lo = nlo;
        hi = nhi;
        M_lo = nMlo;
        M_hi = nMhi;
        G_lo = nGlo;
        G_hi = nGhi;
    }
    return MassOut{(uint32_t)hi, G_hi, G_lo - G_hi, M_hi};
}

// Boundary of "the `need` lowest-index candidates with key v, plus everything
// above v", restricted to c >= filter; N = #{key == v, c >= filter}.
template <int THREADS, class Src>
QRITA_DEV uint64_t tie_boundary(const Src& src, uint64_t filter, uint32_t v, uint32_t need,
                                uint32_t N, uint32_t V, Shared& sh, int& rbuf, int& iters) {
    uint64_t b = (uint64_t)v << 32;
    if (need < N) {
        const int64_t lo = (int64_t)(0xFFFFFFFFu - (uint32_t)(V - 1)) - 1;
        CountOut t = qsearch_count<THREADS>(src, filter, 1, v, need, lo, N, (int64_t)0xFFFFFFFFu, 0u,
                                            0, sh, rbuf, iters);
        b |= t.v;
    }
    return b > filter ? b : filter;
}

// Boundary B of the K largest candidates among c >= filter (which holds
// `total` >= K candidates, all with keys in [lo_key, kmax]).
template <int THREADS, class Src>
QRITA_DEV uint64_t select_boundary(const Src& src, uint64_t filter, uint32_t K, uint32_t total,
                                   uint32_t lo_key, uint32_t kmax, uint32_t V, int mode,
                                   Shared& sh, int& rbuf, int& iters) {
    CountOut r = qsearch_count<THREADS>(src, filter, 0, 0u, K, (int64_t)lo_key - 1, total,
                                        (int64_t)kmax, 0u, mode, sh, rbuf, iters);
    return tie_boundary<THREADS>(src, filter, r.v, K - r.n_gt, r.N, V, sh, rbuf, iters);
}

// Bitonic sort of lds[0, np), descending; np a power of two.
template <int THREADS>
QRITA_DEV void bitonic_desc(uint64_t* a, uint32_t np) {
    for (uint32_t k = 2; k <= np; k <<= 1) {
        for (uint32_t j = k >> 1; j > 0; j >>= 1) {
            for (uint32_t t = threadIdx.x; t < (np >> 1); t += THREADS) {
                uint32_t lo = 2 * j * (t / j) + (t % j);
                uint32_t hi = lo + j;
                uint64_t x = a[lo], y = a[hi];
                bool desc = (lo & k) == 0;
                if ((x < y) == desc) {
                    a[lo] = y;
                    a[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

QRITA_DEV uint32_t next_pow2(uint32_t x) {
    uint32_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

// Gather the candidates in [lo_b, hi_b) (exactly `cnt` of them, cnt <=
// lds_alloc) into LDS, sort them in rank order and write their indices to
// out_idx[row][off ...].
template <int THREADS, class Src>
QRITA_DEV void emit_indices(const Params& P, int64_t row, const Src& src, uint64_t lo_b,
                            uint64_t hi_b, uint32_t cnt, uint32_t off, Shared& sh) {
    uint64_t* a = lds_cands();
    const uint32_t n = src.n;
    if (threadIdx.x == 0) sh.gather_n = 0;
    __syncthreads();
    if (Src::kLds) {
        // In place: round r reads [r*T, (r+1)*T) into registers before any
        // write of that round; writes land below (r+1)*T.
        for (uint32_t base = 0; base < n; base += THREADS) {
            const uint32_t i = base + threadIdx.x;
            uint64_t c = i < n ? a[i] : 0ull;
            bool take = i < n && c >= lo_b && c < hi_b;
            __syncthreads();
            if (take) a[atomicAdd(&sh.gather_n, 1u)] = c;
        }
    } else {
        for (uint32_t base = 0; base < n; base += THREADS) {
            const uint32_t i = base + threadIdx.x;
            if (i < n) {
                uint64_t c = src.get(i);
                if (c >= lo_b && c < hi_b) {
                    uint32_t pos = atomicAdd(&sh.gather_n, 1u);
                    if (pos < (uint32_t)P.tail_alloc) a[pos] = c;
                }
            }
        }
    }
    __syncthreads();
    const uint32_t np = next_pow2(cnt);
    for (uint32_t i = cnt + threadIdx.x; i < np; i += THREADS) a[i] = 0ull;
    __syncthreads();
    bitonic_desc<THREADS>(a, np);
    int32_t* out = P.out_idx + row * (int64_t)P.idx_cap + off;
    for (uint32_t i = threadIdx.x; i < cnt; i += THREADS) out[i] = (int32_t)cand_idx(a[i]);
    __syncthreads();
}

struct TailDiag {
    int32_t n_t;
    int32_t iters;
};

// Steps a4-a7 of the path on one candidate source. Returns false when the
// source does not contain the answer (a truncation miss), in which case
// nothing has been written.
template <int THREADS, bool BF16, class Src>
QRITA_DEV bool finish_row(const Params& P, int64_t row, const RowMode& md, float t_gauss,
                          const Src& src, uint64_t rest_fx, float rest_ref, Shared& sh, int& rbuf,
                          TailDiag& dg) {
    const uint32_t V = (uint32_t)P.vocab;
    const uint32_t n = src.n;
    // candidate count, key range, and #{z >= Gaussian t} for diagnostics
    const uint32_t key_t = f32_key(__float_as_uint(t_gauss));
    Quad q{0u, 0xFFFFFFFFu, 0u, 0ull};
    for (uint32_t i = threadIdx.x; i < n; i += THREADS) {
        uint32_t kk = cand_key(src.get(i));
        q.kmin = min(q.kmin, kk);
        q.kmax = max(q.kmax, kk);
        q.n += kk >= key_t ? 1u : 0u;
    }
    q = block_quad<THREADS>(q, sh, rbuf);
    dg.n_t = (int32_t)q.n;

    bool topk = md.topk, topp = md.topp;
    uint32_t K = md.K;
    // a4: truncation hit test
    if (md.K_t > 0 && n < md.K_t) return false;
    if (topp && n == 0) return false;
    const float m = key_value(q.kmax);
    if (topp && m == -__builtin_inff()) {  // all -inf: keep one token
        topp = false;
        topk = true;
        K = 1;
    }
    uint64_t B = 0ull;     // kept set = {c >= B}
    uint32_t L = V;        // kept count
    uint32_t setn = n;     // candidates with c >= B
    if (topk) {
        B = select_boundary<THREADS>(src, 0ull, K, n, q.kmin, q.kmax, V, P.pivot_mode, sh, rbuf,
                                     dg.iters);
        L = K;
        setn = K;
    }
    if (topp) {
        // mass of the current set (the top-k set, or all candidates)
        Quad ms{0u, 0u, 0u, 0ull};
        for (uint32_t i = threadIdx.x; i < n; i += THREADS) {
            uint64_t c = src.get(i);
            if (c >= B) ms.sum += mass_fx(cand_key(c), m);
        }
        ms = block_quad<THREADS>(ms, sh, rbuf);
        double S;
        if (topk)
            S = (double)ms.sum;
        else if (rest_fx)
            S = (double)ms.sum + (double)rest_fx * exp((double)rest_ref - (double)m);
        else
            S = (double)ms.sum;
        const double T = (double)md.p * S;
        if (!topk && (double)ms.sum < T) return false;  // mass p not inside the candidates
        const int64_t lo = B ? (int64_t)cand_key(B) - 1 : (int64_t)q.kmin - 1;
        MassOut mo = qsearch_mass<THREADS>(src, B, T, m, lo, ms.sum, setn, (int64_t)q.kmax,
                                           P.pivot_mode, sh, rbuf, dg.iters);
        // smallest number of duplicates at v that reaches T
        const uint64_t e = mass_fx(mo.v, m);
        uint32_t need = mo.N;
        if (e > 0) {
            double x = (T - (double)mo.M_gt) / (double)e;
            uint64_t j = x <= 1.0 ? 1ull : (x >= (double)mo.N ? (uint64_t)mo.N : (uint64_t)ceil(x));
            if (j > mo.N) j = mo.N;
            if (j < 1) j = 1;
            while (j > 1 && (double)(mo.M_gt + (j - 1) * e) >= T) --j;
            while (j < mo.N && (double)(mo.M_gt + j * e) < T) ++j;
            need = (uint32_t)j;
        }
        B = tie_boundary<THREADS>(src, B, mo.v, need, mo.N, V, sh, rbuf, dg.iters);
        L = mo.n_gt + need;
        setn = L;
    }
    const int64_t roff = row * (int64_t)V;
    // a7: mask (keep-all rows were written in pass 1)
    if (P.mask && !md.keep_all) {
        uint8_t* mrow = P.mask + roff;
        if (Src::kRow) {
            for (uint32_t i = threadIdx.x; i < V; i += THREADS) mrow[i] = src.get(i) >= B ? 1 : 0;
        } else {
            for (uint32_t i = threadIdx.x; i < n; i += THREADS) {
                uint64_t c = src.get(i);
                if (c >= B) mrow[cand_idx(c)] = 1;
            }
        }
    }
    // a7: indices in rank order
    if (P.out_idx && P.idx_cap > 0) {
        const uint32_t Lout = L < (uint32_t)P.idx_cap ? L : (uint32_t)P.idx_cap;
        const uint32_t cap = (uint32_t)P.tail_alloc;
        if (Lout <= cap) {
            uint64_t Bo = B;
            if (Lout < L)
                Bo = select_boundary<THREADS>(src, B, Lout, setn, B ? cand_key(B) : q.kmin, q.kmax, V,
                                              P.pivot_mode, sh, rbuf, dg.iters);
            emit_indices<THREADS>(P, row, src, Bo, ~0ull, Lout, 0u, sh);
        } else {
            // rank windows of `cap` entries, each found by its own boundary
            uint64_t prev = ~0ull;
            for (uint32_t done = 0; done < Lout;) {
                const uint32_t cnt = min(cap, Lout - done);
                uint64_t Bn = select_boundary<THREADS>(src, 0ull, done + cnt, n, q.kmin, q.kmax, V,
                                                       P.pivot_mode, sh, rbuf, dg.iters);
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
    float x = log2f(ratio);
    float f = ceilf((x - QRITA_LUT_K_MIN) * QRITA_LUT_K_STEPS);
    int i = (int)fminf(fmaxf(f, 0.0f), (float)(QRITA_LUT_K_N - 1));
    return i;
}

// Load the row's sample into registers: 8 chunks of 256 consecutive logits at
// evenly spaced offsets (the whole row when it has at most 2048 logits).
template <bool BF16>
QRITA_DEV void load_sample(const void* rowp, int32_t V, float x[8], bool in[8]) {
    const int tid = threadIdx.x;
    const bool whole = V <= kSampleN;
    int64_t pos0 = whole ? (int64_t)tid * 8
                         : ((int64_t)(tid >> 5) * (int64_t)(V - kSampleChunk)) / (kSampleChunks - 1) +
                               (int64_t)(tid & 31) * 8;
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
QRITA_DEV float sample_rank_value(const void* rowp, int32_t V, uint32_t r, Shared& sh, int& rbuf,
                                  int& iters) {
    float x[8];
    bool in[8];
    load_sample<BF16>(rowp, V, x, in);
    uint64_t* a = lds_cands();
    __syncthreads();
    if (threadIdx.x < kSampleN / 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            a[threadIdx.x * 8 + i] = in[i] ? make_cand(f32_key(__float_as_uint(x[i])), threadIdx.x * 8 + i)
                                           : 0ull;
    }
    __syncthreads();
    SrcLds src{(uint32_t)kSampleN};
    uint32_t ns = (uint32_t)min(V, kSampleN);
    CountOut o = qsearch_count<THREADS>(src, 1ull, 0, 0u, r, -1, ns, (int64_t)0xFFFFFFFFu, 0u, 0, sh,
                                        rbuf, iters);
    __syncthreads();
    return key_value(o.v);
}

template <int THREADS, bool BF16>
QRITA_DEV Thresh compute_threshold(const Params& P, const RowMode& md, const void* rowp, Shared& sh,
                                   int& rbuf) {
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
        bool ok = in[i] && __builtin_isfinite(x[i]);
        sum += ok ? x[i] : 0.0f;
        nf += ok ? 1u : 0u;
    }
    sum = wave_sum_f32(sum);
    nf = wave_sum_u32(nf);
    if (lane == 0) {
        sh.fred[wave] = sum;
        sh.red[rbuf][wave][0] = nf;
    }
    __syncthreads();
    float tot = 0.0f;
    uint32_t n = 0;
    for (int w = 0; w < NW; ++w) {
        tot += sh.fred[w];
        n += (uint32_t)sh.red[rbuf][w][0];
    }
    rbuf ^= 1;
    __syncthreads();
    const float mu = n ? tot / (float)n : 0.0f;
    float d2 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        bool ok = in[i] && __builtin_isfinite(x[i]);
        float d = x[i] - mu;
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
            float s = 1.0f - md.p;
            float f = floorf((log2f(s) - QRITA_LUT_P_MIN) * QRITA_LUT_P_STEPS);
            int i = (int)fminf(fmaxf(f, 0.0f), (float)(QRITA_LUT_P_N - 1));
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
        if (lane == 0) sh.red[rbuf][wave][0] = c;
        __syncthreads();
        uint32_t ct = 0;
        for (int w = 0; w < NW; ++w) ct += (uint32_t)sh.red[rbuf][w][0];
        rbuf ^= 1;
        __syncthreads();
        const float lam = (float)ns * (float)md.K_t / (float)V;
        th.lambda = lam;
        if (lam >= 4.0f && (float)ct < 1.25f * lam + 2.0f) {
            uint32_t r = (uint32_t)ceilf(lam + 6.0f * sqrtf(lam) + 6.0f);
            r = min(r, ns);
            int it = 0;
            float tfb = sample_rank_value<THREADS, BF16>(rowp, V, r, sh, rbuf, it);
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
// store: wavefront ballots count them, one LDS atomic per wave reserves
// space, mbcnt gives each lane its slot. Logit j of this lane has vocabulary
// index idx0 + (j / VE) * vstride + (j % VE).
template <int THREADS, bool BF16, bool REST, int VE>
QRITA_DEV void consume16(const Params& P, int64_t row, const float f[16], uint32_t valid,
                         uint32_t idx0, uint32_t vstride, float tc, Shared& sh, uint64_t& rest) {
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
    base = __shfl(base, 0);
    const uint32_t cap = (uint32_t)P.stage_cap;
    const uint32_t spill_from = base > cap ? base : cap;
    uint32_t gbase = 0;
    if (base + tot > cap) {
        const uint32_t nover = base + tot - spill_from;
        if (lane == 0) gbase = atomicAdd(&P.hdr[row * H_WORDS + H_LIST], nover);
        gbase = __shfl(gbase, 0);
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
                    if (gp < (uint32_t)P.list_cap)
                        P.glist[row * (int64_t)P.list_stride + gp] = make_cand(f32_key(bits), idx);
                    else
                        atomicOr(&sh.flags, 1u);
                }
            }
            run += (uint32_t)__popcll(b);
        }
    }
}

template <int THREADS, bool BF16, bool REST>
QRITA_DEV void stream_slice(const Params& P, int64_t row, int64_t e0, int64_t e1, float tc,
                            uint8_t fill, Shared& sh, uint64_t& rest) {
    const int32_t V = P.vocab;
    const int64_t roff = row * (int64_t)V;
    const void* rowp = BF16 ? (const void*)((const uint16_t*)P.logits + roff)
                            : (const void*)((const float*)P.logits + roff);
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
        if (tid < kWave) consume16<THREADS, BF16, REST, 16>(P, row, f, valid, (uint32_t)e, 0u, tc, sh, rest);
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
                    uint4 w = *(const uint4*)((const uint16_t*)rowp + e);
                    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        f[q * 8 + 2 * r] = __uint_as_float(ws[r] << 16);
                        f[q * 8 + 2 * r + 1] = __uint_as_float(ws[r] & 0xFFFF0000u);
                    }
                } else {
                    float4 w = *(const float4*)((const float*)rowp + e);
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
                                           (uint32_t)(THREADS * VE), tc, sh, rest);
    }
}

// Re-collect the row's candidates >= tr into the per-row list (full-row
// fallback after a miss). Returns the number of candidates (capped at the
// list capacity); *overflow is set when the list was too small.
template <int THREADS, bool BF16>
QRITA_DEV uint32_t collect_row(const Params& P, int64_t row, float tr, bool rest_on, Shared& sh,
                               int& rbuf, uint64_t& rest_out, bool& overflow) {
    const int32_t V = P.vocab;
    const int64_t roff = row * (int64_t)V;
    const void* rowp = BF16 ? (const void*)((const uint16_t*)P.logits + roff)
                            : (const void*)((const float*)P.logits + roff);
    uint32_t* hdr = P.hdr + row * H_WORDS;
    uint64_t* lst = P.glist + row * (int64_t)P.list_stride;
    __syncthreads();
    if (threadIdx.x == 0) {
        hdr[H_LIST] = 0;
        sh.flags = 0;
    }
    __threadfence_block();
    __syncthreads();
    const uint32_t lane = threadIdx.x & (kWave - 1);
    uint64_t rest = 0;
    for (int64_t base = 0; base < V; base += THREADS) {
        const int64_t e = base + threadIdx.x;
        float f = e < V ? load_value<BF16>(rowp, e) : 0.0f;
        bool s = e < V && f >= tr;
        if (rest_on && e < V && !s) rest += fx_from_unit_f32(__expf(f - tr));
        uint64_t b = __ballot(s);
        if (b) {
            uint32_t g = 0;
            if (lane == 0) g = atomicAdd(&hdr[H_LIST], (uint32_t)__popcll(b));
            g = __shfl(g, 0);
            if (s) {
                uint32_t pos = g + lanes_below(b);
                if (pos < (uint32_t)P.list_cap)
                    lst[pos] = make_cand(f32_key(__float_as_uint(f)), (uint32_t)e);
                else
                    atomicOr(&sh.flags, 1u);
            }
        }
    }
    Quad q{0u, 0u, 0u, rest};
    q = block_quad<THREADS>(q, sh, rbuf);
    rest_out = q.sum;
    __threadfence_block();
    __syncthreads();
    if (threadIdx.x == 0) sh.u32[3] = atomicAdd(&hdr[H_LIST], 0u);
    __syncthreads();
    uint32_t cnt = sh.u32[3];
    overflow = sh.flags != 0 || cnt > (uint32_t)P.list_cap;
    __syncthreads();
    return cnt < (uint32_t)P.list_cap ? cnt : (uint32_t)P.list_cap;
}

// Pass 1: one workgroup per (row, slice). Workgroup g runs on XCD g mod 8;
// rows are dealt so that all slices of row r (and its tail) share XCD r mod 8
// and therefore one L2.
template <int THREADS, bool BF16>
__global__ __launch_bounds__(THREADS) void pass1_kernel(Params P) {
    __shared__ Shared sh;
    int rbuf = 0;
    const uint32_t g = blockIdx.x;
    const uint32_t xcd = g & 7u, jj = g >> 3;
    const uint32_t rloc = jj / (uint32_t)P.slices, slice = jj % (uint32_t)P.slices;
    const int64_t row = (int64_t)rloc * 8 + xcd;
    if (row >= P.batch) return;
    const int32_t V = P.vocab;
    const int64_t roff = row * (int64_t)V;
    const void* rowp = BF16 ? (const void*)((const uint16_t*)P.logits + roff)
                            : (const void*)((const float*)P.logits + roff);
    uint32_t* hdr = P.hdr + row * H_WORDS;
    const RowMode md = row_mode(P, row);
    if (threadIdx.x == 0) {
        sh.ncand = 0;
        sh.flags = 0;
    }
    // a2: every slice computes the same threshold from the same sample
    const Thresh th = compute_threshold<THREADS, BF16>(P, md, rowp, sh, rbuf);
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
    if (rest_on)
        stream_slice<THREADS, BF16, true>(P, row, e0, e1, th.tc, fill, sh, rest);
    else
        stream_slice<THREADS, BF16, false>(P, row, e0, e1, th.tc, fill, sh, rest);
    if (rest_on) {
        Quad q{0u, 0u, 0u, rest};
        q = block_quad<THREADS>(q, sh, rbuf);
        rest = q.sum;
    }
    __syncthreads();
    // publish: the staged candidates go to the row list in one reservation
    const uint32_t nst = min(sh.ncand, (uint32_t)P.stage_cap);
    if (threadIdx.x == 0) {
        sh.u32[0] = nst ? atomicAdd(&hdr[H_LIST], nst) : 0u;
        if (rest) atomicAdd((unsigned long long*)(hdr + H_REST), (unsigned long long)rest);
    }
    __syncthreads();
    const uint32_t gb = sh.u32[0];
    uint64_t* a = lds_cands();
    uint64_t* lst = P.glist + row * (int64_t)P.list_stride;
    bool over = false;
    for (uint32_t i = threadIdx.x; i < nst; i += THREADS) {
        const uint64_t r = a[i];
        if (gb + i < (uint32_t)P.list_cap)
            lst[gb + i] = make_cand(f32_key((uint32_t)(r >> 32)), (uint32_t)r);
        else
            over = true;
    }
    if (over) atomicOr(&sh.flags, 1u);
    __syncthreads();
    if (threadIdx.x == 0 && sh.flags) atomicOr(&hdr[H_FLAGS], 1u);
}

// Tail: one workgroup per row, after pass 1 has completed for every row.
template <int THREADS, bool BF16>
__global__ __launch_bounds__(THREADS) void tail_kernel(Params P) {
    __shared__ Shared sh;
    int rbuf = 0;
    const int64_t row = blockIdx.x;
    if (row >= P.batch) return;
    const int32_t V = P.vocab;
    const int64_t roff = row * (int64_t)V;
    const void* rowp = BF16 ? (const void*)((const uint16_t*)P.logits + roff)
                            : (const void*)((const float*)P.logits + roff);
    uint32_t* hdr = P.hdr + row * H_WORDS;
    uint64_t* lst = P.glist + row * (int64_t)P.list_stride;
    const RowMode md = row_mode(P, row);
    const float t = __uint_as_float(hdr[H_T]);
    const float tc = __uint_as_float(hdr[H_TC]);
    const uint32_t nlist = hdr[H_LIST];
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
        if (!overflow) {
            if (nlist <= (uint32_t)P.tail_cap) {
                for (uint32_t i = threadIdx.x; i < nlist; i += THREADS) a[i] = lst[i];
                __syncthreads();
                done = finish_row<THREADS, BF16>(P, row, md, t, SrcLds{nlist}, rest, tc, sh, rbuf, dg);
            } else {
                path = 1;
                done = finish_row<THREADS, BF16>(P, row, md, t, SrcList{lst, nlist}, rest, tc, sh, rbuf,
                                                 dg);
            }
        }
        // a4 fallback: re-collect with lower thresholds taken from the sample's
        // order statistics, then search the full row.
        if (!done) {
            path = 2;
            const uint32_t ns = ns_h ? ns_h : (uint32_t)min(V, kSampleN);
            const float r0 = md.K_t > 0 ? ceilf(lambda + 6.0f * sqrtf(lambda) + 6.0f) : 64.0f;
            float prev = tc;
            for (int attempt = 1; attempt <= 8 && !done; ++attempt) {
                const float rr = r0 * (float)(1u << (2 * attempt));
                float tr;
                if (rr < (float)ns) {
                    int it = 0;
                    tr = sample_rank_value<THREADS, BF16>(rowp, V, (uint32_t)rr, sh, rbuf, it);
                } else if (prev > -__builtin_inff()) {
                    tr = -__builtin_inff();
                } else {
                    break;
                }
                if (!(tr < prev)) continue;
                prev = tr;
                uint64_t rest2 = 0;
                bool ovf = false;
                const uint32_t cnt = collect_row<THREADS, BF16>(P, row, tr, md.topp && !md.topk, sh,
                                                                rbuf, rest2, ovf);
                if (ovf) break;
                done = finish_row<THREADS, BF16>(P, row, md, t, SrcList{lst, cnt}, rest2, tr, sh, rbuf,
                                                 dg);
                if (tr == -__builtin_inff()) break;
            }
            if (!done) {
                path = 3;
                done = finish_row<THREADS, BF16>(P, row, md, t, SrcRow<BF16>{rowp, (uint32_t)V}, 0ull,
                                                 0.0f, sh, rbuf, dg);
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
