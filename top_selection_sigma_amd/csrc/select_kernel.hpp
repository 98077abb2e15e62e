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
//   tail (one workgroup per row, tail_kernel.hpp; the row's candidates are
//   held in registers while the searches run):
//     a4  truncation hit test: |Z_t| >= K (or, for top-p, Z_t holds mass p);
//         on a miss the search falls back to the full row (§1);
//     a5  quaternary pivot search over the candidates: three pivots at
//         25/50/75 % of the search range per iteration, counts above each,
//         and for each pivot the smallest key above it (z_mn) with its
//         multiplicity (N_zmn); the search stops once
//         #{> z_mn} < K <= #{>= z_mn} (§2);
//     a6  the same search over softmax mass for top-p;
//     a7  duplicate resolution: the boundary duplicates kept are the lowest
//         vocabulary indices; then the mask is set and the kept indices are
//         written in rank order ("Pipeline": duplicate-handling mask
//         generation).
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "params.hpp"
#include "philox.hpp"

namespace qrita {

#include "delta_lut.inc"



constexpr int kSampleChunks = 8;
constexpr int kSampleChunk = 256;
constexpr int kSampleN = kSampleChunks * kSampleChunk;

constexpr int kTieDirect = 256;  // tie groups up to this size are ranked directly
constexpr int kTailR = 64;       // tail: candidates per thread held in registers
constexpr int kTailPre = 8;      // tail: list rows per thread read before the row header

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kHistBins = 1024;  // pass 1: sample histogram for the miss prediction (in the LDS stage)

struct Shared {
    alignas(16) uint32_t slot[2][kMaxWaves][16];  // per-wave partial records, double-buffered
    alignas(16) uint32_t ties[kTieDirect + 4];
    float fred[2 * kMaxWaves];
    uint32_t ncand;
    uint32_t flags;
    uint32_t gather_n;
    alignas(8) uint32_t u32[8];
    uint32_t wspill[kMaxWaves];  // pass 1: entries left in each wave's spill buffer
    uint32_t nsub;               // pass 1: entries reserved in the slice's sub-list
    uint32_t cnt[kMaxSlices];    // tail: candidates per slice
    uint32_t pre[kMaxSlices + 1];  // tail: prefix of cnt
    uint32_t row;                  // tail: the row taken from the counter
};

extern __shared__ uint64_t qrita_dyn_lds[];

QRITA_DEV uint64_t* lds_cands() { return qrita_dyn_lds; }

struct RowMode {
    bool topk, topp, keep_all;
    uint32_t K;    // top-k size (V when off)
    float p;
    uint32_t K_t;  // ranks the candidate set must contain (0: mass-driven or none)
    bool need_cand;
    bool sample_all;  // a draw over a row that keeps every token (needs its whole mass)
    float p_table;    // the top-p the threshold table is read at
    QRITA_DEV bool rest_on() const { return (topp && !topk) || sample_all; }
};

QRITA_DEV RowMode row_mode(const Params& P, int64_t row) {
    RowMode m;
    const int32_t V = P.vocab;
    // the same in every lane (readfirstlane keeps what follows in scalar registers)
    const int32_t kb = P.k ? (int32_t)__builtin_amdgcn_readfirstlane(P.k[row]) : 0;
    const float pb = P.p ? __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(P.p[row]))) : 1.0f;
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
    else if (!P.idx_order)
        m.K_t = lcap < (uint32_t)V ? lcap : (uint32_t)V;
    else
        m.K_t = 0;  // keep-all rows in index order: indices 0, 1, ... need no candidates
    m.need_cand = m.topk || m.topp || m.K_t > 0;
    // a draw over a keep-all row: candidates as for top-p 0.999, the mass of
    // the logits left out accumulated so that the draw can tell a miss
    m.sample_all = P.out_token != nullptr && m.keep_all;
    m.p_table = m.sample_all ? 0.999f : m.p;
    if (m.sample_all) m.need_cand = true;
    return m;
}


template <int DT>
QRITA_DEV float load_value(const void* rowp, int64_t e) {
    if constexpr (kW16<DT>) return lo16<DT>(((const uint16_t*)rowp)[e]);
    else return ((const float*)rowp)[e];
}

template <int DT>
QRITA_DEV const void* row_ptr(const Params& P, int64_t row) {
    const int64_t roff = row * (int64_t)P.vocab;
    return kW16<DT> ? (const void*)((const uint16_t*)P.logits + roff)
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
template <int DT>
QRITA_DEV void load_sample(const void* rowp, int32_t V, float x[8], bool in[8]) {
    const int tid = threadIdx.x;
    const bool whole = V <= kSampleN;
    int64_t pos0 =
        whole ? (int64_t)tid * 8
              : ((int64_t)(tid >> 5) * (int64_t)(V - kSampleChunk)) / (kSampleChunks - 1) + (int64_t)(tid & 31) * 8;
    constexpr int64_t ES = kW16<DT> ? 2 : 4;
    const int64_t mis = (int64_t)(((uintptr_t)rowp / ES + (uint64_t)pos0) & (kW16<DT> ? 7 : 3));
    if (!whole && tid < kSampleN / 8 && pos0 >= mis && pos0 - mis + 8 <= V) {
        pos0 -= mis;
#pragma unroll
        for (int i = 0; i < 8; ++i) in[i] = true;
        if (kW16<DT>) {
            const u32x4_t w = *(const u32x4_t*)((const uint16_t*)rowp + pos0);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[2 * r] = lo16<DT>(ws[r]);
                x[2 * r + 1] = hi16<DT>(ws[r]);
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
        x[i] = in[i] ? load_value<DT>(rowp, e) : 0.0f;
    }
}


template <int THREADS, int DT>
QRITA_DEV Thresh compute_threshold(const Params& P, const RowMode& md, const void* rowp, const float (&x)[8],
                                   const bool (&in)[8], float c0, Shared& sh, int& rb) {
    constexpr int NW = THREADS / kWave;
    const float kInf = __builtin_inff();
    Thresh th{kInf, kInf, false, 0u, 0.0f};
    if (!md.need_cand) return th;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int32_t V = P.vocab;
    // the candidate stage is free until the streaming pass: it holds the
    // sample histogram meanwhile
    uint32_t* hist = (uint32_t*)lds_cands();
    for (int i = threadIdx.x; i < kHistBins; i += THREADS) hist[i] = 0u;
    // the table entries depend on K, p and V only: read them while the sample
    // is in flight
    const float cap = qrita_lut_k[lut_k_index(1.0f / (float)V)];
    float tab = 0.0f, tabp = 0.0f;
    if (md.K_t > 0) tab = qrita_lut_k[lut_k_index((float)md.K_t / (float)V)];
    if (md.K_t == 0 || md.sample_all) {
        const float s = 1.0f - md.p_table;
        const float f = floorf((log2f(s) - QRITA_LUT_P_MIN) * QRITA_LUT_P_STEPS);
        const int i = (int)fminf(fmaxf(f, 0.0f), (float)(QRITA_LUT_P_N - 1));
        tabp = qrita_lut_p[i];
    }
    asm volatile("" ::"s"(cap), "s"(tab), "s"(tabp));
    // mean, variance and range of the finite sample values in one reduction
    // (moments about the row's first logit c0, fixed reduction order)
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
        // top-p: softmax mass of N(mu, sigma^2) above t is
        // 1 - Phi((t - mu)/sigma - sigma); keep at least p of it, less a margin.
        const float delta_p = fminf(sigma + tabp - 0.5f, cap);
        if (md.K_t > 0) {
            delta = tab;
            // a draw over a keep-all row with index output: both the ranks
            // and the mass must be covered
            if (md.sample_all) delta = fminf(delta, delta_p);
        } else {
            delta = delta_p;
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
    // (r = lambda + 4 sqrt(lambda) + 4), so the miss is served from the same
    // single pass. That value is read off a 1024-bin histogram of the sample
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
                atomicAdd(&hist[b], 1u);
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
            const uint32_t r = min((uint32_t)ceilf(lam + 4.0f * sqrtf(lam) + 4.0f), ns);
            // every wave scans the histogram from the top: lane l holds bins
            // 16l .. 16l+15, and the suffix counts come from a DPP scan
            constexpr int BPL = kHistBins / kWave;
            uint32_t bc[BPL];
            uint32_t own = 0;
#pragma unroll
            for (int j = 0; j < BPL; ++j) {
                bc[j] = hist[BPL * lane + j];
                own += bc[j];
            }
            const uint32_t above = wave_suffix_sum_excl(own);  // bins of higher lanes
            // highest bin whose count from the top reaches r
            int bin = -1;
            uint32_t run = above;
#pragma unroll
            for (int j = BPL - 1; j >= 0; --j) {
                run += bc[j];
                bin = (bin < 0 && run >= r) ? BPL * lane + j : bin;
            }
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

// Survivors past the LDS stage. Each wave first collects them, already in
// list form, in its own LDS buffer of kWaveSpill entries (after the stage)
// and moves a full buffer to the row list with one reservation; what is left
// joins the stage's reservation at the end of the slice. Only a tile whose
// spill alone exceeds the buffer reserves list space directly.
constexpr uint32_t kWaveSpill = 512;

struct Spill {
    uint32_t kmax;  // largest key spilled by this lane
    uint32_t n;     // entries in this wave's buffer (wave uniform)
};

// the stage takes max(stage_cap, kSampleN) entries; the wave buffers follow
QRITA_DEV uint64_t* wave_spill_buf(const Params& P) {
    const uint32_t stage = (uint32_t)P.stage_cap > (uint32_t)kSampleN ? (uint32_t)P.stage_cap : (uint32_t)kSampleN;
    return lds_cands() + stage + (threadIdx.x / kWave) * kWaveSpill;
}

// The sub-list a slice owns in its row's list.
QRITA_DEV uint64_t* sub_list(const Params& P, int64_t row, uint32_t slice) {
    return P.glist + row * (int64_t)P.list_stride + (int64_t)slice * P.sub_cap;
}

// Move this wave's n buffered entries to the slice's sub-list (space is
// reserved with an LDS counter: the sub-list belongs to this workgroup).
QRITA_DEV void wave_spill_flush(const Params& P, uint64_t* sub, const uint64_t* wb, uint32_t n, Shared& sh) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    uint32_t g = 0;
    if (lane == 0) g = atomicAdd(&sh.nsub, n);
    g = readlane(g, 0);
    for (uint32_t j = lane; j < n; j += kWave) {
        const uint32_t gp = g + j;
        if (gp < (uint32_t)P.sub_cap) sub[gp] = wb[j];
    }
}

// The candidate stage holds kSampleN entries as two arrays of words: the
// logits' bits, then their vocabulary indices (a survivor is two 32-bit
// writes at one address and a fixed offset).
constexpr uint32_t kStageN = kSampleN;

// Compact the survivors (f >= tc) of 16 logits per lane into the candidate
// stage: wavefront ballots count them, one LDS atomic per wave reserves
// space, mbcnt gives each lane its slot. For each of the 16 positions the
// mask of lanes holding a survivor there comes straight from the comparison
// (a scalar register pair), so the wave-uniform tests are scalar. Logit j of this lane has vocabulary
// index idx0 + (j / VE) * vstride + (j % VE); bit j of `valid` marks it as
// present. Survivors past the stage go to the wave's spill buffer (with their
// key, for the list's max). For top-p-only rows (REST) the dropped logits'
// masses exp(f - tc) are summed per lane in float over the 16 and added to
// the fixed-point `rest` once, so the total does not depend on lane order.
template <int THREADS, int DT, bool REST, int VE>
QRITA_DEV void consume16(const Params& P, uint64_t* sub, const float f[16], uint32_t valid, uint32_t idx0,
                         uint32_t vstride, float tc, Shared& sh, uint64_t& rest, Spill& sp) {
    const uint32_t lane = threadIdx.x & (kWave - 1);
    uint32_t tot = 0;
    float dropped = 0.0f;
    // the survivors of logit j of every lane: wave-uniform (every lane takes
    // both masks; valid differs by lane), in scalar registers
    auto mask = [&](int j) { return __builtin_amdgcn_fcmpf(f[j], tc, 3) & __ballot((valid >> j) & 1u); };
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const bool v = (valid >> j) & 1u;
        tot += (uint32_t)__popcll(mask(j));
        if (REST) dropped += (v && !(f[j] >= tc)) ? __expf(f[j] - tc) : 0.0f;
    }
    if (REST) rest += fx_from_unit_f32(fminf(dropped * 0x1p-5f, 1.0f)) << 5;
    if (tot == 0) return;
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&sh.ncand, tot);
    base = readlane(base, 0);
    const uint32_t cap = (uint32_t)P.stage_cap;
    uint32_t* a = (uint32_t*)lds_cands();
    uint32_t run = base;
    if (base + tot <= cap) {
        // the whole group fits the stage
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint64_t b = mask(j);
            if (b) {
                if (((valid >> j) & 1u) && f[j] >= tc) {
                    const uint32_t pos = run + lanes_below(b);
                    a[pos] = __float_as_uint(f[j]);
                    a[kStageN + pos] = idx0 + (uint32_t)(j / VE) * vstride + (uint32_t)(j % VE);
                }
                run += (uint32_t)__popcll(b);
            }
        }
        return;
    }
    const uint32_t spill_from = base > cap ? base : cap;
    const uint32_t nover = base + tot - spill_from;
    uint64_t* wb = wave_spill_buf(P);
    if (sp.n + nover > kWaveSpill) {
        wave_spill_flush(P, sub, wb, sp.n, sh);
        sp.n = 0;
    }
    const bool direct = nover > kWaveSpill;
    uint32_t gbase = 0;
    if (direct) {
        if (lane == 0) gbase = atomicAdd(&sh.nsub, nover);
        gbase = readlane(gbase, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint64_t b = mask(j);
        if (b) {
            if (((valid >> j) & 1u) && f[j] >= tc) {
                const uint32_t pos = run + lanes_below(b);
                const uint32_t bits = __float_as_uint(f[j]);
                const uint32_t idx = idx0 + (uint32_t)(j / VE) * vstride + (uint32_t)(j % VE);
                if (pos < cap) {
                    a[pos] = bits;
                    a[kStageN + pos] = idx;
                } else {
                    const uint32_t off = pos - spill_from;
                    const uint32_t key = f32_key(bits);
                    sp.kmax = key > sp.kmax ? key : sp.kmax;
                    const uint64_t c = make_cand(key, idx);
                    if (!direct) {
                        wb[sp.n + off] = c;
                    } else if (gbase + off < (uint32_t)P.sub_cap) {
                        sub[gbase + off] = c;
                    }
                }
            }
            run += (uint32_t)__popcll(b);
        }
    }
    if (!direct) sp.n += nover;
}

// One tile is THREADS * 16 logits, 16 per lane in 16-byte vectors (two for
// bf16, four for f32). Tiles are loaded raw, marked non-temporal (the logits
// are read once), and unpacked to float only when consumed, so that several
// tiles can be in flight per lane: kTileDepth tiles, 96 bytes of bf16 or
// 128 bytes of f32 per lane, 96-128 KiB per CU at four workgroups.
template <int DT>
struct RawTile {
    u32x4_t v[kW16<DT> ? 2 : 4];
};
template <int DT>
constexpr int kTileDepth = kW16<DT> ? 3 : 2;

template <int THREADS, int DT>
QRITA_DEV void load_raw(const void* rowp, int64_t tile, RawTile<DT>& r) {
    constexpr int VE = kW16<DT> ? 8 : 4;
    constexpr int NV = 16 / VE;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        const int64_t e = tile + (int64_t)q * THREADS * VE + (int64_t)threadIdx.x * VE;
        const u32x4_t* src = kW16<DT> ? (const u32x4_t*)((const uint16_t*)rowp + e) : (const u32x4_t*)((const float*)rowp + e);
        r.v[q] = __builtin_nontemporal_load(src);
    }
}

template <int DT>
QRITA_DEV void unpack_tile(const RawTile<DT>& r, float f[16]) {
    if (kW16<DT>) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t ws[4] = {r.v[q].x, r.v[q].y, r.v[q].z, r.v[q].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f[q * 8 + 2 * i] = lo16<DT>(ws[i]);
                f[q * 8 + 2 * i + 1] = hi16<DT>(ws[i]);
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[q * 4 + 0] = __uint_as_float(r.v[q].x);
            f[q * 4 + 1] = __uint_as_float(r.v[q].y);
            f[q * 4 + 2] = __uint_as_float(r.v[q].z);
            f[q * 4 + 3] = __uint_as_float(r.v[q].w);
        }
    }
}

// The mask bytes of one full tile (this lane's 16 entries).
template <int THREADS, int DT>
QRITA_DEV void fill_tile(uint8_t* mrow, int64_t tile, uint8_t fill) {
    constexpr int VE = kW16<DT> ? 8 : 4;
    constexpr int NV = 16 / VE;
    const uint64_t fill8 = 0x0101010101010101ull * fill;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        const int64_t e = tile + (int64_t)q * THREADS * VE + (int64_t)threadIdx.x * VE;
        if (kW16<DT>)
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

// The streaming pass over [e0, e1); ring[j] holds the slice's full tile j
// for j < kTileDepth (loaded before the threshold was known).
template <int THREADS, int DT, bool REST>
QRITA_DEV void stream_slice(const Params& P, int64_t row, uint64_t* sub, int64_t e0, int64_t e1, float tc,
                            uint8_t fill, RawTile<DT> (&ring)[kTileDepth<DT>], Shared& sh, uint64_t& rest,
                            Spill& sp) {
    const int64_t roff = row * (int64_t)P.vocab;
    const void* rowp = row_ptr<DT>(P, row);
    // the mask slice is filled here only when the tail does not write whole rows
    uint8_t* mrow = (P.mask && !P.bitmap) ? P.mask + roff : nullptr;
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
            f[0] = load_value<DT>(rowp, e);
            valid = 1;
            if (mrow) mrow[e] = fill;
        }
        if (tid < kWave)
            consume16<THREADS, DT, REST, 16>(P, sub, f, valid, (uint32_t)e, 0u, tc, sh, rest, sp);
    }
    constexpr int VE = kW16<DT> ? 8 : 4;  // logits per 16-byte vector
    constexpr int NV = 16 / VE;       // vectors per thread per tile
    constexpr int TB = THREADS * 16;  // logits per tile
    constexpr int D = kTileDepth<DT>;
    // full tiles: tile i sits in ring[i % D]; once unpacked, its slot is
    // refilled with tile i + D
    const int64_t nfull = (e1 - a) / TB;
    for (int64_t i0 = 0; i0 < nfull; i0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int64_t i = i0 + j;
            if (i < nfull) {
                const int64_t tile = a + i * TB;
                float f[16];
                unpack_tile<DT>(ring[j], f);
                if (i + D < nfull) load_raw<THREADS, DT>(rowp, tile + (int64_t)D * TB, ring[j]);
                if (mrow) fill_tile<THREADS, DT>(mrow, tile, fill);
                consume16<THREADS, DT, REST, VE>(P, sub, f, 0xFFFFu, (uint32_t)(tile + (int64_t)tid * VE),
                                                   (uint32_t)(THREADS * VE), tc, sh, rest, sp);
            }
        }
    }
    // ragged last tile: vectors wholly inside the slice as in a full tile,
    // the one that straddles its end element by element
    const int64_t tile = a + nfull * TB;
    if (tile < e1) {
        float f[16];
        uint32_t valid = 0;
        const uint64_t fill8 = 0x0101010101010101ull * fill;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int64_t ev = tile + (int64_t)q * THREADS * VE + (int64_t)tid * VE;
            if (ev + VE <= e1) {
                RawTile<DT> r1;
                const u32x4_t* src = kW16<DT> ? (const u32x4_t*)((const uint16_t*)rowp + ev)
                                          : (const u32x4_t*)((const float*)rowp + ev);
                r1.v[0] = __builtin_nontemporal_load(src);
                const uint32_t ws[4] = {r1.v[0].x, r1.v[0].y, r1.v[0].z, r1.v[0].w};
#pragma unroll
                for (int r = 0; r < VE; ++r)
                    f[q * VE + r] = kW16<DT> ? ((r & 1) ? hi16<DT>(ws[r / 2]) : lo16<DT>(ws[r / 2]))
                                             : __uint_as_float(ws[r]);
                valid |= ((1u << VE) - 1u) << (q * VE);
                if (mrow) {
                    if (kW16<DT>)
                        __builtin_nontemporal_store(fill8, (uint64_t*)(mrow + ev));
                    else
                        __builtin_nontemporal_store((uint32_t)fill8, (uint32_t*)(mrow + ev));
                }
            } else {
#pragma unroll
                for (int r = 0; r < VE; ++r) {
                    const int64_t er = ev + r;
                    if (er < e1) {
                        f[q * VE + r] = load_value<DT>(rowp, er);
                        valid |= 1u << (q * VE + r);
                        if (mrow) mrow[er] = fill;
                    } else {
                        f[q * VE + r] = 0.0f;
                    }
                }
            }
        }
        consume16<THREADS, DT, REST, VE>(P, sub, f, valid, (uint32_t)(tile + (int64_t)tid * VE),
                                           (uint32_t)(THREADS * VE), tc, sh, rest, sp);
    }
}

// Pass 1: one workgroup per (row, slice). Workgroup g runs on XCD g mod 8;
// rows are dealt so that all slices of row r share XCD r mod 8 and therefore
// one L2, which also holds the row list when the row's tail (workgroup r of
// the next launch, on the same XCD, unless rows are counted out) reads it. A
// slice writes only its own sub-list and record: no global atomics, no state
// carried between calls. Workgroup 0 also zeroes the tail's row counter.
//
// pass1_slice is the work of one (row, slice); the tail's one-launch path
// runs it for a whole row (one slice) before the row's selection.
template <int THREADS, int DT>
QRITA_DEV void pass1_slice(const Params& P, int64_t row, uint32_t slice, Shared& sh, int& rb) {
    const int32_t V = P.vocab;
    const int64_t roff = row * (int64_t)V;
    const void* rowp = row_ptr<DT>(P, row);
    uint64_t* sub = sub_list(P, row, slice);
    const RowMode md = row_mode(P, row);
    if (threadIdx.x == 0) {
        sh.ncand = 0;
        sh.nsub = 0;
    }
    // this workgroup's slice; slices after the first start 16-aligned
    const int64_t A = (16 - (roff & 15)) & 15;
    int64_t e0 = slice == 0 ? 0 : A + (int64_t)slice * P.slice_len;
    int64_t e1 = A + (int64_t)(slice + 1) * P.slice_len;
    if (slice + 1 == (uint32_t)P.slices || e1 > V) e1 = V;
    if (e0 > V) e0 = V;
    // a2: every slice computes the same threshold from the same sample, whose
    // loads are issued first; the slice's first kTileDepth full tiles are in
    // flight while the threshold is computed
    float xs[8];
    bool ins[8];
    float c0 = 0.0f;
    if (md.need_cand) {
        load_sample<DT>(rowp, V, xs, ins);
        c0 = load_value<DT>(rowp, 0);
    }
    RawTile<DT> ring[kTileDepth<DT>];
    {
        const int64_t a = aligned_start(roff, e0, e1);
        const int64_t nfull = (e1 - a) / ((int64_t)THREADS * 16);
#pragma unroll
        for (int j = 0; j < kTileDepth<DT>; ++j)
            if (j < nfull) load_raw<THREADS, DT>(rowp, a + (int64_t)j * THREADS * 16, ring[j]);
    }
    const Thresh th = compute_threshold<THREADS, DT>(P, md, rowp, xs, ins, c0, sh, rb);
    if (slice == 0 && threadIdx.x == 0) {
        uint32_t* rr = P.rowrec + row * R_WORDS;
        *(uint4*)rr = make_uint4(__float_as_uint(th.t), __float_as_uint(th.tc), th.predicted ? 1u : 0u,
                                 __float_as_uint(th.lambda));
        rr[R_NS] = th.n_s;
    }
    __syncthreads();
    // a3: the single streaming pass over the slice
    const uint8_t fill = md.keep_all ? 1 : 0;
    const bool rest_on = md.rest_on();
    uint64_t rest = 0;
    Spill sp{0u, 0u};
    if (rest_on)
        stream_slice<THREADS, DT, true>(P, row, sub, e0, e1, th.tc, fill, ring, sh, rest, sp);
    else
        stream_slice<THREADS, DT, false>(P, row, sub, e0, e1, th.tc, fill, ring, sh, rest, sp);
    const uint32_t lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0) sh.wspill[wave] = sp.n;
    __syncthreads();
    // publish: the staged candidates and what the spill buffers still hold go
    // to the sub-list in one reservation
    const uint32_t nst = min(sh.ncand, (uint32_t)P.stage_cap);
    uint32_t wpre = 0, wtot = 0;
#pragma unroll
    for (int w = 0; w < THREADS / kWave; ++w) {
        const uint32_t q = sh.wspill[w];
        wpre += (uint32_t)w < wave ? q : 0u;
        wtot += q;
    }
    uint32_t kmax = sp.kmax;
    uint32_t gb = 0;
    if (threadIdx.x == 0) gb = atomicAdd(&sh.nsub, nst + wtot);
    constexpr int PER = kStageN / THREADS;  // stage entries per thread (stage_cap <= kStageN)
    const uint32_t* a = (const uint32_t*)lds_cands();
    uint32_t keys[PER], lows[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const uint32_t i = (uint32_t)u * THREADS + threadIdx.x;
        keys[u] = i < nst ? f32_key(a[i]) : 0u;
        lows[u] = ~(i < nst ? a[kStageN + i] : 0u);
        kmax = keys[u] > kmax ? keys[u] : kmax;
    }
    if (threadIdx.x == 0) sh.u32[0] = gb;
    uint32_t d0 = 0, d1 = 0;
    block_sum_min_max<THREADS>(d0, d1, kmax, rest, sh, rb);
    gb = sh.u32[0];
    const uint32_t cap = (uint32_t)P.sub_cap;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const uint32_t i = (uint32_t)u * THREADS + threadIdx.x;
        if (i < nst && gb + i < cap) sub[gb + i] = ((uint64_t)keys[u] << 32) | lows[u];
    }
    {
        const uint64_t* wb = wave_spill_buf(P);
        const uint32_t g = gb + nst + wpre;
        for (uint32_t j = lane; j < sp.n; j += kWave)
            if (g + j < cap) sub[g + j] = wb[j];
    }
    // the slice record: its count (above sub_cap: the sub-list overflowed),
    // largest key and dropped mass
    if (threadIdx.x == 0)
        *(uint4*)(P.slrec + (row * kMaxSlices + slice) * S_WORDS) =
            make_uint4(gb + nst + wtot, kmax, (uint32_t)rest, (uint32_t)(rest >> 32));
}

template <int THREADS, int DT>
__global__ __launch_bounds__(THREADS, 4) void pass1_kernel(Params P) {
    __shared__ Shared sh;
    int rb = 0;
    const uint32_t g = blockIdx.x;
    if (P.queue && g == 0 && threadIdx.x == 0) *P.queue = 0u;
    const uint32_t xcd = g & 7u, jj = g >> 3;
    const uint32_t rloc = jj / (uint32_t)P.slices, slice = jj % (uint32_t)P.slices;
    const int64_t row = (int64_t)rloc * 8 + xcd;
    if (row >= P.batch) return;
    pass1_slice<THREADS, DT>(P, row, slice, sh, rb);
}

// Re-collect the row's candidates >= tr into the per-row list (full-row
// fallback after a miss). Returns the number of candidates (capped at the
// list capacity); *overflow is set when the list was too small, *kmax_out is
// the largest key and *rest_out the fixed-point mass (relative to tr) of the
// logits below tr. Survivors are staged in LDS (stage, stage_cap entries)
// and written to the list in bursts between batches of loads: stores mixed
// into the streaming loads would make every batch wait for them.
template <int THREADS, int DT>
QRITA_DEV uint32_t collect_row(const Params& P, int64_t row, float tr, bool rest_on, uint64_t* stage,
                               uint32_t stage_cap, Shared& sh, int& rb, uint64_t& rest_out, uint32_t& kmax_out,
                               bool& overflow) {
    const int32_t V = P.vocab;
    const void* rowp = row_ptr<DT>(P, row);
    uint64_t* lst = P.glist + row * (int64_t)P.list_stride;
    const uint32_t lcap = (uint32_t)P.list_cap;
    __syncthreads();
    if (threadIdx.x == 0) sh.gather_n = 0;
    __syncthreads();
    const uint32_t lane = threadIdx.x & (kWave - 1);
    uint64_t rest = 0;
    uint32_t kmax = 0;
    uint32_t flushed = 0;  // entries below this position are in the list already
    // stage entries [flushed, flushed + stage_cap) go to stage[pos - flushed];
    // two batches add at most 2 * THREADS * U, so with a flush once half the
    // stage is used, later positions only arise when the stage is smaller
    // than that (they are then written to the list directly)
    constexpr int U = 16;
    auto flush = [&](uint32_t upto) {
        const uint32_t n = min(upto - flushed, stage_cap);
        for (uint32_t i = threadIdx.x; i < n; i += THREADS)
            if (flushed + i < lcap) lst[flushed + i] = stage[i];
        flushed = upto;
    };
    // the index is clamped and the value masked afterwards, so the loads do
    // not turn into branches that wait for each load in turn
    auto load = [&](int64_t base, float (&fv)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = base + (int64_t)u * THREADS + threadIdx.x;
            const float x = load_value<DT>(rowp, e < V ? e : V - 1);
            fv[u] = e < V ? x : 0.0f;
        }
    };
    // one batch of U logits per thread: the wave's survivors are counted
    // first and reserved with a single LDS atomic, then written to the stage
    auto consume = [&](int64_t base, const float (&fv)[U]) {
        uint32_t tot = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = base + (int64_t)u * THREADS + threadIdx.x;
            const bool s = e < V && fv[u] >= tr;
            if (rest_on && e < V && !s) rest += fx_from_unit_f32(__expf(fv[u] - tr));
            tot += (uint32_t)__popcll(__ballot(s));
        }
        if (tot == 0) return;
        uint32_t g = 0;
        if (lane == 0) g = atomicAdd(&sh.gather_n, tot);
        uint32_t run = readlane(g, 0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = base + (int64_t)u * THREADS + threadIdx.x;
            const bool s = e < V && fv[u] >= tr;
            const uint64_t b = __ballot(s);
            if (s) {
                const uint32_t pos = run + lanes_below(b);
                const uint32_t key = f32_key(__float_as_uint(fv[u]));
                kmax = key > kmax ? key : kmax;
                const uint64_t c = make_cand(key, (uint32_t)e);
                if (pos - flushed < stage_cap)
                    stage[pos - flushed] = c;
                else if (pos < lcap)
                    lst[pos] = c;
            }
            run += (uint32_t)__popcll(b);
        }
    };
    // two batches alternate: the next one's loads are in flight while the
    // current one is consumed; the stage is flushed when half full
    const int64_t step = (int64_t)THREADS * U;
    float fa[U], fb[U];
    load(0, fa);
    for (int64_t base = 0; base < V; base += 2 * step) {
        if (base + step < V) load(base + step, fb);
        consume(base, fa);
        if (base + 2 * step < V) load(base + 2 * step, fa);
        if (base + step < V) consume(base + step, fb);
        __syncthreads();
        const uint32_t now = sh.gather_n;
        if (now - flushed > stage_cap / 2) {
            flush(now);
            __syncthreads();  // the stage is read before later batches refill it
        }
    }
    flush(sh.gather_n);
    uint32_t d0 = 0, d1 = 0;
    block_sum_min_max<THREADS>(d0, d1, kmax, rest, sh, rb);
    __syncthreads();
    rest_out = rest;
    kmax_out = kmax;
    const uint32_t cnt = sh.gather_n;
    overflow = cnt > lcap;
    __syncthreads();
    return cnt < lcap ? cnt : lcap;
}

}  // namespace qrita

#include "tail_kernel.hpp"
