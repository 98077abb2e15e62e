// Host side of libqrita: argument checks, launch-tier choice and the C ABI
// declared in include/qrita.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "qrita.h"
#include "select_kernel.hpp"

namespace {

using qrita::Params;

constexpr int64_t kHeaderBytes = qrita::H_WORDS * 4;
constexpr int64_t kListMax = 32768;
// tail workgroup: one wave per SIMD; up to 64 candidate keys per thread in
// registers (16384 per row) with their indices in LDS, and an LDS buffer of
// 8192 candidates for gathering the kept set (sets above 4096 are sorted in
// windows) that holds the candidates' softmax masses before that
constexpr int kTailThreads = 256;
constexpr int kTailRegCap = kTailThreads * qrita::kTailR;
constexpr int kTailLdsEntries = 8192;
// tail LDS: gather/sort buffer and masses, the candidates' indices (then the
// sort's second buffer), and the sort's bin counts
constexpr size_t kTailLds = (size_t)kTailLdsEntries * 8 + (size_t)kTailRegCap * 4 + (qrita::kSortBins + 4) * 4;

int64_t list_stride_for(int64_t vocab) { return std::min<int64_t>(vocab, kListMax); }

struct Tier {
    int threads;      // pass 1 workgroup size
    int slices;       // pass 1 workgroups per row
    int slice_len;    // logits per slice
    int stage_cap;    // pass 1 LDS candidate stage
    int stage_alloc;  // pass 1 LDS entries (>= the 2048-entry sample)
    int tail_threads;
    int tail_cap;     // tail: largest list searched in registers
    int tail_alloc;   // tail LDS entries for sorting (power of two)
    int list_cap;
};

int64_t next_pow2(int64_t x) {
    int64_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

// Tier table (the summary's tiered block sizes, "Autotuning": large blocks
// for full rows, small ones for truncated sets). Here it is a static function
// of the shape: pass 1 gets at least 1024 workgroups (all resident together
// on 256 CUs); from 512 rows on, long rows get up to eight slices of about
// 64 KiB, which keeps several rounds of workgroups queued so that the CUs
// finishing early take more, while the per-workgroup sample stays small next
// to the streamed bytes (slices of at least 8192 logits); the tail gets one
// 256-thread workgroup per row over the much smaller candidate set.
Tier choose_tier(int64_t B, int64_t V, int64_t esize, const qrita_options* o) {
    Tier t;
    int64_t S = std::max<int64_t>(1, (1024 + B - 1) / B);
    if (B >= 512) S = std::max<int64_t>(S, std::min<int64_t>(8, (V * esize + 65535) / 65536));
    S = std::min<int64_t>(S, 64);
    S = std::min<int64_t>(S, std::max<int64_t>(1, (V + 8191) / 8192));
    if (o && o->slices > 0) S = std::min<int64_t>(o->slices, std::max<int64_t>(1, V));
    // 256-thread workgroups: 1024 of them stay resident together on 256 CUs;
    // slices are whole tiles of 16 logits per thread (only a row's last slice
    // ends in a part tile), and after the first they start 16-aligned
    t.threads = 256;
    const int64_t TB = (int64_t)t.threads * 16;
    int64_t L = (V + S - 1) / S;
    L = ((L + TB - 1) / TB) * TB;
    if (o && o->slices > 0) L = ((((V + S - 1) / S) + 15) / 16) * 16;
    S = (V + L - 1) / L;
    t.slices = (int)S;
    t.slice_len = (int)L;
    int stage = 2048;
    int tail = kTailRegCap;
    if (o && o->lds_cap > 0) {
        stage = std::max(64, std::min(stage, (int)o->lds_cap));
        tail = std::max(64, std::min(tail, (int)o->lds_cap));
    }
    t.stage_cap = stage;
    t.stage_alloc = std::max(stage, qrita::kSampleN);
    t.tail_threads = kTailThreads;
    t.tail_cap = tail;
    t.tail_alloc = kTailLdsEntries;
    int64_t lc = list_stride_for(V);
    if (o && o->list_cap > 0) lc = std::max<int64_t>(1, std::min<int64_t>(lc, o->list_cap));
    t.list_cap = (int)lc;
    return t;
}

// Dynamic LDS above 64 KiB must be enabled per kernel; the largest request is
// the tail's (kTailLds, about 144 KiB) next to its static LDS.
constexpr int kMaxDynLds = 150 * 1024;

template <class Kern>
hipError_t allow_lds(Kern kern, std::once_flag& once, hipError_t& err) {
    std::call_once(once, [&] {
        err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  kMaxDynLds);
    });
    return err;
}

template <int THREADS, bool BF16>
hipError_t launch_pass1(const Params& P, const Tier& t, hipStream_t stream) {
    auto kern = qrita::pass1_kernel<THREADS, BF16>;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    if (allow_lds(kern, once, attr) != hipSuccess) return attr;
    const int64_t groups = ((P.batch + 7) / 8) * 8 * (int64_t)t.slices;
    const size_t lds = ((size_t)t.stage_alloc + (size_t)(THREADS / qrita::kWave) * qrita::kWaveSpill) * sizeof(uint64_t);
    hipLaunchKernelGGL(kern, dim3((unsigned)groups), dim3(THREADS), lds, stream, P);
    return hipGetLastError();
}

template <int THREADS, bool BF16>
hipError_t launch_tail(const Params& P, const Tier& t, hipStream_t stream) {
    auto kern = qrita::tail_kernel<THREADS, BF16>;
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    if (allow_lds(kern, once, attr) != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3((unsigned)P.batch), dim3(THREADS), kTailLds, stream, P);
    return hipGetLastError();
}

int select_impl(const void* logits, int64_t batch, int64_t vocab, int dtype, const int32_t* k,
                const float* p, uint8_t* out_mask, int32_t* out_idx, int32_t* out_count,
                int64_t idx_cap, void* workspace, size_t workspace_bytes, void* stream,
                const qrita_options* opt) {
    if (!logits || batch < 0 || vocab <= 0 || vocab > INT32_MAX || idx_cap < 0 ||
        idx_cap > INT32_MAX)
        return QRITA_EINVAL;
    if (dtype != QRITA_F32 && dtype != QRITA_BF16) return QRITA_EINVAL;
    if (out_idx && !out_count) return QRITA_EINVAL;
    if (!out_mask && !out_idx && !out_count) return QRITA_EINVAL;
    if (((uintptr_t)logits & 15u) || ((uintptr_t)out_mask & 15u)) return QRITA_EINVAL;
    if (((uintptr_t)k & 3u) || ((uintptr_t)p & 3u) || ((uintptr_t)out_idx & 3u) ||
        ((uintptr_t)out_count & 3u))
        return QRITA_EINVAL;
    if (batch > (int64_t)(INT32_MAX / 64)) return QRITA_EINVAL;
    if (batch == 0) return QRITA_OK;
    const size_t need = qrita_workspace_bytes(batch, vocab, dtype, idx_cap);
    if (!workspace || workspace_bytes < need) return QRITA_EWORKSPACE;
    if ((uintptr_t)workspace & 255u) return QRITA_EWORKSPACE;

    const Tier t = choose_tier(batch, vocab, dtype == QRITA_BF16 ? 2 : 4, opt);
    Params P;
    P.logits = logits;
    P.mask = out_mask;
    P.out_idx = out_idx;
    P.out_count = out_count;
    P.k = k;
    P.p = p;
    P.hdr = (uint32_t*)workspace;
    P.glist = (uint64_t*)((char*)workspace + ((batch * kHeaderBytes + 255) / 256) * 256);
    P.diag = opt ? opt->diag : nullptr;
    P.batch = batch;
    P.vocab = (int32_t)vocab;
    P.idx_cap = out_idx ? (int32_t)idx_cap : 0;
    P.slices = t.slices;
    P.slice_len = t.slice_len;
    P.stage_cap = t.stage_cap;
    P.tail_cap = t.tail_cap;
    P.tail_alloc = t.tail_alloc;
    P.list_cap = t.list_cap;
    P.list_stride = (int32_t)list_stride_for(vocab);
    P.force_miss = opt ? opt->force_miss : 0;
    P.delta_scale = (opt && opt->delta_scale != 0.0f) ? opt->delta_scale : 1.0f;
    P.pivot_mode = opt ? opt->pivot_mode : 0;

    hipStream_t s = (hipStream_t)stream;
    hipError_t err;
    const bool bf16 = dtype == QRITA_BF16;
    if (t.threads == 512)
        err = bf16 ? launch_pass1<512, true>(P, t, s) : launch_pass1<512, false>(P, t, s);
    else
        err = bf16 ? launch_pass1<256, true>(P, t, s) : launch_pass1<256, false>(P, t, s);
    if (err != hipSuccess) return QRITA_ELAUNCH;
    if (opt && opt->mid_event) {
        if (hipEventRecord((hipEvent_t)opt->mid_event, s) != hipSuccess) return QRITA_ELAUNCH;
    }
    err = bf16 ? launch_tail<kTailThreads, true>(P, t, s) : launch_tail<kTailThreads, false>(P, t, s);
    return err == hipSuccess ? QRITA_OK : QRITA_ELAUNCH;
}

}  // namespace

extern "C" {

size_t qrita_workspace_bytes(int64_t batch, int64_t vocab, int dtype, int64_t idx_cap) {
    (void)idx_cap;
    if (batch < 0 || vocab <= 0 || vocab > INT32_MAX) return 0;
    if (dtype != QRITA_F32 && dtype != QRITA_BF16) return 0;
    const int64_t hdr = ((batch * kHeaderBytes + 255) / 256) * 256;
    return (size_t)(hdr + batch * list_stride_for(vocab) * (int64_t)sizeof(uint64_t));
}

int qrita_workspace_init(void* workspace, size_t bytes, void* stream) {
    if (!workspace) return QRITA_EINVAL;
    if (bytes == 0) return QRITA_OK;
    if (((uintptr_t)workspace & 3u) || (bytes & 3u)) return QRITA_EINVAL;
    const uint64_t words = bytes / 4;
    const unsigned blocks = (unsigned)std::min<uint64_t>((words + 255) / 256, 4096);
    hipLaunchKernelGGL(qrita::zero_fill_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (uint32_t*)workspace, words);
    return hipGetLastError() == hipSuccess ? QRITA_OK : QRITA_ELAUNCH;
}

int qrita_select(const void* logits, int64_t batch, int64_t vocab, int dtype, const int32_t* k,
                 const float* p, uint8_t* out_mask, int32_t* out_idx, int32_t* out_count,
                 int64_t idx_cap, void* workspace, size_t workspace_bytes, void* stream) {
    return select_impl(logits, batch, vocab, dtype, k, p, out_mask, out_idx, out_count, idx_cap,
                       workspace, workspace_bytes, stream, nullptr);
}

int qrita_select_ex(const void* logits, int64_t batch, int64_t vocab, int dtype, const int32_t* k,
                    const float* p, uint8_t* out_mask, int32_t* out_idx, int32_t* out_count,
                    int64_t idx_cap, void* workspace, size_t workspace_bytes, void* stream,
                    const qrita_options* opt) {
    if (opt && (((uintptr_t)opt->diag & 3u) || opt->pivot_mode < 0 || opt->pivot_mode > 1 ||
                opt->slices < 0 || opt->lds_cap < 0 || opt->list_cap < 0 ||
                !(opt->delta_scale == opt->delta_scale)))
        return QRITA_EINVAL;
    return select_impl(logits, batch, vocab, dtype, k, p, out_mask, out_idx, out_count, idx_cap,
                       workspace, workspace_bytes, stream, opt);
}

const char* qrita_strerror(int status) {
    switch (status) {
        case QRITA_OK: return "success";
        case QRITA_EINVAL: return "invalid argument";
        case QRITA_EWORKSPACE: return "workspace missing, misaligned or too small";
        case QRITA_ELAUNCH: return "kernel launch failed";
        case QRITA_EUNSUPPORTED: return "unsupported device";
        default: return "unknown status";
    }
}

}  // extern "C"
