// Host side of libqrita: argument checks, the tier table and the C ABI
// declared in include/qrita.h. The kernels are compiled in their own
// translation units (pass1.hip, tail_light.hip, tail_heavy.hip).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "philox.hpp"
#include "qrita.h"

namespace {

using qrita::Params;

constexpr int64_t kListMax = 32768;   // per-row candidate list (entries of 8 bytes)
constexpr int kMaxChunks = 16;        // row chunks of one call
constexpr int kSmallSet = 4096;       // candidate sets sorted and scanned instead of searched
constexpr int kPass1Threads = 256;
constexpr int kSampleN = 2048;        // pass 1 sample (its LDS stage holds at least this many entries)
constexpr int kStageCap = 2048;       // pass 1 LDS candidate stage
constexpr int kWaveSpill = 512;       // pass 1 per-wave spill buffer entries

int64_t list_stride_for(int64_t vocab) { return std::min<int64_t>(vocab, kListMax); }
int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

// Workspace layout: row records, slice records, the tail's row counter, row
// lists. Nothing in it is expected to hold any value when a call starts.
struct WsLayout {
    int64_t rowrec, slrec, queue, lists, total;
};
WsLayout ws_layout(int64_t B, int64_t V) {
    WsLayout w;
    w.rowrec = 0;
    w.slrec = round256(B * qrita::R_WORDS * 4);
    w.queue = w.slrec + round256(B * qrita::kMaxSlices * qrita::S_WORDS * 4);
    w.lists = w.queue + (B > 0 ? 256 : 0);
    w.total = w.lists + B * list_stride_for(V) * 8;
    return w;
}

struct Plan {
    int slices;      // pass 1 workgroups per row
    int slice_len;   // logits per slice
    int stage_cap;   // pass 1 LDS candidate stage
    bool heavy;      // tail tier
    int tail_cap;    // candidates the tail holds in LDS
    int list_cap;    // usable entries of a row list
    int sub_cap;     // list entries per slice
    bool bitmap;     // the tail writes whole mask rows
    int chunks;      // row chunks whose tails overlap the next chunk's streaming pass
    bool one_launch; // no pass-1 launch: the tail streams each row (one slice per row)
};

bool dtype_ok(int d) { return d == QRITA_F32 || d == QRITA_BF16 || d == QRITA_F16; }

// The tier table (the summary's tiered block sizes, "Autotuning": large blocks
// for full rows, small ones for truncated sets), a static function of the
// call's shape (B rows, V logits of `esize` bytes, idx_cap for the expected
// top-k range):
//  - pass 1: 256-thread workgroups, at least 1024 of them (all resident
//    together on 256 CUs); from 512 rows on, long rows get up to eight slices
//    of about 64 KiB (256 KiB from 2048 rows on) so several rounds of
//    workgroups balance the CUs; slices of at least 8192 logits;
//  - tail: the light tier (two rows per CU) for batches of 256 rows or more
//    whose index output is at most 4096 ranks, else the heavy tier (one row
//    per CU, twice the LDS capacities, kept sets up to 8192 sorted at once);
//  - from 512 rows on, the mask is written by the tail from an LDS bitmap
//    whenever the row fits the tier's bitmap, so pass 1 only reads (with
//    fewer rows, the whole-row writes would fall on too few CUs: pass 1
//    zero-fills the mask at streaming bandwidth and the tail stores the kept
//    bytes).
Plan choose_plan(int64_t B, int64_t V, int64_t esize, int64_t idx_cap, const qrita_options* o) {
    Plan t;
    int64_t S = std::max<int64_t>(1, (1024 + B - 1) / B);
    // many rows: slices of about 64 KiB (512-2047 rows) or 256 KiB (2048
    // rows and more; there every CU already holds several rows' slices, and
    // each slice's threshold set-up is better spread over more logits)
    const int64_t slice_bytes = B >= 2048 ? 262144 : 65536;
    if (B >= 512) S = std::max<int64_t>(S, std::min<int64_t>(8, (V * esize + slice_bytes - 1) / slice_bytes));
    S = std::min<int64_t>(S, qrita::kMaxSlices);
    S = std::min<int64_t>(S, std::max<int64_t>(1, (V + 8191) / 8192));
    if (o && o->slices > 0) S = std::min<int64_t>(std::min<int64_t>(o->slices, qrita::kMaxSlices), std::max<int64_t>(1, V));
    // on request, one launch: each row's tail workgroup streams its whole
    // row (measured slower than two launches at every shape: ablation leg)
    t.one_launch = o && o->launches == 1;
    if (t.one_launch) S = 1;
    // slices are whole tiles of 16 logits per thread (only a row's last slice
    // ends in a part tile), and after the first they start 16-aligned
    const int64_t TB = (int64_t)kPass1Threads * 16;
    int64_t L = (V + S - 1) / S;
    L = ((L + TB - 1) / TB) * TB;
    if (o && o->slices > 0 && !t.one_launch) L = ((((V + S - 1) / S) + 15) / 16) * 16;
    S = (V + L - 1) / L;
    t.slices = (int)S;
    t.slice_len = (int)L;
    int stage = kStageCap;
    if (o && o->lds_cap > 0) stage = std::max(64, std::min(stage, (int)o->lds_cap));
    t.stage_cap = stage;
    t.heavy = B < 256 || idx_cap > 4096;
    // index-ordered output needs the row's bitmap in LDS
    if (o && o->idx_order && V + 64 > (int64_t)qrita::tier_light().bitmap_bits) t.heavy = true;
    if (o && o->tier == 1) t.heavy = false;
    if (o && o->tier == 2) t.heavy = true;
    const qrita::TierInfo ti = t.heavy ? qrita::tier_heavy() : qrita::tier_light();
    int tail = ti.cfull;
    if (o && o->lds_cap > 0) tail = std::max(64, std::min(tail, (int)o->lds_cap));
    t.tail_cap = tail;
    int64_t lc = list_stride_for(V);
    if (o && o->list_cap > 0) lc = std::max<int64_t>(1, std::min<int64_t>(lc, o->list_cap));
    t.list_cap = (int)lc;
    t.sub_cap = (int)std::max<int64_t>(1, lc / S);
    t.bitmap = B >= 512 && (uint64_t)V <= (uint64_t)ti.bitmap_bits && !(o && o->mask_mode == 1);
    // on request, the batch is cut into chunks of whole multiples of 8 rows
    // (the XCD dealing of rows): the tail of chunk c runs on a second stream
    // while the streaming pass reads chunk c + 1
    int ch = 1;  // measured: overlapping on two streams was slower at every shape (ablation leg)
    if (o && o->chunks > 0) ch = o->chunks;
    ch = (int)std::min<int64_t>(ch, std::max<int64_t>(1, B / 8));
    t.chunks = t.one_launch ? 1 : std::min(ch, kMaxChunks);
    return t;
}

// gfx950 check, once per device (kernels built for gfx950 cannot run elsewhere).
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cus[kMaxDevices];   // compute units (published before g_arch)

bool device_supported() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
    if (dev >= kMaxDevices) return false;
    int s = g_arch[dev].load(std::memory_order_acquire);
    if (s == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
        s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        g_arch[dev].store(s, std::memory_order_release);
    }
    return s == 1;
}

// The second stream of chunked calls, per device: created once (default
// priority, non-blocking), with a pool of ordering events. The launch
// sequence of a chunked call holds the device's mutex, so concurrent calls
// never interleave their uses of the events.
struct SideStream {
    std::mutex mu;
    std::once_flag once;
    hipStream_t stream = nullptr;
    hipEvent_t ev[kMaxChunks + 1] = {};
    bool ok = false;
};
SideStream g_side[kMaxDevices];

SideStream* side_for(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    SideStream& sd = g_side[dev];
    std::call_once(sd.once, [&sd] {
        bool ok = hipStreamCreateWithFlags(&sd.stream, hipStreamNonBlocking) == hipSuccess;
        for (int i = 0; ok && i <= kMaxChunks; ++i)
            ok = hipEventCreateWithFlags(&sd.ev[i], hipEventDisableTiming) == hipSuccess;
        sd.ok = ok;
    });
    return sd.ok ? &sd : nullptr;
}

// The draw of a sampling call (null for a selection).
struct Draw {
    int32_t* token;
    float* prob;
    uint64_t seed, offset;
};

bool options_valid(const qrita_options* opt) {
    return !opt || !(((uintptr_t)opt->diag & 3u) || opt->pivot_mode < 0 || opt->pivot_mode > 2 ||
                     opt->slices < 0 || opt->lds_cap < 0 || opt->list_cap < 0 || opt->tier < 0 ||
                     opt->tier > 2 || opt->mask_mode < 0 || opt->mask_mode > 1 || opt->idx_order < 0 ||
                     opt->idx_order > 1 || opt->chunks < 0 || opt->chunks > kMaxChunks ||
                     opt->pivot_search_only < 0 || opt->pivot_search_only > 1 || opt->launches < 0 ||
                     opt->launches > 2 ||
                     !(opt->delta_scale == opt->delta_scale));
}

// The params of rows [r0, r0 + n) of a call as a batch of its own.
Params rows_of(const Params& P, int64_t r0, int64_t n) {
    Params c = P;
    const int64_t V = P.vocab, es = P.dtype == 0 ? 4 : 2;
    c.logits = (const char*)P.logits + r0 * V * es;
    if (P.mask) c.mask = P.mask + r0 * V;
    if (P.out_idx) c.out_idx = P.out_idx + r0 * (int64_t)P.idx_cap;
    if (P.out_count) c.out_count = P.out_count + r0;
    if (P.k) c.k = P.k + r0;
    if (P.p) c.p = P.p + r0;
    if (P.diag) c.diag = P.diag + r0 * 8;
    if (P.out_token) c.out_token = P.out_token + r0;
    if (P.out_prob) c.out_prob = P.out_prob + r0 * (int64_t)P.idx_cap;
    c.rowrec = P.rowrec + r0 * qrita::R_WORDS;
    c.slrec = P.slrec + r0 * qrita::kMaxSlices * qrita::S_WORDS;
    c.glist = P.glist + r0 * (int64_t)P.list_stride;
    c.batch = n;
    c.row0 = P.row0 + r0;
    return c;
}

int select_impl(const void* logits, int64_t batch, int64_t vocab, int dtype, const int32_t* k,
                const float* p, uint8_t* out_mask, int32_t* out_idx, int32_t* out_count,
                int64_t idx_cap, void* workspace, size_t workspace_bytes, void* stream,
                const qrita_options* opt, const Draw* draw = nullptr, bool one_stream = false) {
    if (!logits || batch < 0 || vocab <= 0 || vocab > INT32_MAX || idx_cap < 0 ||
        idx_cap > INT32_MAX)
        return QRITA_EINVAL;
    if (!dtype_ok(dtype)) return QRITA_EINVAL;
    if (out_idx && !out_count) return QRITA_EINVAL;
    if (!out_mask && !out_idx && !out_count && !draw) return QRITA_EINVAL;
    if (draw && (!draw->token || ((uintptr_t)draw->token & 3u) || ((uintptr_t)draw->prob & 3u) ||
                 (draw->prob && !out_idx)))
        return QRITA_EINVAL;
    if (((uintptr_t)logits & 15u) || ((uintptr_t)out_mask & 15u)) return QRITA_EINVAL;
    if (((uintptr_t)k & 3u) || ((uintptr_t)p & 3u) || ((uintptr_t)out_idx & 3u) ||
        ((uintptr_t)out_count & 3u))
        return QRITA_EINVAL;
    if (batch > (int64_t)(INT32_MAX / 64)) return QRITA_EINVAL;
    if (batch == 0) return QRITA_OK;
    const size_t need = qrita_workspace_bytes(batch, vocab, dtype, idx_cap);
    if (!workspace || workspace_bytes < need) return QRITA_EWORKSPACE;
    if ((uintptr_t)workspace & 255u) return QRITA_EWORKSPACE;
    const int64_t esize = dtype == QRITA_F32 ? 4 : 2;
    const Plan t = choose_plan(batch, vocab, esize, out_idx ? idx_cap : 0, opt);
    if (opt && opt->idx_order) {
        const qrita::TierInfo ti = t.heavy ? qrita::tier_heavy() : qrita::tier_light();
        if (vocab + 64 > (int64_t)ti.bitmap_bits) return QRITA_EINVAL;
    }
    if (!device_supported()) return QRITA_EUNSUPPORTED;

    const WsLayout w = ws_layout(batch, vocab);
    Params P;
    std::memset(&P, 0, sizeof P);
    P.logits = logits;
    P.mask = out_mask;
    P.out_idx = out_idx;
    P.out_count = out_count;
    P.k = k;
    P.p = p;
    P.rowrec = (uint32_t*)((char*)workspace + w.rowrec);
    P.slrec = (uint32_t*)((char*)workspace + w.slrec);
    P.glist = (uint64_t*)((char*)workspace + w.lists);
    P.queue = nullptr;
    P.fused = t.one_launch ? 1 : 0;
    P.diag = opt ? opt->diag : nullptr;
    P.batch = batch;
    P.vocab = (int32_t)vocab;
    P.idx_cap = out_idx ? (int32_t)idx_cap : 0;
    P.slices = t.slices;
    P.slice_len = t.slice_len;
    P.stage_cap = t.stage_cap;
    P.sub_cap = t.sub_cap;
    P.list_cap = t.list_cap;
    P.list_stride = (int32_t)list_stride_for(vocab);
    P.tail_cap = t.tail_cap;
    P.force_miss = opt ? opt->force_miss : 0;
    P.delta_scale = (opt && opt->delta_scale != 0.0f) ? opt->delta_scale : 1.0f;
    P.pivot_mode = opt ? opt->pivot_mode : 0;
    P.bitmap = t.bitmap ? 1 : 0;
    P.dtype = dtype;
    // rows with at most kSmallSet candidates are sorted outright and scanned
    // (unless the options ask for the pivot searches on every row)
    P.small_max = (opt && opt->pivot_search_only)
                      ? 0
                      : std::min(kSmallSet, (t.heavy ? qrita::tier_heavy().csort : qrita::tier_light().csort) / 2);
    P.idx_order = (opt && opt->idx_order) ? 1 : 0;
    if (draw) {
        P.out_token = draw->token;
        P.out_prob = draw->prob;
        P.seed = draw->seed;
        P.offset = draw->offset;
    }

    hipStream_t s = (hipStream_t)stream;
    const size_t lds = ((size_t)std::max(t.stage_cap, kSampleN) + (size_t)(kPass1Threads / 64) * kWaveSpill) * 8;
    auto pass1 = [&](const Params& Q, hipStream_t st) {
        const unsigned groups = (unsigned)(((Q.batch + 7) / 8) * 8 * (int64_t)t.slices);
        return qrita::launch_pass1(Q, groups, lds, st);
    };
    auto tail = [&](const Params& Q, hipStream_t st) {
        return t.heavy ? qrita::launch_tail_heavy(Q, st) : qrita::launch_tail_light(Q, st);
    };
    SideStream* sd = nullptr;
    if (t.chunks > 1 && !one_stream) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return QRITA_ELAUNCH;
        sd = side_for(dev);  // no second stream: one chunk
    }
    if (!sd && t.one_launch) {
        if (opt && opt->mid_event) {  // no streaming pass: the whole call is the tail
            if (hipEventRecord((hipEvent_t)opt->mid_event, s) != hipSuccess) return QRITA_ELAUNCH;
        }
        return tail(P, s) == hipSuccess ? QRITA_OK : QRITA_ELAUNCH;
    }
    if (!sd) {
        // rows for more than one and at most two rounds of the tail
        // workgroups resident at once: each tail workgroup takes the next row
        // from a counter when it starts. (With more rounds, the counter's
        // round trip at every start costs more than the balance gains.)
        {
            int dev = 0;
            if (hipGetDevice(&dev) != hipSuccess) return QRITA_ELAUNCH;
            const qrita::TierInfo ti = t.heavy ? qrita::tier_heavy() : qrita::tier_light();
            const int64_t per_cu = std::max<int64_t>(1, (int64_t)(160 * 1024) / (int64_t)(ti.lds + 4096));
            const int64_t resident = per_cu * std::max(1, g_cus[dev].load(std::memory_order_relaxed));
            if (batch > resident && batch <= 2 * resident) P.queue = (uint32_t*)((char*)workspace + w.queue);
        }
        if (pass1(P, s) != hipSuccess) return QRITA_ELAUNCH;
        if (opt && opt->mid_event) {
            if (hipEventRecord((hipEvent_t)opt->mid_event, s) != hipSuccess) return QRITA_ELAUNCH;
        }
        return tail(P, s) == hipSuccess ? QRITA_OK : QRITA_ELAUNCH;
    }
    // chunk c: pass 1 on the caller's stream, then its tail on the side
    // stream once that pass is done, while pass 1 of chunk c + 1 runs; the
    // caller's stream finally waits for the last tail
    std::lock_guard<std::mutex> lock(sd->mu);
    const int C = t.chunks;
    const int64_t per = (batch + C - 1) / C;
    const int64_t step = (per + 7) / 8 * 8;
    int used = 0;
    for (int64_t r0 = 0; r0 < batch; r0 += step, ++used) {
        const Params Q = rows_of(P, r0, std::min(step, batch - r0));
        if (pass1(Q, s) != hipSuccess) return QRITA_ELAUNCH;
        if (hipEventRecord(sd->ev[used], s) != hipSuccess) return QRITA_ELAUNCH;
        if (hipStreamWaitEvent(sd->stream, sd->ev[used], 0) != hipSuccess) return QRITA_ELAUNCH;
        if (tail(Q, sd->stream) != hipSuccess) return QRITA_ELAUNCH;
    }
    if (opt && opt->mid_event) {  // after the last streaming pass
        if (hipEventRecord((hipEvent_t)opt->mid_event, s) != hipSuccess) return QRITA_ELAUNCH;
    }
    if (hipEventRecord(sd->ev[kMaxChunks], sd->stream) != hipSuccess) return QRITA_ELAUNCH;
    if (hipStreamWaitEvent(s, sd->ev[kMaxChunks], 0) != hipSuccess) return QRITA_ELAUNCH;
    return QRITA_OK;
}

// Static device scratch for qrita_select_noalloc: the workspace of callers
// that cannot allocate. Every GPU the library runs on holds its own copy
// until the process ends; its contents never matter to a call (every word a
// call reads is written earlier in the same call).
static __device__ __align__(256) unsigned char scratch[QRITA_NOALLOC_SCRATCH_BYTES];

// The array's device address, looked up once per device with that device
// current (in host code the array's name is only a host-side stand-in).
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

int scratch_for_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QRITA_EUNSUPPORTED;
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return QRITA_ELAUNCH;
    *out = g_scratch_ptr[dev];
    return QRITA_OK;
}

}  // namespace

extern "C" {

int qrita_select_noalloc(const void* logits, int64_t batch, int64_t vocab, int dtype, const int32_t* k,
                         const float* p, uint8_t* out_mask, int32_t* out_idx, int32_t* out_count,
                         int64_t idx_cap, void* stream) {
    // shape and argument checks first (nothing touches the GPU before them)
    if (!logits || batch < 0 || vocab <= 0 || vocab > INT32_MAX || idx_cap < 0 || idx_cap > INT32_MAX)
        return QRITA_EINVAL;
    if (!dtype_ok(dtype)) return QRITA_EINVAL;
    if (batch == 0) return QRITA_OK;
    if (qrita_workspace_bytes(batch, vocab, dtype, idx_cap) > (size_t)QRITA_NOALLOC_SCRATCH_BYTES)
        return QRITA_ESCRATCH;
    if (!out_mask && !out_idx && !out_count) return QRITA_EINVAL;
    if (out_idx && !out_count) return QRITA_EINVAL;
    if (!device_supported()) return QRITA_EUNSUPPORTED;
    void* ws = nullptr;
    const int st = scratch_for_current_device(&ws);
    if (st != QRITA_OK) return st;
    return select_impl(logits, batch, vocab, dtype, k, p, out_mask, out_idx, out_count, idx_cap, ws,
                       (size_t)QRITA_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr, true);
}

size_t qrita_workspace_bytes(int64_t batch, int64_t vocab, int dtype, int64_t idx_cap) {
    (void)idx_cap;
    if (batch < 0 || vocab <= 0 || vocab > INT32_MAX) return 0;
    if (!dtype_ok(dtype)) return 0;
    return (size_t)ws_layout(batch, vocab).total;
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
    if (!options_valid(opt)) return QRITA_EINVAL;
    return select_impl(logits, batch, vocab, dtype, k, p, out_mask, out_idx, out_count, idx_cap,
                       workspace, workspace_bytes, stream, opt);
}

int qrita_sample(const void* logits, int64_t batch, int64_t vocab, int dtype, const int32_t* k,
                 const float* p, uint64_t seed, uint64_t offset, int32_t* out_token, float* out_prob,
                 uint8_t* out_mask, int32_t* out_idx, int32_t* out_count, int64_t idx_cap,
                 void* workspace, size_t workspace_bytes, void* stream, const qrita_options* opt) {
    if (!options_valid(opt)) return QRITA_EINVAL;
    const Draw d{out_token, out_prob, seed, offset};
    return select_impl(logits, batch, vocab, dtype, k, p, out_mask, out_idx, out_count, idx_cap,
                       workspace, workspace_bytes, stream, opt, &d);
}

void qrita_philox4x64_10(const uint64_t counter[4], const uint64_t key[2], uint64_t out[4]) {
    qrita::philox4x64_10(counter, key, out);
}

double qrita_uniform(uint64_t seed, uint64_t offset, uint64_t row) {
    return qrita::row_uniform(seed, offset, row);
}

const char* qrita_strerror(int status) {
    switch (status) {
        case QRITA_OK: return "success";
        case QRITA_EINVAL: return "invalid argument";
        case QRITA_EWORKSPACE: return "workspace missing, misaligned or too small";
        case QRITA_ELAUNCH: return "kernel launch failed";
        case QRITA_EUNSUPPORTED: return "unsupported device (the library is built for gfx950)";
        case QRITA_ESCRATCH: return "problem larger than the static scratch of qrita_select_noalloc";
        default: return "unknown status";
    }
}

}  // extern "C"
