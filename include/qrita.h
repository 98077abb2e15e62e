/*
 * qrita.h - exact, deterministic top-k / top-p candidate-set selection over
 * large-vocabulary logits on AMD MI355X (gfx950).
 *
 * The operation is the one the Qrita summary (gist.science paper 2602.01518,
 * Spanish and Korean pages) describes for an LLM sampler: for every row of
 * logits, return the full top-k / top-p candidate set with the exact
 * semantics of sort-based top-k and top-p ("Declaración del Problema";
 * "Contribuciones Clave" 1 and 4), computed by Gaussian sigma-truncation
 * ("Metodología" §1), a quaternary pivot search with duplicate tracking
 * (§2) and a duplicate-handling mask ("Detalles de Implementación",
 * Pipeline).
 *
 * Semantics per row b (V = vocab):
 *   - Order: value descending; equal values (including -0.0 == +0.0 and
 *     -inf == -inf) by ascending vocabulary index. This is the order a stable
 *     descending sort produces, and it fixes which boundary duplicates are
 *     kept (the pages require a deterministic count, §2).
 *   - Top-k: K = k[b] if 0 < k[b] < V, otherwise top-k is off (K = V).
 *     Exactly K tokens are kept (§2: exactly k elements at or above the
 *     pivot).
 *   - Top-p: on iff p[b] < 1 (NaN means off). p[b] <= 0 keeps one token.
 *     Otherwise the kept set is the shortest rank prefix of the top-k set
 *     whose softmax mass, renormalised over the top-k set, is >= p[b].
 *     Masses are formed in float64 fixed point on the GPU; on rows whose
 *     cumulative mass at the cut lies within 1e-5 of p the cut may differ from
 *     an exact float64 computation by the ranks inside that band.
 *   - An all -inf row keeps one token when top-p is on.
 *   Logits must be finite or -inf; NaN and +inf give unspecified (but
 *   memory-safe) output.
 *
 * All pointers are device pointers owned by the caller. Calls are
 * asynchronous on `stream` (a hipStream_t; NULL is the default stream),
 * allocate nothing, do not synchronise, and launch two kernels in stream
 * order: the single streaming pass over the logits and a per-row tail.
 * Argument errors are reported before anything is launched or written.
 * The library keeps no state between calls: calls on different streams are
 * safe as long as each in-flight call has a workspace of its own.
 */
#ifndef QRITA_H
#define QRITA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the logits. */
typedef enum {
    QRITA_F32 = 0,  /* IEEE float32 */
    QRITA_BF16 = 1, /* bfloat16 (upper half of a float32) */
    QRITA_F16 = 2   /* IEEE binary16 */
} qrita_dtype_t;

/* Return codes. */
typedef enum {
    QRITA_OK = 0,
    QRITA_EINVAL = 1,      /* bad argument: nothing launched, nothing written */
    QRITA_EWORKSPACE = 2,  /* workspace NULL or smaller than qrita_workspace_bytes() */
    QRITA_ELAUNCH = 3,     /* the HIP runtime reported an error at launch */
    QRITA_EUNSUPPORTED = 4, /* the current device cannot run this library */
    QRITA_ESCRATCH = 5     /* qrita_select_noalloc: the shape needs more than its static scratch */
} qrita_status_t;

/*
 * Bytes of device workspace qrita_select needs for this shape. The workspace
 * holds a 32-byte record per row, a 16-byte record per (row, slice of the
 * streaming pass) and a per-row candidate list (at most min(vocab, 32768)
 * entries of 8 bytes): O(batch) memory, against the O(batch * vocab)
 * value+index buffers a full sort needs (the summary reports about 50 % lower
 * memory than sort-based selection, "Resultados").
 * Every word a call reads from the workspace is written earlier in the same
 * call: the workspace needs no initialisation and may hold anything when a
 * call starts. Two calls sharing one workspace must not overlap in time.
 * Returns 0 for an invalid shape.
 */
size_t qrita_workspace_bytes(int64_t batch, int64_t vocab, int dtype, int64_t idx_cap);

/*
 * Select the top-k / top-p candidate set of every row.
 *
 * logits     device, [batch][vocab] contiguous rows of `dtype`; 16-byte aligned.
 * batch      rows (>= 0; 0 is a no-op).
 * vocab      logits per row, 1 .. 2^31 - 1.
 * dtype      QRITA_F32, QRITA_BF16 or QRITA_F16 (16-bit types are widened to
 *            float32 exactly; order and ties are those of the logits).
 * k          device int32 [batch], or NULL (top-k off for all rows).
 * p          device float32 [batch], or NULL (top-p off for all rows).
 * out_mask   device uint8 [batch][vocab]: 1 = kept, 0 = dropped; or NULL.
 *            16-byte aligned.
 * out_idx    device int32 [batch][idx_cap]: the first min(count, idx_cap)
 *            kept indices in rank order (value descending, index ascending);
 *            later entries of each row are left untouched. Or NULL.
 * out_count  device int32 [batch]: number of kept tokens. Required when
 *            out_idx is given; may be NULL otherwise.
 * idx_cap    row stride of out_idx (>= 0).
 * idx_cap    also the expected range of k: above 4096 the per-row tail takes
 *            the tier that sorts up to 8192 kept tokens at once.
 * workspace  device scratch of at least qrita_workspace_bytes(...) bytes,
 *            256-byte aligned; its contents on entry do not matter.
 * stream     hipStream_t to launch on (NULL = default stream).
 *
 * At least one of out_mask, out_idx, out_count must be non-NULL.
 * Returns QRITA_OK, QRITA_EINVAL, QRITA_EWORKSPACE, QRITA_EUNSUPPORTED (the
 * current device is not gfx950; checked after the arguments) or
 * QRITA_ELAUNCH.
 */
int qrita_select(const void* logits, int64_t batch, int64_t vocab, int dtype,
                 const int32_t* k, const float* p,
                 uint8_t* out_mask, int32_t* out_idx, int32_t* out_count, int64_t idx_cap,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Options for qrita_select_ex: ablation and test controls. None of them can
 * change a selection result; they only change how it is reached.
 *   force_miss   nonzero: no truncation survivors, every row takes the
 *                full-row fallback (the summary's truncation miss, §1).
 *   delta_scale  multiplies the table delta (0 means 1).
 *   pivot_mode   0: pivots at 25/50/75 % of the key range (§2);
 *                1: the same fractions of the value range;
 *                2: one pivot at 50 % of the key range (a binary search with
 *                   the same duplicate tracking, for the quaternary-vs-binary
 *                   ablation of "Resultados").
 *   slices       workgroups per row (0 = automatic tier).
 *   lds_cap      candidate capacity in LDS per workgroup (0 = automatic;
 *                otherwise clamped to [64, automatic]).
 *   list_cap     per-row overflow-list capacity (0 = automatic; otherwise
 *                clamped to [1, automatic]).
 *   diag         device int32 [batch][QRITA_DIAG_FIELDS] or NULL: per-row
 *                diagnostics, see QRITA_DIAG_* below.
 *   mid_event    a hipEvent_t or NULL: recorded on the stream between the
 *                streaming pass and the per-row tail, for per-stage timing
 *                (with one launch: before it).
 *   tier         tail tier: 0 automatic, 1 light (two rows per CU),
 *                2 heavy (one row per CU, larger capacities).
 *   mask_mode    0 automatic; 1: pass 1 zero-fills the mask and the tail
 *                stores the kept bytes one by one (instead of the tail
 *                writing whole rows from an LDS bitmap).
 *   idx_order    0: out_idx in rank order; 1: out_idx holds the first
 *                min(count, idx_cap) kept indices in ascending vocabulary
 *                order (the kept set itself is unchanged), for consumers
 *                that gather from the kept set (a restricted vocabulary
 *                of top-K marginals, beam pruning). Needs vocab + 64 <=
 *                688256 (the row's bitmap in LDS); larger vocabularies
 *                return QRITA_EINVAL. With qrita_sample, out_prob follows
 *                the same order.
 *   chunks       0 automatic (one chunk); n in 1..16: the batch is cut into
 *                n row chunks and the per-row tail of chunk c runs on a
 *                second stream of the library (one per device) while the
 *                streaming pass reads chunk c + 1; the caller's stream waits
 *                for the last tail before anything queued after the call.
 *   pivot_search_only  0 automatic: rows whose candidate set has at most 4096
 *                entries (2048 on the light tier) are sorted once and answered
 *                from the rank order;
 *                1: every row takes the pivot searches (for the ablations).
 *   launches     0 automatic (two launches: the streaming pass over
 *                (row, slice) workgroups, then the per-row tail);
 *                1: one launch, in which each row's tail workgroup first
 *                streams its whole row itself (slower at every measured
 *                shape: one workgroup's ALUs bound the pass over a row; for
 *                the ablation); 2: two launches. The outputs are the same
 *                either way.
 */
typedef struct {
    int32_t force_miss;
    float delta_scale;
    int32_t pivot_mode;
    int32_t slices;
    int32_t lds_cap;
    int32_t list_cap;
    int32_t* diag;
    void* mid_event;
    int32_t tier;
    int32_t mask_mode;
    int32_t idx_order;
    int32_t chunks;
    int32_t pivot_search_only;
    int32_t launches;
} qrita_options;

#define QRITA_DIAG_FIELDS 8
#define QRITA_DIAG_T 0          /* Gaussian threshold mu + delta*sigma (float bits) */
#define QRITA_DIAG_TC 1         /* threshold used for collection (float bits) */
#define QRITA_DIAG_NT 2         /* #{z >= Gaussian threshold}, or -1 if unknown */
#define QRITA_DIAG_NCAND 3      /* candidates collected in the single pass */
#define QRITA_DIAG_PATH 4       /* 0 LDS, 1 overflow list, 2 list after re-collection, 3 full row */
#define QRITA_DIAG_HIT 5        /* 1 if the Gaussian threshold alone was a truncation hit */
#define QRITA_DIAG_ITERS 6      /* pivot-search iterations spent on the row */
#define QRITA_DIAG_PREDICTED 7  /* 1 if the sample predicted a miss and lowered the threshold */

/* qrita_select with options (opt may be NULL: same as qrita_select). */
int qrita_select_ex(const void* logits, int64_t batch, int64_t vocab, int dtype,
                    const int32_t* k, const float* p,
                    uint8_t* out_mask, int32_t* out_idx, int32_t* out_count, int64_t idx_cap,
                    void* workspace, size_t workspace_bytes, void* stream,
                    const qrita_options* opt);

/*
 * qrita_select for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same selection and outputs as qrita_select, with the workspace taken
 * from a static device array of the library (QRITA_NOALLOC_SCRATCH_BYTES,
 * one per GPU, held until the process ends) instead of a caller's buffer.
 * Shapes whose qrita_workspace_bytes exceeds that size return
 * QRITA_ESCRATCH before anything is launched. The call allocates nothing
 * (no hipMalloc, no allocating library routine); its first call on a device
 * looks up the array's device address once. All calls on one GPU share the
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. The array's contents
 * left by one call never affect the next.
 * Returns the codes of qrita_select, or QRITA_ESCRATCH.
 */
#define QRITA_NOALLOC_SCRATCH_BYTES (32 << 20)
int qrita_select_noalloc(const void* logits, int64_t batch, int64_t vocab, int dtype,
                         const int32_t* k, const float* p,
                         uint8_t* out_mask, int32_t* out_idx, int32_t* out_count, int64_t idx_cap,
                         void* stream);

/*
 * Select, then draw one token per row from the kept set: the sampling step
 * the candidate set exists for (the summary motivates returning the whole
 * top-k / top-p set because an LLM sampler draws from it next, "Declaración
 * del Problema"). The selection and its outputs are those of qrita_select_ex;
 * in addition, per row b with kept set of L tokens in rank order r = 0..L-1:
 *   p_r   = exp(z_r - m) / sum_{s<L} exp(z_s - m)   (m = row maximum),
 *   c_r   = p_0 + ... + p_r,
 *   u     = the row's uniform in [0, 1): the first 64-bit output of
 *           Philox4x64-10 (Salmon et al., SC 2011) at counter
 *           (b, offset, 0, 0) under key (seed, 0), top 53 bits times 2^-53
 *           (qrita_uniform returns it on the host),
 *   token = the index of the smallest rank r with c_r >= u (inverse CDF).
 * An all -inf row draws rank 0. Masses are formed in the same fixed point as
 * the top-p cut: when u lies within 1e-6 of some c_r, the drawn rank may
 * differ from an exact float64 computation by the ranks inside that band.
 * The draw is a function of (logits, k, p, seed, offset, b) only: the same
 * call gives the same tokens on any stream, any batch position is
 * independent of the others, and a new offset gives new draws.
 *
 * out_token  device int32 [batch]: the drawn vocabulary index. Required.
 * out_prob   device float32 [batch][idx_cap] or NULL: p_r beside out_idx for
 *            the ranks out_idx holds (requires out_idx).
 * seed, offset  the Philox key word and counter word above.
 * out_mask, out_idx, out_count, idx_cap, workspace, stream, opt: as for
 *            qrita_select_ex; all three outputs may be NULL here.
 * Returns the codes of qrita_select_ex.
 */
int qrita_sample(const void* logits, int64_t batch, int64_t vocab, int dtype,
                 const int32_t* k, const float* p, uint64_t seed, uint64_t offset,
                 int32_t* out_token, float* out_prob,
                 uint8_t* out_mask, int32_t* out_idx, int32_t* out_count, int64_t idx_cap,
                 void* workspace, size_t workspace_bytes, void* stream,
                 const qrita_options* opt);

/*
 * Philox4x64-10 on the host (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011): out = the ten-round bijection of
 * the 256-bit counter under the 128-bit key. The same routine the device
 * draw runs; exported so that callers and tests can reproduce the draws.
 * Host pointers; no GPU involved.
 */
void qrita_philox4x64_10(const uint64_t counter[4], const uint64_t key[2], uint64_t out[4]);

/* The uniform qrita_sample draws for row `row` under (seed, offset); host only. */
double qrita_uniform(uint64_t seed, uint64_t offset, uint64_t row);

/* Static description of a status code. */
const char* qrita_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* QRITA_H */
