// Kernel parameters and the records pass 1 leaves for the tail.
#pragma once

#include <stdint.h>

namespace qrita {

struct Params {
    const void* logits;
    uint8_t* mask;
    int32_t* out_idx;
    int32_t* out_count;
    const int32_t* k;
    const float* p;
    uint32_t* rowrec;   // [batch][R_WORDS] per-row record, written by slice 0
    uint32_t* slrec;    // [batch][kMaxSlices][S_WORDS] per-slice records
    uint64_t* glist;    // [batch][list_stride] per-row candidate list (slice s owns
                        // entries [s * sub_cap, (s + 1) * sub_cap))
    int32_t* diag;      // [batch][8] or null
    int64_t batch;
    int32_t vocab;
    int32_t idx_cap;
    int32_t slices;
    int32_t slice_len;   // logits per slice (multiple of 16)
    int32_t stage_cap;   // pass 1: candidate capacity of the LDS stage (entries)
    int32_t sub_cap;     // list entries owned by one slice
    int32_t list_cap;    // usable entries of the per-row list (re-collection)
    int32_t list_stride;
    int32_t tail_cap;    // tail: most candidates held in LDS
    int32_t force_miss;
    float delta_scale;
    int32_t pivot_mode;  // 0 key quartiles, 1 value quartiles, 2 one pivot at the key midpoint
    int32_t bitmap;      // 1: the tail writes whole mask rows; pass 1 leaves the mask alone
    int32_t dtype;  // 0 float32, 1 bfloat16, 2 float16
    int32_t idx_order;  // out_idx in ascending vocabulary index instead of rank order
    int32_t* out_token;  // sampling: [batch] drawn token, or null (no draw)
    float* out_prob;     // sampling: [batch][idx_cap] probabilities beside out_idx, or null
    uint64_t seed;       // sampling: Philox key
    uint64_t offset;     // sampling: Philox counter word 1
    int64_t row0;        // batch row of this launch's row 0 (the draw's counter uses batch rows)
    int32_t small_max;   // rows with at most this many candidates take the sort-and-scan path (0: none)
    uint32_t* queue;     // tail row counter (null: workgroup g takes row g)
    int32_t fused;       // 1: one launch, the tail streams each row itself (pass 1 with one slice)
};

// Records that pass 1 leaves for the tail. Every word is written by plain
// stores in the call that reads it (the tail's row counter is zeroed by pass
// 1 and then counted up by the tail), so the workspace carries no state from
// one call to the next (no word is expected to start at zero).
enum : int {
    R_T = 0,       // row record: Gaussian threshold (float bits)
    R_TC = 1,      // collection threshold (float bits)
    R_PRED = 2,    // 1 if a miss was predicted
    R_LAMBDA = 3,  // expected sample count above the K-th value (float bits)
    R_NS = 4,      // sample size
    R_WORDS = 8,
    S_CNT = 0,     // slice record: candidates the slice found (more than sub_cap: overflow)
    S_KMAX = 1,    // largest candidate key of the slice
    S_REST = 2,    // two words: fixed-point mass of the slice's dropped logits (top-p rows)
    S_WORDS = 4
};
constexpr int kMaxSlices = 64;

}  // namespace qrita
