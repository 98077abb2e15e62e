// Kernel launchers shared by the host code and the kernel translation units
// (each kernel family is compiled on its own so the build runs in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include "params.hpp"

namespace qrita {

// pass 1 over `groups` workgroups of 256 threads with `lds` bytes of dynamic LDS
hipError_t launch_pass1(const Params& P, unsigned groups, size_t lds, hipStream_t stream);
// the tail, one workgroup per row, light tier (two workgroups per CU)
hipError_t launch_tail_light(const Params& P, hipStream_t stream);
// the tail, heavy tier (one workgroup per CU, twice the capacities)
hipError_t launch_tail_heavy(const Params& P, hipStream_t stream);

// capacities of the tail tiers (host view of the kernels' constants)
struct TierInfo {
    int cfull;          // candidates held in LDS
    int csort;          // largest set sorted in one piece
    unsigned bitmap_bits;  // largest vocabulary whose mask row is written from LDS
    size_t lds;         // dynamic LDS bytes
};
TierInfo tier_light();
TierInfo tier_heavy();

}  // namespace qrita
