// Translation unit of the tail kernel, heavy tier.
#include <mutex>

#include "launch.hpp"
#include "select_kernel.hpp"

namespace qrita {

TierInfo tier_heavy() {
    return TierInfo{TierHeavy::CFULL, TierHeavy::CSORT, TierHeavy::BITMAP_BITS, TierHeavy::LDS};
}

hipError_t launch_tail_heavy(const Params& P, hipStream_t stream) {
    static std::once_flag once;
    static hipError_t err = hipSuccess;
    std::call_once(once, [] {
        err = hipFuncSetAttribute((const void*)tail_kernel<TierHeavy>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)TierHeavy::LDS);
    });
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(tail_kernel<TierHeavy>, dim3((unsigned)P.batch), dim3(TierHeavy::NT), TierHeavy::LDS, stream, P);
    return hipGetLastError();
}

}  // namespace qrita
