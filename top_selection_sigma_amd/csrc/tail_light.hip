// Translation unit of the tail kernel, light tier.
#include <mutex>

#include "launch.hpp"
#include "select_kernel.hpp"

namespace qrita {

TierInfo tier_light() {
    return TierInfo{TierLight::CFULL, TierLight::CSORT, TierLight::BITMAP_BITS, TierLight::LDS};
}

hipError_t launch_tail_light(const Params& P, hipStream_t stream) {
    static std::once_flag once;
    static hipError_t err = hipSuccess;
    std::call_once(once, [] {
        err = hipFuncSetAttribute((const void*)tail_kernel<TierLight>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)TierLight::LDS);
    });
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(tail_kernel<TierLight>, dim3((unsigned)P.batch), dim3(TierLight::NT), TierLight::LDS, stream, P);
    return hipGetLastError();
}

}  // namespace qrita
