// Translation unit of the streaming pass (pass1_kernel for both dtypes).
#include <mutex>

#include "launch.hpp"
#include "select_kernel.hpp"

namespace qrita {

namespace {
// Dynamic LDS above 64 KiB must be enabled per kernel.
template <bool BF16>
hipError_t allow_lds() {
    static std::once_flag once;
    static hipError_t err = hipSuccess;
    std::call_once(once, [] {
        err = hipFuncSetAttribute((const void*)pass1_kernel<256, BF16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  96 * 1024);
    });
    return err;
}
}  // namespace

hipError_t launch_pass1(const Params& P, unsigned groups, size_t lds, bool bf16, hipStream_t stream) {
    const hipError_t a = bf16 ? allow_lds<true>() : allow_lds<false>();
    if (a != hipSuccess) return a;
    auto kern = bf16 ? pass1_kernel<256, true> : pass1_kernel<256, false>;
    hipLaunchKernelGGL(kern, dim3(groups), dim3(256), lds, stream, P);
    return hipGetLastError();
}

}  // namespace qrita
