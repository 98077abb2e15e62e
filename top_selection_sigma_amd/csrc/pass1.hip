// Translation unit of the streaming pass (pass1_kernel for the three dtypes).
#include <mutex>

#include "launch.hpp"
#include "select_kernel.hpp"

namespace qrita {

namespace {
// Dynamic LDS above 64 KiB must be enabled per kernel.
template <int DT>
hipError_t allow_lds() {
    static std::once_flag once;
    static hipError_t err = hipSuccess;
    std::call_once(once, [] {
        err = hipFuncSetAttribute((const void*)pass1_kernel<256, DT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  96 * 1024);
    });
    return err;
}
}  // namespace

hipError_t launch_pass1(const Params& P, unsigned groups, size_t lds, hipStream_t stream) {
    const hipError_t a = P.dtype == 1 ? allow_lds<1>() : (P.dtype == 2 ? allow_lds<2>() : allow_lds<0>());
    if (a != hipSuccess) return a;
    auto kern = P.dtype == 1 ? pass1_kernel<256, 1> : (P.dtype == 2 ? pass1_kernel<256, 2> : pass1_kernel<256, 0>);
    hipLaunchKernelGGL(kern, dim3(groups), dim3(256), lds, stream, P);
    return hipGetLastError();
}

}  // namespace qrita
