// Kernel launchers for the host-check build of the library: plan.cpp and
// api.cpp compiled as plain C++ under AddressSanitizer and
// UndefinedBehaviorSanitizer, with no device code linked in. Every launcher
// (and the scratch lookup of the no-allocation entry point) reports that no
// kernel is available, so an entry point whose validation passes returns
// JFA_ERR_HIP instead of reaching a GPU. Tests of the planner and of the
// entry points' argument checks run against this build on the CPU.
#include <hip/hip_runtime_api.h>

#include "internal.h"

namespace jfa {
namespace {
constexpr int32_t kNoKernel = (int32_t)hipErrorNoBinaryForGpu;
}

int32_t launch_fwd(const FwdArgs&, int32_t, Mode, bool, void*) { return kNoKernel; }
int32_t launch_fwd_mx(const FwdArgs&, Mode, bool, void*) { return kNoKernel; }
int32_t launch_bwd(const BwdArgs&, int32_t, Mode, bool, int32_t, void*) { return kNoKernel; }
int32_t launch_dq(const DqArgs&, int32_t, Mode, bool, bool, void*) { return kNoKernel; }
int32_t launch_dq_reduce(const DqReduceArgs&, int32_t, void*) { return kNoKernel; }
int32_t launch_dq_zero(float*, int64_t, void*) { return kNoKernel; }
int32_t launch_dq_convert(const float*, uint16_t*, int64_t, void*) { return kNoKernel; }
int32_t launch_dq_mx(const DqArgs&, Mode, bool, void*) { return kNoKernel; }
int32_t launch_dkdv_mx(const BwdArgs&, Mode, bool, void*) { return kNoKernel; }
int32_t launch_mx_quant_rows(const uint16_t*, int64_t, int32_t, int32_t, uint8_t*, uint8_t*, void*) {
    return kNoKernel;
}
int32_t launch_mx_quant_v(const uint16_t*, const int32_t*, const int32_t*, int32_t, int32_t, int32_t,
                          int32_t, uint8_t*, uint8_t*, void*) {
    return kNoKernel;
}
int32_t noalloc_scratch(void**) { return kNoKernel; }

}  // namespace jfa
