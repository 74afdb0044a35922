// Stand-ins for the kernel launchers (dqg_kernels.hip), for a host-only
// build of the C-ABI layer (dqg_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  The driver only makes calls that validation
// must reject, so any call that reaches a launcher is counted as a failure.
#include "../../dequant_gemv_expert_amd/csrc/dqg_internal.h"

namespace dqg {

int g_stub_launches = 0;

hipError_t launch_matmul(int, const MatDev &, const float *, int, float *, hipStream_t) {
    ++g_stub_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_gate_up(int, const MatDev &, const MatDev &, const float *, int, float *, float, hipStream_t) {
    ++g_stub_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_dequant(int, const MatDev &, float *, hipStream_t) {
    ++g_stub_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_route(const RouteArgs &, hipStream_t) {
    ++g_stub_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_group(int, int, const GroupArgs &, hipStream_t, int *) {
    ++g_stub_launches;
    return hipErrorInvalidValue;
}
hipError_t launch_read(const void *, uint64_t, uint32_t *, int, hipStream_t) {
    ++g_stub_launches;
    return hipErrorInvalidValue;
}
hipError_t static_scratch(void **ptr) {
    ++g_stub_launches;
    *ptr = nullptr;
    return hipErrorNoDevice;
}

}  // namespace dqg
