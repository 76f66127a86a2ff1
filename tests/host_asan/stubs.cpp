// Host-only stand-ins for the kernel launchers and workspace sizes that kda_api.cpp calls, so that
// the argument checks of the C ABI can be built with AddressSanitizer and UBSan by g++ (no device
// code, no GPU). Every launcher reports hipErrorNotSupported; the checked calls never reach them.
#include "kda_internal.h"
namespace kda {
bool fused_supported(const LaunchArgs&) { return true; }
hipError_t launch_backward(const BwdArgs&, void*, TimingHook*) { return hipErrorNotSupported; }
hipError_t noalloc_scratch(void**) { return hipErrorNotSupported; }
hipError_t launch_forward_wy(const LaunchArgs&, void*, TimingHook*) { return hipErrorNotSupported; }
hipError_t launch_short_conv(const ConvArgs&, void*, TimingHook*) { return hipErrorNotSupported; }
hipError_t launch_forward_seq(const LaunchArgs&) { return hipErrorNotSupported; }
size_t wy_workspace_bytes(int64_t, int32_t, int32_t, int, int) { return 4096; }
size_t bwd_workspace_bytes(int64_t, int32_t, int32_t, int, int) { return 4096; }
size_t conv_workspace_bytes(int32_t) { return 4096; }
hipError_t launch_forward_fused(const LaunchArgs&, void*, TimingHook*, size_t) { return hipErrorNotSupported; }
size_t fused_workspace_bytes(int64_t, int32_t, int32_t, size_t) { return 4096; }
size_t noalloc_scratch_bytes() { return 1 << 20; }
size_t conv_bwd_workspace_bytes(int32_t, int32_t, int32_t, int32_t, int32_t, int32_t) { return 4096; }
hipError_t launch_short_conv_backward(const ConvBwdArgs&, void*, TimingHook*) { return hipErrorNotSupported; }
}
