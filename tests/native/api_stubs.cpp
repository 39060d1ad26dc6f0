// Host-only stand-ins for the kernel launchers (gdn_launch.h) and for the
// HIP runtime calls that gdn_api.cpp makes, so that the C ABI's host code
// (argument validation, workspace layout, option handling, graph-cache
// bookkeeping) can be built and run under AddressSanitizer and
// UndefinedBehaviorSanitizer with no GPU and no HIP runtime.  Every launch
// and runtime call reports hipErrorNoDevice, so calls that pass validation
// end with GDN_ERR_HIP.
#include <hip/hip_runtime_api.h>

#include "gdn_internal.h"
#include "gdn_launch.h"

namespace gdn {

bool kernels_available(bool bf16, int chunk, int dk) { return bf16 || chunk < 64 || dk < 128; }
int scan_slices_per_group(bool, int, int, int, int64_t) { return 1; }
hipError_t launch_table(const TableParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_wy(bool, int, int, const WyParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_scan(bool, int, int, const ScanParams&, int, hipStream_t) { return hipErrorNoDevice; }
bool two_level_available(bool bf16, int chunk, int dk) { return bf16 && chunk >= 32 && dk >= 32; }
hipError_t launch_scan_two_level(int, int, const ScanParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode(bool, int, const DecodeParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_conv_state(bool, const ConvStateParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_check_cu(const void*, bool, int64_t, int64_t, int32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t debug_word_region(int32_t**) { return hipErrorNoDevice; }
hipError_t launch_output_gate(bool, int, const GateParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t scratch_region(void**) { return hipErrorNoDevice; }

}  // namespace gdn

extern "C" {
const char* hipGetErrorString(hipError_t) { return "no device (host-only build)"; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipMallocAsync(void**, size_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t hipFreeAsync(void*, hipStream_t) { return hipErrorNoDevice; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return hipErrorNoDevice; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipErrorNoDevice; }
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus*) { return hipErrorNoDevice; }
hipError_t hipStreamCreateWithFlags(hipStream_t*, unsigned int) { return hipErrorNoDevice; }
hipError_t hipStreamDestroy(hipStream_t) { return hipErrorNoDevice; }
hipError_t hipStreamBeginCapture(hipStream_t, hipStreamCaptureMode) { return hipErrorNoDevice; }
hipError_t hipStreamEndCapture(hipStream_t, hipGraph_t*) { return hipErrorNoDevice; }
hipError_t hipGraphInstantiate(hipGraphExec_t*, hipGraph_t, hipGraphNode_t*, char*, size_t) {
  return hipErrorNoDevice;
}
hipError_t hipGraphLaunch(hipGraphExec_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t hipGraphExecDestroy(hipGraphExec_t) { return hipErrorNoDevice; }
hipError_t hipGraphDestroy(hipGraph_t) { return hipErrorNoDevice; }
hipError_t hipGraphExecUpdate(hipGraphExec_t, hipGraph_t, hipGraphNode_t*, hipGraphExecUpdateResult*) {
  return hipErrorNoDevice;
}
}
