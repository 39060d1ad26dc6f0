// Host-side launchers of the gfx950 kernels (defined in gdn_kernels.hip).
#pragma once

#include <hip/hip_runtime_api.h>

#include "gdn_internal.h"

namespace gdn {

// True when kernels for this element type / chunk / d_k were built (some
// fp32 combinations exceed the 160 KiB of LDS and are not).
bool kernels_available(bool bf16, int chunk, int dk);

// 16-column state slices per scan workgroup (1 or 2) for this problem;
// seq_heads = sequences x value heads.  Queries the current device.
int scan_slices_per_group(bool bf16, int chunk, int dk, int dv, int64_t seq_heads);

hipError_t launch_table(const TableParams& p, hipStream_t s);
// One WY workgroup per (chunk, key head) item.
hipError_t launch_wy(bool bf16, int chunk, int dk, const WyParams& p, hipStream_t s);
hipError_t launch_scan(bool bf16, int chunk, int dk, const ScanParams& p,
                       int grid_x, hipStream_t s);

// The two-level scan: both segments in one launch, then the correction of
// the second segment's outputs and the final state.
bool two_level_available(bool bf16, int chunk, int dk);
hipError_t launch_scan_two_level(int chunk, int dk, const ScanParams& p, hipStream_t s);

hipError_t launch_decode(bool bf16, int dk, const DecodeParams& p, hipStream_t s);

// The short convolution's state after a prefill or a decode step: the last
// width - 1 raw rows of every sequence and channel.
hipError_t launch_conv_state(bool bf16, const ConvStateParams& p, hipStream_t s);

// GDN_DEBUG_CHECK: ORs the fault bits (gdn_cu_check.h) of cu[0 .. n_seq]
// (int32 entries, or int64 with cu_i64) into one word and stores it at
// *faults (one workgroup).
hipError_t launch_check_cu(const void* cu, bool cu_i64, int64_t n_seq, int64_t t_total,
                           int32_t* faults, hipStream_t s);

// Device address of the current device's fault word for launch_check_cu
// (a static device variable, looked up once per device).
hipError_t debug_word_region(int32_t** ptr);

// The gated output norm (dv in {16, 32, 64, 128}).
hipError_t launch_output_gate(bool bf16, int dv, const GateParams& p, hipStream_t s);

// Size of the device scratch that serves as the workspace of
// gdn_prefill_noalloc (include/gdn.h: GDN_NOALLOC_SCRATCH_BYTES).
constexpr size_t kScratchBytes = (size_t)96 << 20;

// Device address of the current device's scratch (looked up on the first
// call per device; no allocation).
hipError_t scratch_region(void** ptr);

}  // namespace gdn
