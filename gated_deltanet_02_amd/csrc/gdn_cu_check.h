// The preconditions of a cu_seqlens table, as one predicate shared by the
// host validator (gdn_check_cu_seqlens) and the device check that
// GDN_DEBUG_CHECK=1 runs before a packed prefill (include/gdn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Fault bits of a table entry (0: the entry is well formed).
enum : int32_t {
  kCuFirstNonzero = 1,  // cu[0] != 0
  kCuDecreasing = 2,    // cu[i] < cu[i - 1]
  kCuPastEnd = 4,       // cu[N] > T
};

// Faults of entry i (0 .. n_seq) of cu[n_seq + 1] (int32 or int64 entries)
// for t_total tokens.
template <typename I>
__host__ __device__ inline int32_t cu_entry_faults(const I* cu, int64_t i, int64_t n_seq,
                                                   int64_t t_total) {
  int32_t f = 0;
  if (i == 0 && cu[0] != 0) f |= kCuFirstNonzero;
  if (i > 0 && cu[i] < cu[i - 1]) f |= kCuDecreasing;
  if (i == n_seq && (int64_t)cu[i] > t_total) f |= kCuPastEnd;
  return f;
}

}  // namespace gdn
