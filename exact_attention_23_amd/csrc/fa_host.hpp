// fa_host.hpp - host-side helpers shared by the entry points of libfa.so.
#pragma once
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace fa {

// Compute units of the current device (256 if the query fails).
int device_cus();

// True when the byte ranges [a, a+an) and [b, b+bn) intersect.
inline bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

// FA_OK for hipSuccess (the return value of the launch itself); otherwise
// records HIP's description of the error for fa_last_launch_error() on this
// thread and returns FA_ERR_LAUNCH.
int launch_status(hipError_t e);

// Workgroup scheduling shared by the kernels: logical work items are spread
// over the 8 XCDs in contiguous ranges (see the kernels' work mapping).
struct XcdSplit {
  int q, r;
};
inline XcdSplit xcd_split(int64_t total) { return {(int)(total / 8), (int)(total % 8)}; }

}  // namespace fa
