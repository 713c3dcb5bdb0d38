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

// Order of a causal launch's blocks (the kernels' work_item): heads are taken
// in groups whose blocks are interleaved heaviest first, and either each XCD
// gets a contiguous range of the logical numbering (launch_order 0) or the
// numbering follows the launch order, block b on XCD b % 8 (launch_order 1).
// Heaviest first over several heads is what balances the launch: the last
// blocks to start are the lightest of every head.
//   * When the heads split evenly over the XCDs (B*H a multiple of 8), each
//     XCD takes B*H/8 heads, and a group is the largest divisor of that count
//     of at most 8 heads whose K and V fit 16 MiB. No group straddles two
//     XCDs (a straddling group puts its heavy blocks on one XCD and its light
//     blocks on the next), and the eight XCDs' groups in flight stay within
//     half of the 256 MB last-level cache.
//   * Otherwise per-XCD ranges would split heads the same way, so the launch
//     order deals every rank of a group round-robin over the XCDs, and one
//     group, spread over all eight, takes as many heads as fit 128 MiB, at
//     most 64.
// Measured forward (fp16/bf16, us per call against one head per group or
// groups whose K and V fit 2 MiB, interleaved on one box), d = 64: N = 2048
// B*H = 512 343 vs 353 (16 heads 340, at twice the L2 misses), N = 4096
// B*H = 128 296 vs 325, N = 8192 B*H = 32 282 vs 315, N = 16384 B*H = 16 546
// vs 574, N = 32768 B*H = 2 372 vs 492-521, N = 8192 B*H = 6 98 vs 131-134;
// d = 128: N = 16384 B*H = 32 1826 vs 1860, B*H = 12 732 vs 830-962,
// B*H = 4 389 vs 395-425, N = 8192 B*H = 32 477 vs 503, N = 2048 B*H = 128
// 160 vs 187; d = 32 N = 6400 B*H = 64 244 vs 277.
struct CausalOrder {
  int group, launch_order;
};
inline CausalOrder causal_order(int64_t heads, int64_t kv_head_bytes) {
  const int64_t kv = kv_head_bytes > 0 ? kv_head_bytes : 1;
  if (heads % 8 == 0) {
    int64_t cap = ((int64_t)16 << 20) / kv;
    cap = cap > 8 ? 8 : cap;
    const int64_t per_xcd = heads / 8;
    int64_t g = 1;
    for (int64_t c = cap; c > 1; --c)
      if (per_xcd % c == 0) {
        g = c;
        break;
      }
    return {(int)g, 0};
  }
  int64_t cap = ((int64_t)128 << 20) / kv;
  cap = cap < 1 ? 1 : (cap > 64 ? 64 : cap);
  return {(int)(heads < cap ? heads : cap), 1};
}

}  // namespace fa
