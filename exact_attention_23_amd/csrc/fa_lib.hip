// fa_lib.hip - library-wide entry points of libfa.so: version, status strings
// and the last launch error, plus the host helpers of fa_host.hpp.
#include <hip/hip_runtime.h>

#include "../../include/fa.h"
#include "fa_host.hpp"

namespace {

constexpr int kVersion = 200;  // 0.2.0: adds the backward pass

// HIP's description of the last failed launch on this thread.
thread_local const char* g_launch_error = "";

}  // namespace

namespace fa {

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 256;
  return n > 0 ? n : 256;
}

int launch_status(hipError_t e) {
  // Only the launch's own return value counts: hipGetLastError here would
  // also pick up (and clear) an error some earlier, unrelated HIP call left
  // on this thread.
  if (e != hipSuccess) {
    g_launch_error = hipGetErrorString(e);
    return FA_ERR_LAUNCH;
  }
  return FA_OK;
}

}  // namespace fa

extern "C" {

int fa_version(void) { return kVersion; }

const char* fa_last_launch_error(void) { return g_launch_error; }

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULLPTR: return "a tensor pointer is null";
    case FA_ERR_SHAPE: return "B, H, Nq and Nk must be >= 1 and Nq*d, Nk*d < 2^29";
    case FA_ERR_HEADDIM: return "head width d must be 32, 64 or 128";
    case FA_ERR_DTYPE: return "dtype must be FA_DTYPE_FP16 or FA_DTYPE_BF16";
    case FA_ERR_SCALE: return "scale must be finite";
    case FA_ERR_CAUSAL: return "causal must be 0 or 1";
    case FA_ERR_ALIGN: return "tensors must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_ALIAS: return "an output overlaps an input, another output or the workspace";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_PATH: return "unknown path or kernel selection, or the short path with too many keys for it";
    case FA_ERR_STRIDE: return "strides missing, misaligned, overlapping or too large for one head";
    case FA_ERR_WORKSPACE: return "workspace is null, misaligned or smaller than fa_bwd_workspace_bytes";
    case FA_ERR_SCRATCH: return "sizes need more than the static scratch of fa_bwd_noalloc (16 MiB)";
    default: return "unknown status";
  }
}

}  // extern "C"
