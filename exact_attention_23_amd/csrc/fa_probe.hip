// fa_probe.hip - vector-unit throughput probe (libfa_probe.so): how many
// v_exp_f32 and v_fma_f32 per second the chip retires when every SIMD has
// several waves of independent work. The declarations live in
// include/fa_probe.h.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/fa_probe.h"

namespace {

constexpr int kChains = 8;

// Each chain stays in (0.5, 2): 2^-x and 2^(x/2 - 1/4) for the exp chains, a
// contraction toward 1 for the FMA chains, so no value overflows or turns
// denormal.
template <int OP>
__global__ __launch_bounds__(256) void probe_kernel(int iters, float* out) {
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = 1.0f + 0.01f * (float)((threadIdx.x + c) & 7);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (OP == FA_PROBE_EXP2) {
        x[c] = __builtin_amdgcn_exp2f(-x[c]);  // one v_exp_f32 with a negated source
      } else if constexpr (OP == FA_PROBE_FMA) {
        x[c] = __builtin_fmaf(x[c], 0.999f, 0.001f);
      } else {
        x[c] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[c], -0.5f, 0.25f));
      }
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc += x[c];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" int fa_probe_vector_rate(int op, int blocks, int iters, int chains, float* out, void* stream) {
  if (op < FA_PROBE_EXP2 || op > FA_PROBE_MIX || blocks < 1 || iters < 1 || chains != kChains ||
      out == nullptr)
    return 1;
  void* args[] = {&iters, &out};
  const void* fn = op == FA_PROBE_EXP2 ? (const void*)probe_kernel<FA_PROBE_EXP2>
                   : op == FA_PROBE_FMA ? (const void*)probe_kernel<FA_PROBE_FMA>
                                        : (const void*)probe_kernel<FA_PROBE_MIX>;
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, (hipStream_t)stream) == hipSuccess ? 0 : 2;
}
