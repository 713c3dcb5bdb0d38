// fa_probe.hip - throughput probes (libfa_probe.so): how many v_exp_f32 and
// v_fma_f32 per second the chip retires when every SIMD has several waves of
// independent work, the rate of the forward's matrix instruction on its own,
// and how far matrix and vector work of different waves on one SIMD overlap.
// The declarations live in include/fa_probe.h.
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

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMatrixChains = 4;

// kMatrixChains independent accumulators per wave, each taking one
// v_mfma_f32_32x32x16_f16 per step (accumulators in vector registers, as in
// the forward). Operands are small, so the sums stay finite.
__device__ __forceinline__ float matrix_chains(int iters) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (float)((lane + i) & 31));
    b[i] = (_Float16)(0.001f * (float)((lane + 3 * i) & 31));
  }
  f32x16 acc[kMatrixChains];
#pragma unroll
  for (int c = 0; c < kMatrixChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMatrixChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int c = 0; c < kMatrixChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[c][i];
  return r;
}

// The 16x16x32 shape: 8 independent accumulator chains per wave, so a step
// is the same FLOP count as a step of the 32x32x16 chains above.
__device__ __forceinline__ float matrix_chains16(int iters) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (float)((lane + i) & 31));
    b[i] = (_Float16)(0.001f * (float)((lane + 3 * i) & 31));
  }
  f32x4 acc[2 * kMatrixChains];
#pragma unroll
  for (int c = 0; c < 2 * kMatrixChains; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 2 * kMatrixChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int c = 0; c < 2 * kMatrixChains; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) r += acc[c][i];
  return r;
}

template <int SHAPE>
__global__ __launch_bounds__(256) void matrix_kernel(int iters, float* out) {
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = SHAPE == 0 ? matrix_chains(iters) : matrix_chains16(iters);
}

// Softmax-shaped vector work per step: for 32 values per lane, one FMA, one
// exp2 and (per pair) one round-to-half pack, as the forward does per score.
// Each value maps to 2^(-1.44 x - 0.5), which keeps it in [0.35, 0.71].
__device__ __forceinline__ float vector_steps(int iters) {
  const int lane = threadIdx.x & 63;
  float s[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) s[i] = 0.01f * (float)((lane + i) & 15);
  uint32_t w = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i], -1.4426950f, -0.5f));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i + 1], -1.4426950f, -0.5f));
      const f32x2 f = {p0, p1};
      w ^= __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
      s[2 * i] = p0;
      s[2 * i + 1] = p1;
    }
  }
  float r = (float)(w & 1);
#pragma unroll
  for (int i = 0; i < 32; ++i) r += s[i];
  return r;
}

// Waves 0-3 of a 512-thread workgroup (one per SIMD) run matrix chains when
// bit 0 of roles is set; waves 4-7 (the second wave of each SIMD) run the
// vector steps when bit 1 is set.
__global__ __launch_bounds__(512) void coexec_kernel(int roles, int miters, int viters, float* out) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  float r = 1.f;
  if (wave < 4) {
    if (roles & 1) r = matrix_chains(miters);
  } else {
    if (roles & 2) r = vector_steps(viters);
  }
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = r;
}

// One wave per SIMD per workgroup of 256 threads; per step, 16 matrix
// instructions (8 chains of v_mfma_f32_16x16x32_f16, two each) and/or the
// vector steps' work on 32 values. MODE 1: matrix only; 2: vector only; 3:
// both, in the compiler's order; 4: both, the instruction stream interleaved
// one matrix instruction to five vector instructions (scheduling groups).
template <int MODE>
__global__ __launch_bounds__(256) void coissue_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (float)(lane + i));
    b[i] = (_Float16)(0.002f * (float)(i - lane));
  }
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float s[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) s[i] = 0.01f * (float)((lane + i) & 15);
  uint32_t w = 0;
  for (int it = 0; it < iters; ++it) {
    if (MODE != 2) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
    }
    if (MODE != 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i], -1.4426950f, -0.5f));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i + 1], -1.4426950f, -0.5f));
        const f32x2 f = {p0, p1};
        w ^= __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
        s[2 * i] = p0;
        s[2 * i + 1] = p1;
      }
    }
    if (MODE == 4) {
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix instruction
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // five vector instructions
      }
    }
  }
  float r = (float)(w & 1);
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) r += acc[c][i];
#pragma unroll
  for (int i = 0; i < 32; ++i) r += s[i];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = r;
}

}  // namespace

extern "C" int fa_probe_matrix_rate(int shape, int blocks, int iters, float* out, void* stream) {
  if (shape < 0 || shape > 1 || blocks < 1 || iters < 1 || out == nullptr) return 1;
  void* args[] = {&iters, &out};
  const void* fn = shape == 0 ? (const void*)matrix_kernel<0> : (const void*)matrix_kernel<1>;
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, (hipStream_t)stream) == hipSuccess ? 0 : 2;
}

extern "C" int fa_probe_coexec(int roles, int blocks, int matrix_iters, int vector_iters, float* out,
                               void* stream) {
  if (roles < 1 || roles > 3 || blocks < 1 || matrix_iters < 1 || vector_iters < 1 || out == nullptr)
    return 1;
  void* args[] = {&roles, &matrix_iters, &vector_iters, &out};
  return hipLaunchKernel((const void*)coexec_kernel, dim3((unsigned)blocks), dim3(512), args, 0,
                         (hipStream_t)stream) == hipSuccess ? 0 : 2;
}

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

extern "C" int fa_probe_coissue(int mode, int blocks, int iters, float* out, void* stream) {
  if (mode < 1 || mode > 4 || blocks < 1 || iters < 1 || out == nullptr) return 1;
  void* args[] = {&iters, &out};
  const void* fn = mode == 1   ? (const void*)coissue_kernel<1>
                   : mode == 2 ? (const void*)coissue_kernel<2>
                   : mode == 3 ? (const void*)coissue_kernel<3>
                               : (const void*)coissue_kernel<4>;
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, (hipStream_t)stream) == hipSuccess ? 0 : 2;
}
