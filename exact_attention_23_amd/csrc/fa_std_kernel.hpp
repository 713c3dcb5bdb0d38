// fa_std_kernel.hpp - standard (unfused) attention on gfx950: the baseline the
// fused forward is measured against.
//
// Standard attention as the cited articles describe it ("FlashAttention
// 深度解读", section 背景; ai2ai.xin flash-attention-principle page, its
// five-step list of the self-attention bottleneck; kwkr.cn YOLO11
// FlashAttention-2 article, section 1.1): the score matrix S = scale Q K^T is
// written to device memory, read back for the row softmax, the probabilities
// P are written, read back and multiplied by V. Three kernels, each a full
// pass over an Nq x Nk matrix in HBM:
//   1. fa_std_scores_kernel   S = scale * Q K^T          (fp32 S written)
//   2. fa_std_softmax_kernel  P = softmax_rows(mask(S))  (S read, P written,
//                                                         LSE written)
//   3. fa_std_pv_kernel       O = P V                    (P read)
// Causal masking is applied by the softmax (j > i -> weight 0); both products
// run over the whole Nq x Nk square, as a standard implementation does.
//
// Layouts: S is [B, H, Nq, NkP] fp32 and P is [B, H, Nq, NkP] in the input
// type, NkP = Nk rounded up to a multiple of 64, so every row starts 256-byte
// aligned (S) or 128-byte aligned (P) and the products take whole 64-key
// tiles. Columns Nk..NkP-1 of P are written as zeros; those of S are not
// written.
//
// gfx950 mapping: both products use v_mfma_f32_32x32x16_{f16,bf16} with fp32
// accumulation, with operands read from HBM (through L2) by 128-bit buffer
// loads; the P V product stages each 64-key V tile in LDS and takes its
// transposed operand with ds_read_b64_tr_b16. The softmax is one 256-thread
// workgroup per row, holding the row in registers (up to 16384 keys; longer
// rows are streamed three times).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"

namespace fa {

struct StdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  float* s;    // [B*H][Nq][NkP] fp32
  void* p;     // [B*H][Nq][NkP] input type
  int B, H, Nq, Nk, NkP;
  float scale;
  int causal;
  int nqb;  // 128-row blocks per head
  int nkb;  // 64-key blocks per head (score kernel)
};

constexpr float kLog2e = 1.4426950408889634f;

// ---- 1. S = scale * Q K^T, one workgroup per (head, 128 query rows, 64 keys)
template <int D, typename T>
__global__ __launch_bounds__(256) void fa_std_scores_kernel(StdParams p) {
  using M = Mma<T>;
  using vec = typename M::vec;
  constexpr int KS = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, r32 = lane & 31;
  int bid = blockIdx.x;
  const int kb = bid % p.nkb;
  bid /= p.nkb;
  const int qb = bid % p.nqb;
  const int head = bid / p.nqb;
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.q + (int64_t)head * p.Nq * D), (short)0, p.Nq * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.k + (int64_t)head * p.Nk * D), (short)0, p.Nk * D * 2, kBufferFlags);
  // A operand: query rows (lane: row r32, k elements 8*half..+7 of each
  // 16-wide step); B operand: key rows likewise. Rows past the end read 0.
  const int q_row = qb * 128 + wave * 32 + r32;
  vec qf[KS], kf[2][KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = __builtin_bit_cast(vec, __builtin_amdgcn_raw_buffer_load_b128(
                                        q_rsrc, q_row * D * 2 + 2 * (16 * s + 8 * half), 0, 0));
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kf[t][s] = __builtin_bit_cast(vec, __builtin_amdgcn_raw_buffer_load_b128(
                                             k_rsrc, (kb * 64 + 32 * t + r32) * D * 2 + 2 * (16 * s + 8 * half),
                                             0, 0));
  float* Sh = p.s + (int64_t)head * p.Nq * p.NkP;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = M::run(qf[s], kf[t][s], acc);
    // accumulator register i of lane l: query row 8*(i/4) + 4*half + i%4 of
    // the wave's 32, key r32 of the 32-key tile t
    const int key = kb * 64 + 32 * t + r32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = qb * 128 + wave * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (row < p.Nq && key < p.Nk) Sh[(int64_t)row * p.NkP + key] = acc[i] * p.scale;
    }
  }
}

// Workgroup-wide maximum / sum of one value per thread (256 threads).
__device__ __forceinline__ float block_reduce_max(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = vmax(x, __shfl_xor(x, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return vmax(vmax(red[0], red[1]), vmax(red[2], red[3]));
}
__device__ __forceinline__ float block_reduce_sum(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// ---- 2. row softmax: one workgroup of 256 threads per row of S. Thread x
// owns the 4-key groups x, x + 256, ... of the row. E > 0: the row (E groups
// per thread) stays in registers between the passes; E == 0: any length,
// the row is read from memory once per pass.
template <int E, typename T>
__global__ __launch_bounds__(256) void fa_std_softmax_kernel(StdParams p) {
  using M = Mma<T>;
  __shared__ float red[4];
  const int64_t row = blockIdx.x;  // over B*H*Nq
  const int i = (int)(row % p.Nq);
  const float* Sr = p.s + row * p.NkP;
  T* Pr = (T*)p.p + row * p.NkP;
  const int lim = p.causal ? (i + 1 < p.Nk ? i + 1 : p.Nk) : p.Nk;  // keys < lim are visible
  const int tid = threadIdx.x;
  const int ngroups = p.NkP / 4;
  auto load = [&](int g) -> f32x4 {
    f32x4 x = *(const f32x4*)(Sr + 4 * g);
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = (4 * g + c < lim) ? x[c] : -__builtin_inff();
    return x;
  };
  constexpr int NR = E > 0 ? E : 1;
  f32x4 keep[NR];
  float m = -__builtin_inff();
  if constexpr (E > 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int g = tid + 256 * e;
      keep[e] = g < ngroups ? load(g) : f32x4{-__builtin_inff(), -__builtin_inff(), -__builtin_inff(),
                                              -__builtin_inff()};
#pragma unroll
      for (int c = 0; c < 4; ++c) m = vmax(m, keep[e][c]);
    }
  } else {
    for (int g = tid; g < ngroups; g += 256) {
      const f32x4 x = load(g);
#pragma unroll
      for (int c = 0; c < 4; ++c) m = vmax(m, x[c]);
    }
  }
  m = block_reduce_max(m, red);  // finite: key 0 is always visible
  const float mc = m * kLog2e;
  float l = 0.f;
  if constexpr (E > 0) {
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        keep[e][c] = __builtin_amdgcn_exp2f(__builtin_fmaf(keep[e][c], kLog2e, -mc));
        l += keep[e][c];
      }
  } else {
    for (int g = tid; g < ngroups; g += 256) {
      const f32x4 x = load(g);
#pragma unroll
      for (int c = 0; c < 4; ++c) l += __builtin_amdgcn_exp2f(__builtin_fmaf(x[c], kLog2e, -mc));
    }
  }
  l = block_reduce_sum(l, red);
  const float inv = 1.0f / l;
  auto store = [&](int g, f32x4 e4) {
    u32x2 w;
    w[0] = __builtin_bit_cast(uint32_t, M::cvt(e4[0] * inv, e4[1] * inv));
    w[1] = __builtin_bit_cast(uint32_t, M::cvt(e4[2] * inv, e4[3] * inv));
    *(u32x2*)(Pr + 4 * g) = w;
  };
  if constexpr (E > 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int g = tid + 256 * e;
      if (g < ngroups) store(g, keep[e]);
    }
  } else {
    for (int g = tid; g < ngroups; g += 256) {
      f32x4 x = load(g);
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[c], kLog2e, -mc));
      store(g, x);
    }
  }
  if (p.lse != nullptr && tid == 0) p.lse[row] = m + 0.69314718055994531f * log2f(l);
}

// ---- 3. O = P V, one workgroup per (head, 128 query rows); wave w owns rows
// 32w..32w+31 and computes O^T = V^T P^T over 64-key tiles. The P^T operand
// (lane: query r32, keys 16s + 8*half .. +7 of k-step s) is one 16-byte
// load from the P row; the V^T operand (lane: d row 32dt + r32, the same
// keys) comes from the tile in LDS through two transpose reads. The V tile
// is double-buffered: one barrier per tile.
template <int D, typename T>
__global__ __launch_bounds__(256) void fa_std_pv_kernel(StdParams p) {
  using M = Mma<T>;
  using vec = typename M::vec;
  constexpr int NDT = D / 32;
  constexpr int CPR = D / 8;                 // 16-byte chunks per V row
  constexpr int CPT = 64 * CPR / 256;        // chunks per thread per tile
  __shared__ __attribute__((aligned(1024))) char vt[2][64 * D * 2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, r32 = lane & 31;
  const int head = blockIdx.x / p.nqb;
  const int qb = blockIdx.x - head * p.nqb;
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.v + (int64_t)head * p.Nk * D), (short)0, p.Nk * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t p_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.p + (int64_t)head * p.Nq * p.NkP), (short)0, p.Nq * p.NkP * 2, kBufferFlags);
  const int q_row = qb * 128 + wave * 32 + r32;
  const int ntiles = p.NkP / 64;
  // byte offset of this lane's P row; rows past Nq point past the buffer's
  // range (they read zeros), which also keeps the offset from wrapping
  const uint32_t prow = q_row < p.Nq ? (uint32_t)q_row * (uint32_t)p.NkP * 2u : 0x80000000u;

  auto fetch = [&](int kt, u32x4 (&r)[CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + 256 * c;
      r[c] = __builtin_amdgcn_raw_buffer_load_b128(v_rsrc, (kt * 64 + ch / CPR) * D * 2 + 16 * (ch % CPR), 0, 0);
    }
  };
  auto stash = [&](int buf, const u32x4 (&r)[CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + 256 * c;
      *(u32x4*)(vt[buf] + lds_off<2 * D>(ch / CPR, ch % CPR)) = r[c];
    }
  };
  // transpose-read addresses of k-step s, d tile dt (first of the two reads;
  // the second is 4 keys further): in 16-lane group g the block starts at
  // key 16s + 8*half and d column 32dt + 16*(g%2); lane x points at key
  // k0 + x/4, columns d0 + 4*(x%4)..+3 and receives keys k0..k0+3 of
  // column d0 + x.
  const int x = lane & 15;
  const int d0b = 16 * ((lane >> 4) & 1);

  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
  {
    u32x4 r[CPT];
    fetch(0, r);
    stash(0, r);
  }
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    u32x4 nxt[CPT];
    if (kt + 1 < ntiles) fetch(kt + 1, nxt);
    vec pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      pf[s] = __builtin_bit_cast(vec, __builtin_amdgcn_raw_buffer_load_b128(
                                          p_rsrc, prow + 2 * (kt * 64 + 16 * s + 8 * half), 0, 0));
    const char* tile = vt[kt & 1];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int k0 = 16 * s + 8 * half;
        const int col = 32 * dt + d0b + 4 * (x & 3);
        const int a0 = lds_off<2 * D>(k0 + (x >> 2), col >> 3) + 2 * (col & 7);
        const int a1 = lds_off<2 * D>(k0 + 4 + (x >> 2), col >> 3) + 2 * (col & 7);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + a0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + a1));
        const u32x2 wl = __builtin_bit_cast(u32x2, lo), wh = __builtin_bit_cast(u32x2, hi);
        const u32x4 w = {wl[0], wl[1], wh[0], wh[1]};
        oacc[dt] = M::run(__builtin_bit_cast(vec, w), pf[s], oacc[dt]);
      }
    if (kt + 1 < ntiles) stash((kt + 1) & 1, nxt);
    __syncthreads();
  }
  if (q_row < p.Nq) {
    T* Oh = (T*)p.o + ((int64_t)head * p.Nq + q_row) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = __builtin_bit_cast(uint32_t, M::cvt(oacc[dt][4 * g + 0], oacc[dt][4 * g + 1]));
        w[1] = __builtin_bit_cast(uint32_t, M::cvt(oacc[dt][4 * g + 2], oacc[dt][4 * g + 3]));
        *(u32x2*)(Oh + 32 * dt + 8 * g + 4 * half) = w;
      }
  }
}

}  // namespace fa
