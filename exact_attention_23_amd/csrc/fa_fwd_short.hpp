// fa_fwd_short.hpp - the exact-attention forward for short key ranges on
// gfx950: the keys of a head are split over the waves of one workgroup.
//
// Method: the same attention, and the same exactness argument, as the tiled
// kernel (kwkr.cn YOLO11 FlashAttention-2 article, section 1.2; "FlashAttention
// 深度解读", section 原理 items 1-2). A row's softmax over its keys is the
// combination of softmaxes over disjoint key ranges: with per-range maxima
// m_w, sums l_w and unnormalised outputs O_w, the row's maximum is
// M = max_w m_w, its sum L = sum_w 2^(m_w - M) l_w and its output
// O = sum_w 2^(m_w - M) O_w / L (exp2 domain). The articles' online update is
// the sequential form of this combination; here it runs in parallel.
//
// gfx950 mapping
//   * A workgroup owns 32 query rows of one (batch, head) and one wave per
//     64-key tile of the head (up to kShortMaxWaves), so a short sequence is
//     a single tile deep: its latency is one tile, not Nk/64 tiles in turn.
//   * Each wave reads its K rows straight from global memory as MFMA A
//     operands (in the permuted key order that makes the score accumulators
//     the P operand, as in the tiled kernel) and its V tile into its own LDS
//     region; the V^T operands of P V come from that region through
//     ds_read_b64_tr_b16 (two transpose reads give the 8 keys of a fragment).
//   * Each wave takes the exact maximum of its tile, forms P = 2^(S*c - m_w)
//     (at most 1), its row sum on the matrix cores from the rounded P (the
//     normaliser of O; for bf16 also the fp32 sum of the unrounded P, for the
//     LSE) and O_w, and leaves m_w, the sums and the unnormalised O_w in LDS
//     (O_w in its own region, which only it has read). After one barrier
//     each thread merges 8 columns of one row over the waves, normalises and
//     stores them (and the row's LSE).
//   * The chain is latency-bound (one tile deep): every Q and K load is
//     issued before the first MFMA, so it pays one memory round trip.
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa {

// Most 64-key tiles (one wave each) a short-range workgroup takes; LDS holds
// one V tile, later one fp32 partial O, per wave.
template <int D>
constexpr int kShortMaxWaves = D == 128 ? 9 : 16;

template <int D, bool CAUSAL, typename T>
__global__ __launch_bounds__(1024) void fa_fwd_short_kernel(Params p) {
  using M = Mma<T>;
  using vec = typename M::vec;
  using pair = typename M::pair;
  constexpr int KS = D / 16;    // k-steps of the QK^T contraction
  constexpr int NDT = D / 32;   // 32-wide d tiles of O
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int MAXW = kShortMaxWaves<D>;
  constexpr int PS = D + 4;                 // floats per row of a partial O (padded; rows stay 16-byte aligned)
  constexpr int REGION = 32 * PS * 4;       // per-wave LDS bytes: partial O ...
  static_assert(REGION >= 64 * D * 2, "... and, before it, the wave's V tile");
  __shared__ __attribute__((aligned(1024))) char smem[MAXW * REGION];
  // per wave and row: reference, normaliser sum, log-sum-exp sum
  __shared__ float s_m[MAXW][32], s_l[MAXW][32], s_l32[MAXW][32];

  // Workgroup w runs on XCD w % 8 (round-robin dispatch); number the blocks
  // contiguously per XCD so that a head's blocks share one or two XCDs and
  // their K and V reads are served by one L2 instead of every XCD's.
  const int xcd = blockIdx.x & 7;
  const int L = xcd * p.xcd_q + (xcd < p.xcd_r ? xcd : p.xcd_r) + (blockIdx.x >> 3);
  const int head = L / p.num_qb;
  const int qb = L - head * p.num_qb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // scalar wave index: every per-wave choice below is a scalar branch
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int r32 = lane & 31;
  const int Nq = p.Nq, Nk = p.Nk, nw = p.nkt;

  const int hb = head / p.H, hh = head - hb * p.H;
  const int qrs = 2 * p.sq.n, krs = 2 * p.sk.n, vrs = 2 * p.sv.n;  // row strides in bytes
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)head_base<const T>(p.q, p.sq, hb, hh), (short)0, head_bytes<D>(Nq, p.sq), kBufferFlags);
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)head_base<const T>(p.k, p.sk, hb, hh), (short)0, head_bytes<D>(Nk, p.sk), kBufferFlags);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)head_base<const T>(p.v, p.sv, hb, hh), (short)0, head_bytes<D>(Nk, p.sv), kBufferFlags);

  const int q0 = qb * 32;
  const int q_row = q0 + r32;
  const int kb = wave * 64;  // this wave's first key
  char* vreg = smem + wave * REGION;

  // ---- this wave's V tile (64 keys, rows past Nk read as zero) -> its LDS
  // region, rows XOR-swizzled in 16-byte chunks as in the tiled kernel
  {
    const uint32_t lds_v = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)vreg;
#pragma unroll
    for (int i = 0; i < CPR; ++i) {
      const int sl = i * 64 + lane;
      const int r = sl / CPR;
      const int ch = (lds_off<2 * D>(r, sl % CPR) - r * (2 * D)) >> 4;  // logical chunk
      dma_to_lds(v_rsrc, __builtin_amdgcn_readfirstlane(lds_v + i * 1024),
                 (uint32_t)((kb + r) * vrs + 16 * ch));
    }
  }

  // ---- Q rows (B operands) and K rows (A operands, permuted key order).
  // Every load is issued before the first is used, so the chain pays one
  // memory round trip, not one per k-step.
  u32x4 qw[KS], kw[2][KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qw[s] = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, q_row * qrs + 2 * (16 * s + 8 * half), 0, 0);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int krow = kb + 32 * t + lds_row_to_key(r32);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kw[t][s] = __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, krow * krs + 2 * (16 * s + 8 * half), 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  vec qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int e = 0; e < 4; ++e) qw[s][e] = (qw[s][e] & p.q_and) ^ p.q_xor;
    qf[s] = __builtin_bit_cast(vec, qw[s]);
  }
  f32x16 sacc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sacc[t] = M::run(__builtin_bit_cast(vec, kw[t][s]), qf[s], s == 0 ? f32x16{} : sacc[t]);

  // ---- mask (keys past Nk; causal: keys after the row), exact maximum of
  // the tile, P and its row sum
  const float c = p.c;
  {
    int lim = CAUSAL ? (q_row + 1 < Nk ? q_row + 1 : Nk) : Nk;
    lim -= kb + 16 * half;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[t][i] = (32 * t + i < lim) ? sacc[t][i] : -__builtin_inff();
  }
  float m;
  {
    float m4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) m4[k] = vmax(sacc[0][k], sacc[1][k]);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 4; i < 16; ++i) m4[i & 3] = vmax(m4[i & 3], sacc[t][i]);
    m = max_with_partner(vmax(vmax(m4[0], m4[1]), vmax(m4[2], m4[3]))) * c;
  }
  const bool empty = m == -__builtin_inff();  // no visible key in this tile
  const float negm = empty ? 0.f : -m;        // then every score is -inf and P = 0
  vec pf[2][2];
  float lsum = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    u32x4 w[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][2 * i], c, negm));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][2 * i + 1], c, negm));
      const pair pp = M::cvt(p0, p1);
      lsum = M::lse_sum(p0, p1, lsum);
      w[i >> 2][i & 3] = __builtin_bit_cast(uint32_t, pp);
    }
    pf[t][0] = __builtin_bit_cast(vec, w[0]);
    pf[t][1] = __builtin_bit_cast(vec, w[1]);
  }
  // row sum of the rounded P (selector of the tiled kernel: lane l's sum
  // lands in every register), and for bf16 the fp32 sum for the LSE
  float l, l32;
  {
    const vec row_sel = M::selector((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) acc = M::sel_sum(row_sel, pf[t][s2], acc);
    l = acc[0];
    l32 = M::kLse32 ? sum_with_partner(lsum) : l;
  }

  // ---- O_w^T = V^T P^T. The V^T fragment for d tile dt, unit t, half s2 is
  // d row 32*dt + lane%32 and keys 32t + 16*half + 8*s2 .. +7: two transpose
  // reads, each handing lane x of a 16-lane group keys k0..k0+3 of column
  // d0 + x while pointing at key k0 + x/4, columns d0 + 4*(x%4) .. +3.
  wait_vmcnt<0>();  // this wave's V tile has landed (only this wave reads it)
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  {
    const int x = lane & 15;
    const int d0b = 16 * ((lane >> 4) & 1);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int k0 = 32 * t + 16 * half + 8 * s2;
          const int col = 32 * dt + d0b + 4 * (x & 3);
          const int a0 = lds_off<2 * D>(k0 + (x >> 2), col >> 3) + 2 * (col & 7);
          const int a1 = lds_off<2 * D>(k0 + 4 + (x >> 2), col >> 3) + 2 * (col & 7);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vreg + a0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vreg + a1));
          const u32x2 wl = __builtin_bit_cast(u32x2, lo), wh = __builtin_bit_cast(u32x2, hi);
          const u32x4 w = {wl[0], wl[1], wh[0], wh[1]};
          oacc[dt] = M::run(__builtin_bit_cast(vec, w), pf[t][s2], oacc[dt]);
        }
  }

  // ---- combine the waves. Each wave leaves its reference m_w, row sums
  // (n_w of the rounded P, l_w for the LSE) and unnormalised O_w (rows =
  // queries) in its own LDS region, which only it has read so far; after one
  // barrier every thread merges, for its rows and columns, M = max m_w,
  // O = sum 2^(m_w - M) O_w / sum 2^(m_w - M) n_w and
  // LSE = ln2 (M + log2 sum 2^(m_w - M) l_w).
  if (half == 0) {
    s_m[wave][r32] = m;  // -inf for a tile with no visible key
    s_l[wave][r32] = l;
    s_l32[wave][r32] = l32;
  }
  // accumulator registers 4g..4g+3 hold columns 32dt + 8g + 4half .. +3 of
  // the lane's query: one 16-byte store each
  float* part = (float*)vreg;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(f32x4*)(part + r32 * PS + 32 * dt + 8 * g + 4 * half) =
          f32x4{oacc[dt][4 * g], oacc[dt][4 * g + 1], oacc[dt][4 * g + 2], oacc[dt][4 * g + 3]};
  __syncthreads();

  // Thread e merges row e / (D/8), columns 8*(e % (D/8)) .. +7.
  T* Oh = head_base<T>(p.o, p.so, hb, hh);
  for (int e = tid; e < 4 * D; e += 64 * nw) {
    const int r = e / (D / 8), d = 8 * (e % (D / 8));
    if (q0 + r >= Nq) continue;
    float mw[MAXW];
    float Mx = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < MAXW; ++w) {
      mw[w] = w < nw ? s_m[w][r] : -__builtin_inff();
      Mx = vmax(Mx, mw[w]);
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float L = 0.f, L32 = 0.f;
#pragma unroll
    for (int w = 0; w < MAXW; ++w) {
      if (w < nw) {
        const float f = mw[w] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mw[w] - Mx);
        const float* pw = (const float*)(smem + w * REGION) + r * PS + d;
        const f32x4 x0 = *(const f32x4*)pw, x1 = *(const f32x4*)(pw + 4);
        L += f * s_l[w][r];
        L32 += f * s_l32[w][r];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] += f * x0[i];
          acc[4 + i] += f * x1[i];
        }
      }
    }
    const float inv = 1.0f / L;
    u32x4 ow;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ow[i] = __builtin_bit_cast(uint32_t, M::cvt(acc[2 * i] * inv, acc[2 * i + 1] * inv));
    *(u32x4*)(Oh + (int64_t)(q0 + r) * p.so.n + d) = ow;
    if (p.lse != nullptr && d == 0)
      p.lse[(size_t)head * Nq + q0 + r] = 0.69314718055994531f * (Mx + log2f(L32));
  }
}

}  // namespace fa
