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
//   * A workgroup owns QB blocks of 16 query rows of one (batch, head) and
//     one wave per 64-key tile of the head (up to kShortMaxWaves), so a short
//     sequence is a single tile deep: its latency is one tile, not Nk/64
//     tiles in turn. One block per workgroup halves each wave's chain; two
//     keep the workgroups to one per compute unit when one-block workgroups
//     would have to share them.
//     Workgroups are numbered contiguously per XCD (workgroup w runs on XCD
//     w % 8), so a head's blocks share one or two L2s.
//   * The register layouts are those of the tiled kernel (fa_fwd16.hpp) for
//     16-row blocks on v_mfma_f32_16x16x32_{f16,bf16}: each wave reads its
//     K rows (A operands) and the block's Q rows (B operands) straight from
//     memory, every load issued before the first MFMA, so the chain pays one
//     memory round trip; its V tile goes by DMA into its own LDS region, and
//     the V^T operands of P V come from there by transpose reads.
//   * Each wave takes the exact maximum of its tile, so P = 2^(S*c - m_w) is
//     at most 1, its row sum on the matrix cores from the rounded P (the
//     normaliser of O; for bf16 also the fp32 sum of the unrounded P, for the
//     LSE) and O_w, and leaves m_w, the sums and the unnormalised O_w in LDS
//     (O_w over its own V tile, which only it has read). After one barrier
//     each thread merges 4 (one block) or 8 (two) columns of one row over the
//     waves, normalises and stores them (and the row's LSE).
//   * The LDS footprint is sized for NWMAX waves (8 or 16; 9 at d = 128), so
//     workgroups of up to 8 tiles at d <= 64 fit two to a compute unit.
#pragma once

#include "fa_fwd16.hpp"

namespace fa {

// Most 64-key tiles (one wave each) a short-range workgroup takes.
template <int D>
constexpr int kShortMaxWaves = D == 128 ? 9 : 16;

// LDS bytes per wave: its V tile (64 keys x D, 16-bit), later its partial O
// (16 QB rows of D + 4 floats); a multiple of 256 bytes, so every region
// keeps the tile swizzle's bank pattern.
template <int D, int QB>
constexpr int kShortRegion = 64 * D * 2 > 16 * QB * (D + 4) * 4 ? 64 * D * 2 : 16 * QB * (D + 4) * 4;

template <int D, int NWMAX, int QB, bool CAUSAL, typename T>
__global__ __launch_bounds__(64 * NWMAX) void fa_fwd_short_kernel(Params p) {
  using M = Mma<T>;
  using vec = typename M::vec;
  constexpr int KS = D / 32;   // k-steps of Q K^T
  constexpr int NDB = D / 16;  // 16-wide d blocks of O
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  constexpr int PS = D + 4;    // floats per row of a partial O (padded; rows stay 16-byte aligned)
  constexpr int ROWS = 16 * QB;
  constexpr int REGION = kShortRegion<D, QB>;
  static_assert(NWMAX <= kShortMaxWaves<D>, "wave count");
  static_assert(REGION % 256 == 0, "regions keep the swizzle's bank pattern");
  __shared__ __attribute__((aligned(1024))) char smem[NWMAX * REGION];
  // per wave and row: reference, normaliser sum, log-sum-exp sum
  __shared__ float s_m[NWMAX][ROWS], s_l[NWMAX][ROWS], s_l32[NWMAX][ROWS];

  const int xcd = blockIdx.x & 7;
  const int L = xcd * p.xcd_q + (xcd < p.xcd_r ? xcd : p.xcd_r) + (blockIdx.x >> 3);
  const int head = L / p.num_qb;
  const int qb = L - head * p.num_qb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // scalar wave index: every per-wave choice below is a scalar branch
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int x = lane & 15;
  const int g = lane >> 4;
  const int Nq = p.Nq, Nk = p.Nk, nw = p.nkt;

  const int hb = head / p.H, hh = head - hb * p.H;
  const int qrs = 2 * p.sq.n, krs = 2 * p.sk.n, vrs = 2 * p.sv.n;  // row strides in bytes
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)head_base<const T>(p.q, p.sq, hb, hh), (short)0, head_bytes<D>(Nq, p.sq), kBufferFlags);
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)head_base<const T>(p.k, p.sk, hb, hh), (short)0, head_bytes<D>(Nk, p.sk), kBufferFlags);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)head_base<const T>(p.v, p.sv, hb, hh), (short)0, head_bytes<D>(Nk, p.sv), kBufferFlags);

  const int q0 = qb * ROWS;
  const int kb = wave * 64;  // this wave's first key
  char* vreg = smem + wave * REGION;

  // ---- this wave's V tile (64 keys, rows past Nk read as zero) -> its LDS
  // region, rows in natural order, swizzled as in the tiled kernel: load i
  // fills 1 KB block i, slot sl = 64 i + lane is physical chunk sl % CPR of
  // row sl / CPR, which holds logical chunk (sl % CPR) ^ swizzle(row).
  {
    const uint32_t lds_v = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)vreg;
#pragma unroll
    for (int i = 0; i < CPR; ++i) {
      const int sl = i * 64 + lane;
      const int r = sl / CPR;
      const int ch = (f16_off<2 * D>(r, sl % CPR) - r * (2 * D)) >> 4;
      dma_to_lds(v_rsrc, __builtin_amdgcn_readfirstlane(lds_v + i * 1024),
                 (uint32_t)((kb + r) * vrs + 16 * ch));
    }
  }

  // ---- Q rows (B operands of block b: query q0 + 16b + x, d 32s + 8g ..
  // +7) and K rows (A operands of key block kb2: key kb + 16 kb2 + x, same
  // d), all issued before the first is used.
  u32x4 qw[QB][KS], kw[4][KS];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qw[b][s] = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, (q0 + 16 * b + x) * qrs + 2 * (32 * s + 8 * g),
                                                       0, 0);
#pragma unroll
  for (int kb2 = 0; kb2 < 4; ++kb2) {
    const int krow = kb + 16 * kb2 + x;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kw[kb2][s] = __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, krow * krs + 2 * (32 * s + 8 * g), 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  vec qf[QB][KS];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int e = 0; e < 4; ++e) qw[b][s][e] = (qw[b][s][e] & p.q_and) ^ p.q_xor;
      qf[b][s] = __builtin_bit_cast(vec, qw[b][s]);
    }
  // S^T = K Q^T: lane (x, g) holds keys kb + 16 kb2 + 4g + 0..3 of query
  // q0 + 16b + x; each K fragment serves the QB blocks
  f32x4 sacc[4][QB];
#pragma unroll
  for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const vec a = __builtin_bit_cast(vec, kw[kb2][s]);
#pragma unroll
      for (int b = 0; b < QB; ++b)
        sacc[kb2][b] = M::sel_sum(a, qf[b][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[kb2][b]);
    }

  // ---- mask (keys past Nk; causal: keys after the row), exact maximum of
  // the tile, P and its row sums
  const float c = p.c;
  const vec ones = M::selector(true);
  float m[QB], l[QB], l32[QB];
  vec pf[2][QB];  // P^T operands: key step cs, block b
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int q_row = q0 + 16 * b + x;
    int lim = CAUSAL ? (q_row + 1 < Nk ? q_row + 1 : Nk) : Nk;
    lim -= kb + 4 * g;
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[kb2][b][i] = (16 * kb2 + i < lim) ? sacc[kb2][b][i] : -__builtin_inff();
    float mb = sacc[0][b][0];
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
      for (int i = 0; i < 4; ++i) mb = vmax(mb, sacc[kb2][b][i]);
    mb = vmax(mb, __shfl_xor(mb, 16));
    mb = vmax(mb, __shfl_xor(mb, 32));
    mb *= c;                                      // c > 0 (the sign of the scale is carried by Q)
    const float negm = mb == -__builtin_inff() ? 0.f : -mb;  // a tile with no visible key: P = 0
    m[b] = mb;
    // the lane's own accumulators of key blocks 2cs and 2cs + 1, rounded in
    // pairs, are the P^T operand of key step cs
    float lsum = 0.f;
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
      u32x4 w;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[2 * cs + h][b][2 * i], c, negm));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[2 * cs + h][b][2 * i + 1], c, negm));
          lsum = M::lse_sum(p0, p1, lsum);
          w[2 * h + i] = __builtin_bit_cast(uint32_t, M::cvt(p0, p1));
        }
      pf[cs][b] = __builtin_bit_cast(vec, w);
    }
    // row sum of the rounded P against a matrix of ones (every lane of the
    // query gets it), and for bf16 the fp32 sum of the unrounded P (LSE)
    f32x4 racc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) racc = M::sel_sum(ones, pf[cs][b], racc);
    l[b] = racc[0];
    l32[b] = l[b];
    if constexpr (M::kLse32) {
      l32[b] = lsum + __shfl_xor(lsum, 16);
      l32[b] += __shfl_xor(l32[b], 32);
    }
  }

  // ---- O_w^T = V^T P^T. V^T operand of d block db, key step cs: lane x of
  // 16-lane group g points at key 32cs + 4g + x/4 (then 16 on), d columns
  // 16db + 4(x%4) .. +3, and receives 4 consecutive keys of d column 16db + x.
  wait_vmcnt<0>();  // this wave's V tile has landed (only this wave reads it)
  const int tr_row = 4 * g + (x >> 2);
  const int tr_col = 4 * (x & 3);
  f32x4 oacc[QB][NDB];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[b][db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int cs = 0; cs < 2; ++cs)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int row = tr_row + 32 * cs;
      const int col = tr_col + 16 * db;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vreg + f16_off<2 * D>(row, col >> 3) + 2 * (col & 7)));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vreg + f16_off<2 * D>(row + 16, col >> 3) + 2 * (col & 7)));
      const u32x2 wl = __builtin_bit_cast(u32x2, lo), wh = __builtin_bit_cast(u32x2, hi);
      const vec a = __builtin_bit_cast(vec, u32x4{wl[0], wl[1], wh[0], wh[1]});
#pragma unroll
      for (int b = 0; b < QB; ++b) oacc[b][db] = M::sel_sum(a, pf[cs][b], oacc[b][db]);
    }

  // ---- combine the waves. Each wave leaves its reference m_w (-inf for a
  // tile with no visible key), row sums (n_w of the rounded P, l_w for the
  // LSE) and unnormalised O_w (rows = queries) in its own LDS region; after
  // one barrier every thread merges, for its row and 4 columns,
  // M = max m_w, O = sum 2^(m_w - M) O_w / sum 2^(m_w - M) n_w and
  // LSE = ln2 (M + log2 sum 2^(m_w - M) l_w).
  if (g == 0) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      s_m[wave][16 * b + x] = m[b];
      s_l[wave][16 * b + x] = l[b];
      s_l32[wave][16 * b + x] = l32[b];
    }
  }
  // accumulator register i of d block db holds d column 16db + 4g + i of the
  // lane's query: one 16-byte store per block
  float* part = (float*)vreg;
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int db = 0; db < NDB; ++db) *(f32x4*)(part + (16 * b + x) * PS + 16 * db + 4 * g) = oacc[b][db];
  __syncthreads();

  // Thread e merges row e / (D/CW), columns CW*(e % (D/CW)) .. +CW-1: CW = 4
  // with one block, 8 with two, so one pass of the threads covers the rows.
  constexpr int CW = QB == 1 ? 4 : 8;
  T* Oh = head_base<T>(p.o, p.so, hb, hh);
  for (int e = tid; e < ROWS * D / CW; e += 64 * nw) {
    const int r = e / (D / CW), dc = CW * (e % (D / CW));
    if (q0 + r >= Nq) continue;
    float Mx = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < NWMAX; ++w)
      if (w < nw) Mx = vmax(Mx, s_m[w][r]);
    float acc[CW];
#pragma unroll
    for (int i = 0; i < CW; ++i) acc[i] = 0.f;
    float Ls = 0.f, L32 = 0.f;
#pragma unroll
    for (int w = 0; w < NWMAX; ++w) {
      if (w < nw) {
        const float mw = s_m[w][r];
        const float f = mw == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mw - Mx);
        const float* pw = (const float*)(smem + w * REGION) + r * PS + dc;
        Ls += f * s_l[w][r];
        L32 += f * s_l32[w][r];
#pragma unroll
        for (int h = 0; h < CW / 4; ++h) {
          const f32x4 xo = *(const f32x4*)(pw + 4 * h);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[4 * h + i] += f * xo[i];
        }
      }
    }
    const float inv = 1.0f / Ls;
    uint32_t ow[CW / 2];
#pragma unroll
    for (int i = 0; i < CW / 2; ++i) ow[i] = __builtin_bit_cast(uint32_t, M::cvt(acc[2 * i] * inv, acc[2 * i + 1] * inv));
    T* orow = Oh + (int64_t)(q0 + r) * p.so.n + dc;
    if constexpr (CW == 4) {
      *(u32x2*)orow = u32x2{ow[0], ow[1]};
    } else {
      *(u32x4*)orow = u32x4{ow[0], ow[1], ow[2], ow[3]};
    }
    if (p.lse != nullptr && dc == 0)
      p.lse[(size_t)head * Nq + q0 + r] = 0.69314718055994531f * (Mx + log2f(L32));
  }
}

}  // namespace fa
