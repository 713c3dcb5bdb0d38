// fa_fwd16.hpp - the tiled exact-attention forward on the 16x16x32 matrix
// instructions of gfx950 (v_mfma_f32_16x16x32_{f16,bf16}).
//
// Same method as fa_fwd_kernel.hpp (kwkr.cn YOLO11 FlashAttention-2 article,
// section 1.2; "FlashAttention 深度解读", section 原理 items 1-2): a workgroup
// owns a block of query rows of one head, streams the head's K and V through
// an LDS ring in tiles of 64 keys, forms the scores on the matrix cores, keeps
// a (lagging) reference maximum and the running sums, and accumulates P V in
// registers. What differs is the instruction shape, and with it every
// register layout. On this chip a kernel of nothing but 16x16x32 instructions
// retires about 15% more FLOP per second than one of 32x32x16 instructions
// (fewer accumulator registers per FLOP), and the layouts below need no key
// permutation, no selector matrix and fewer address registers.
//
// Layouts (lane l, x = l % 16, g = l / 16; a wave owns QB blocks of 16 query
// rows):
//   * S^T = K Q^T per 16-key block kb and 16-query block qb2: K rows are the A
//     operand (lane: key 16kb + x, d 32s + 8g .. +7 of k-step s, one 16-byte
//     LDS read), the wave's Q rows the B operand (lane: query 16qb2 + x, same
//     d), kept in VGPRs. The accumulator gives lane l keys 16kb + 4g + 0..3 of
//     query 16qb2 + x, so a query's 64 scores of a tile sit in the four lanes
//     x, x+16, x+32, x+48, sixteen each.
//   * P^T as the B operand of O^T += V^T P^T for the 32 keys of step c takes,
//     in k order, the lane's keys 32c + 4g + 0..3 (block 2c) and then
//     32c + 16 + 4g + 0..3 (block 2c+1): exactly the lane's own accumulator
//     registers, rounded in pairs. The V^T operand (lane: d row 16db + x, the
//     same 8 keys) comes from two ds_read_b64_tr_b16 reads of the V tile.
//   * The row sum of the rounded P is one 16x16x32 instruction per step
//     against a matrix of ones: every lane of the query gets the sum.
//   * K and V rows stay in natural order in LDS, swizzled (f16_off) so that
//     both the operand reads (one chunk of 16 consecutive rows per 16 lanes)
//     and the transpose reads (two chunks of 8 consecutive rows per 32 lanes)
//     are free of bank conflicts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fa_device.hpp"
#include "fa_fwd_kernel.hpp"

namespace fa {

// Byte offset of chunk c of row r in this kernel's K and V tiles: rows XOR-
// swizzled in 16-byte chunks so that neither read pattern meets a bank
// conflict on the 64 banks x 4 bytes of the LDS. A 16-byte read is served in
// four passes of 16 lanes, one lane of each residue mod 16 (within each half
// wave, the 4-lane blocks whose index has even parity form one pass, those
// with odd parity the other; measured lane pair by lane pair with
// SQ_LDS_BANK_CONFLICT on gfx950). In the K operand read (lane x + 16g: row
// x, chunk c + g) a pass thus reads 8 of the 16 rows at chunk c and the other
// 8 at chunk c + 1. The swizzle is even, so the two chunks never meet, and
// depends on row bits 0-2 (256- and 128-byte rows) or bit 2 (64-byte rows)
// only, which keeps the 8 rows of each chunk apart. The transpose reads
// (8 bytes, 32 lanes per pass: chunks c and c+1 of 8 consecutive rows) then
// also cover 16 distinct 16-byte bank groups.
template <int ROW_BYTES>
__device__ __forceinline__ int f16_off(int r, int c) {
  static_assert(ROW_BYTES == 64 || ROW_BYTES == 128 || ROW_BYTES == 256, "row size");
  int swz;
  if constexpr (ROW_BYTES == 256) swz = (r & 7) << 1;               // one row per 256 bytes
  else if constexpr (ROW_BYTES == 128) swz = ((r >> 1) & 3) << 1;   // two rows
  else swz = ((r >> 2) & 1) << 1;                                   // four rows
  return r * ROW_BYTES + 16 * (c ^ swz);
}

// One query block (head, qb) over the head's whole key range; strict as in
// fa_fwd_block (false: the optimistic pass, which returns false when the block
// must be redone with the tests).
template <int D, int NW, int QB, int S, bool CAUSAL, typename T>
__device__ __forceinline__ bool fa_fwd16_block(const Params& p, int head, int qb,
                                               char (&smem)[S][2][64 * D * 2], bool strict) {
  using M = Mma<T>;
  using vec = typename M::vec;
  constexpr int BN = 64;               // keys per tile
  constexpr int WR = 16 * QB;          // query rows per wave (QB blocks of 16)
  constexpr int BM = WR * NW;          // query rows per workgroup
  constexpr int NT = 64 * NW;          // threads per workgroup
  constexpr int KS = D / 32;           // k-steps of Q K^T
  constexpr int NDB = D / 16;          // 16-wide d blocks of O
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int CHUNKS = BN * CPR;
  constexpr int CPT = CHUNKS / NT;     // 16-byte chunks per thread per tensor
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int LOADS = 2 * CPT;
  // Loads left in flight at the end of tile j: tile j+1 must have landed.
  constexpr int PENDING = (S - 2) * LOADS;
  static_assert(CPT >= 1 && CPT * NT == CHUNKS, "tile must split evenly over threads");
  static_assert(S >= 2 && PENDING < 64, "stage count out of range");
  static_assert(BM % BN == 0, "a query block must cover whole key tiles");

  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // address arithmetic is redone in each pass
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int x = lane & 15;
  const int g = lane >> 4;

  const int Nq = p.Nq, Nk = p.Nk;
  const int hb = head / p.H, hh = head - hb * p.H;
  const int qrs = 2 * p.sq.n, krs = 2 * p.sk.n, vrs = 2 * p.sv.n;
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)head_base<const T>(p.q, p.sq, hb, hh), (short)0, head_bytes<D>(Nq, p.sq), kBufferFlags);
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)head_base<const T>(p.k, p.sk, hb, hh), (short)0, head_bytes<D>(Nk, p.sk), kBufferFlags);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)head_base<const T>(p.v, p.sv, hb, hh), (short)0, head_bytes<D>(Nk, p.sv), kBufferFlags);

  const int wave_q0 = qb * BM + wave * WR;

  // ---- Q as B operands: query 16*qb2 + x of the wave, d 32s + 8g .. +7
  vec qf[QB][KS];
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2) {
    const int row = wave_q0 + 16 * qb2 + x;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, row * qrs + 2 * (32 * s + 8 * g), 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (w[e] & p.q_and) ^ p.q_xor;
      qf[qb2][s] = __builtin_bit_cast(vec, w);
    }
  }

  int kv_end = Nk;
  if (CAUSAL) {
    const int last = qb * BM + BM;
    kv_end = last < Nk ? last : Nk;
  }
  const int t_lo = 0, t_hi = (kv_end + BN - 1) / BN;

  f32x4 oacc[QB][NDB];
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2)
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[qb2][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Per query block: the reference maximum (exp2 domain), the row sum of the
  // rounded P (the same in the query's four lanes) and, for bf16, this lane's
  // share of the fp32 sum of the unrounded P (its 16 keys of each tile).
  float m_run[QB], l_run[QB], l32_run[QB];
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2) {
    m_run[qb2] = -__builtin_inff();
    l_run[qb2] = 0.f;
    l32_run[qb2] = 0.f;
  }
  const vec ones = M::selector(true);
  const float c = p.c;

  // ---- tile loads (HBM -> LDS), rows in natural order: load i of this wave
  // fills 1 KB block wave*CPT + i; slot sl is physical chunk sl % CPR of row
  // sl / CPR, which holds logical chunk (sl % CPR) ^ swizzle(row).
  uint32_t k_goff[CPT], v_goff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int sl = (wave * CPT + i) * 64 + lane;
    const int r = sl / CPR;
    const int ch = (f16_off<2 * D>(r, sl % CPR) - r * (2 * D)) >> 4;
    k_goff[i] = r * krs + 16 * ch;
    v_goff[i] = r * vrs + 16 * ch;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  constexpr uint32_t kOutOfRange = 0x40000000u;  // tiles past the end load zeros
  auto issue = [&](int t, int st) {
    const uint32_t kbase = t < t_hi ? (uint32_t)(t * BN * krs) : kOutOfRange;
    const uint32_t vbase = t < t_hi ? (uint32_t)(t * BN * vrs) : kOutOfRange;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const uint32_t blk = (uint32_t)((wave * CPT + i) * 1024);
      dma_to_lds(k_rsrc, __builtin_amdgcn_readfirstlane(lds_base + (2 * st) * TILE_BYTES + blk),
                 k_goff[i] + kbase);
      dma_to_lds(v_rsrc, __builtin_amdgcn_readfirstlane(lds_base + (2 * st + 1) * TILE_BYTES + blk),
                 v_goff[i] + vbase);
    }
  };

  // K operand of key block kb, k-step s: row 16kb + x, chunk 4s + g. The
  // swizzle depends on row bits 0-2 only, so the key block is an offset.
  int k_roff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) k_roff[s] = f16_off<2 * D>(x, 4 * s + g);
  // V^T operand of d block db, key step cs: lane x of 16-lane group g points
  // at key 32cs + 4g + x/4 (then 16 on), d columns 16db + 4(x%4) .. +3, and
  // receives 4 consecutive keys of d column 16db + x.
  const int tr_row = 4 * g + (x >> 2);
  const int tr_col = 4 * (x & 3);
  auto vt_op = [&](const char* vs, int cs, int db) -> vec {
    const int row = tr_row + 32 * cs;
    const int col = tr_col + 16 * db;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(vs + f16_off<2 * D>(row, col >> 3) + 2 * (col & 7)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(vs + f16_off<2 * D>(row + 16, col >> 3) + 2 * (col & 7)));
    const u32x2 wl = __builtin_bit_cast(u32x2, lo), wh = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(vec, u32x4{wl[0], wl[1], wh[0], wh[1]});
  };

  f32x4 sacc[4][QB];   // scores: key block kb, query block qb2
  vec pf[2][QB];       // P^T operands: key step cs, query block qb2
  float psum[QB], ps32[QB];

  auto qk_step = [&](int st) {
    const char* ks = smem[st][0];
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const vec a = *(const vec*)(ks + k_roff[s] + kb * 16 * (2 * D));
#pragma unroll
        for (int qb2 = 0; qb2 < QB; ++qb2)
          sacc[kb][qb2] = M::sel_sum(a, qf[qb2][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[kb][qb2]);
      }
  };
  // keys past Nk and (causal) keys after the row -> -inf
  auto mask_tile = [&](int j) {
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2) {
      const int q_row = wave_q0 + 16 * qb2 + x;
      int lim = CAUSAL ? (q_row + 1 < Nk ? q_row + 1 : Nk) : Nk;
      lim -= j * BN + 4 * g;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sacc[kb][qb2][i] = (16 * kb + i < lim) ? sacc[kb][qb2][i] : -__builtin_inff();
    }
  };
  // P of query block qb2 against reference -negm: packed P^T operands, the
  // rounded row sum (matrix cores) and this lane's fp32 sum (bf16).
  auto exp_block = [&](int qb2, float negm) {
    float lsum = 0.f;
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
      u32x4 w;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[2 * cs + h][qb2][2 * i], c, negm));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[2 * cs + h][qb2][2 * i + 1], c, negm));
          lsum = M::lse_sum(p0, p1, lsum);
          w[2 * h + i] = __builtin_bit_cast(uint32_t, M::cvt(p0, p1));
        }
      pf[cs][qb2] = __builtin_bit_cast(vec, w);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) acc = M::sel_sum(ones, pf[cs][qb2], acc);
    psum[qb2] = acc[0];
    ps32[qb2] = lsum;
  };
  auto block_max = [&](int qb2) -> float {
    float m = sacc[0][qb2][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = vmax(m, sacc[kb][qb2][i]);
    m = vmax(m, __shfl_xor(m, 16));
    m = vmax(m, __shfl_xor(m, 32));
    return m * c;
  };
  auto raise_max = [&](int qb2, float mx) {
    float m_new = vmax(m_run[qb2], mx);
    m_new = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run[qb2] - m_new);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[qb2][db][i] *= alpha;
    l_run[qb2] *= alpha;
    l32_run[qb2] *= alpha;
    m_run[qb2] = m_new;
  };
  auto softmax_step = [&](auto mask_tag, int j) {
    if (decltype(mask_tag)::value) mask_tile(j);
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2) exp_block(qb2, -m_run[qb2]);
    bool ok = true;
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2) ok &= psum[qb2] <= kTileSumLimit;
    if ((strict || j == t_lo) && __any(!ok)) {
#pragma unroll
      for (int qb2 = 0; qb2 < QB; ++qb2) {
        raise_max(qb2, block_max(qb2));
        exp_block(qb2, -m_run[qb2]);
      }
    }
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2) {
      l_run[qb2] += psum[qb2];
      if constexpr (M::kLse32) l32_run[qb2] += ps32[qb2];
    }
  };
  auto pv_step = [&](int st) {
    const char* vs = smem[st][1];
#pragma unroll
    for (int cs = 0; cs < 2; ++cs)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const vec a = vt_op(vs, cs, db);
#pragma unroll
        for (int qb2 = 0; qb2 < QB; ++qb2) oacc[qb2][db] = M::sel_sum(a, pf[cs][qb2], oacc[qb2][db]);
      }
  };

  // P V of query block qb2 alone (its V^T operands read for it only)
  auto pv_block = [&](int st, int qb2) {
    const char* vs = smem[st][1];
#pragma unroll
    for (int cs = 0; cs < 2; ++cs)
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[qb2][db] = M::sel_sum(vt_op(vs, cs, db), pf[cs][qb2], oacc[qb2][db]);
  };
  int first_masked = (Nk % BN == 0) ? t_hi : Nk / BN;
  if (CAUSAL) {
    const int diag = (qb * BM) / BN;
    first_masked = diag < first_masked ? diag : first_masked;
  }
  first_masked = first_masked < t_hi ? first_masked : t_hi;

  // ---- prologue: tiles t_lo .. t_lo+S-2 requested, the first landed
#pragma unroll
  for (int t = 0; t < S - 1; ++t) issue(t_lo + t, t);
  wait_vmcnt<PENDING>();
  __syncthreads();

  auto beyond_rows = [&](int j) { return CAUSAL && j * BN > wave_q0 + WR - 1; };
  const auto unmasked = std::integral_constant<bool, false>{};
  const auto masked = std::integral_constant<bool, true>{};
  // Tile j sits in ring stage (j - t_lo) % S and requests tile j+S-1 into the
  // stage of tile j-1 (free since the last barrier).
  auto tile = [&](auto mask_tag, int j, int st) {
    issue(j + S - 1, (st + S - 1) % S);
    qk_step(st);
    softmax_step(mask_tag, j);
    pv_step(st);
    wait_vmcnt<PENDING>();
    __syncthreads();
  };
  // Unmasked tile of the optimistic pass after the first (no row-sum test),
  // d = 128: P V of query block q-1 is issued among the exponentials of
  // block q, so that one wave's matrix and vector instructions overlap (the
  // two waves of a SIMD run in lockstep there); the V^T operands are read
  // once per block instead of once for all blocks.
  auto tile_split = [&](int j, int st) {
    issue(j + S - 1, (st + S - 1) % S);
    qk_step(st);
    exp_block(0, -m_run[0]);
#pragma unroll
    for (int qb2 = 1; qb2 < QB; ++qb2) {
      pv_block(st, qb2 - 1);
      exp_block(qb2, -m_run[qb2]);
    }
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2) {
      l_run[qb2] += psum[qb2];
      if constexpr (M::kLse32) l32_run[qb2] += ps32[qb2];
    }
    pv_block(st, QB - 1);
    wait_vmcnt<PENDING>();
    __syncthreads();
  };
  auto stage = [&](int jj) { return (jj - t_lo) % S; };
  int j = t_lo;
  // d <= 64: unmasked tiles S at a time, so every ring stage is a constant
  // and the LDS operand addresses are per-lane bases plus immediates (at
  // d = 128 the bases do not fit beside the operands).
  if constexpr (D <= 64)
    for (; j + S <= first_masked; j += S)
      [&]<int... I>(std::integer_sequence<int, I...>) {
        (tile(unmasked, j + I, I), ...);
      }(std::make_integer_sequence<int, S>{});
  if constexpr (D == 128)
    if (!strict && j < first_masked) {
      tile(unmasked, j, stage(j));  // the first tile sets the reference maximum
      for (++j; j < first_masked; ++j) tile_split(j, stage(j));
    }
  for (; j < first_masked; ++j) tile(unmasked, j, stage(j));
  for (; j < t_hi && !beyond_rows(j); ++j) tile(masked, j, stage(j));
  for (; j < t_hi; ++j) {  // past this wave's rows: its share of loads and barriers
    issue(j + S - 1, stage(j + S - 1));
    wait_vmcnt<PENDING>();
    __syncthreads();
  }

  if (!strict) {
    // every row sum and output finite, or the workgroup redoes the block
    bool bad = false;
#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2) {
      float om = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) om = vmax(om, __builtin_fabsf(oacc[qb2][db][i]));
      const float l_tot = l_run[qb2] + (M::kLse32 ? l32_run[qb2] : 0.f);
      bad |= !(l_tot < __builtin_inff()) || !(om < __builtin_inff());
    }
    const int wave_bad = __any(bad) ? 1 : 0;
    wait_vmcnt<0>();
    __syncthreads();
    int* verdict = (int*)&smem[0][0][0];
    if (lane == 0) verdict[wave] = wave_bad;
    __syncthreads();
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any_bad |= verdict[w];
    if (any_bad) {
      __syncthreads();
      return false;
    }
  }

  // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l). Lane l holds d
  // 16db + 4g .. +3 of query 16qb2 + x.
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2) {
    const int q_row = wave_q0 + 16 * qb2 + x;
    float l_lse = l_run[qb2];
    if constexpr (M::kLse32) {
      l_lse = l32_run[qb2];
      l_lse += __shfl_xor(l_lse, 16);
      l_lse += __shfl_xor(l_lse, 32);
    }
    const float inv = 1.0f / l_run[qb2];
    if (q_row < Nq) {
      T* Oh = head_base<T>(p.o, p.so, hb, hh) + (int64_t)q_row * p.so.n;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        u32x2 w;
        w[0] = __builtin_bit_cast(uint32_t, M::cvt(oacc[qb2][db][0] * inv, oacc[qb2][db][1] * inv));
        w[1] = __builtin_bit_cast(uint32_t, M::cvt(oacc[qb2][db][2] * inv, oacc[qb2][db][3] * inv));
        *(u32x2*)(Oh + 16 * db + 4 * g) = w;
      }
      if (p.lse != nullptr && g == 0)
        p.lse[(size_t)head * Nq + q_row] = 0.69314718055994531f * (m_run[qb2] + log2f(l_lse));
    }
  }
  return true;
}

// Waves per SIMD the register allocation must allow: one 8-wave workgroup per
// CU at d = 128, three (d = 64) or four (d = 32) 4-wave workgroups.
#ifndef FA_FWD16_MIN_WAVES_D64
#define FA_FWD16_MIN_WAVES_D64 3
#endif
#ifndef FA_FWD16_MIN_WAVES_D32
#define FA_FWD16_MIN_WAVES_D32 4
#endif
constexpr int fwd16_min_waves(int d, int qb) {
  return d == 128 ? 1 : (d == 64 ? FA_FWD16_MIN_WAVES_D64 : (qb > 2 ? 2 : FA_FWD16_MIN_WAVES_D32));
}

template <int D, int NW, int QB, int S, bool CAUSAL, typename T>
__global__ __launch_bounds__(NW * 64, fwd16_min_waves(D, QB)) void fa_fwd16_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) char smem[S][2][64 * D * 2];
  int head, qb;
  work_item<CAUSAL>(p, blockIdx.x, head, qb);
  // the optimistic pass, then (rarely) the strict one
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass)
    if (fa_fwd16_block<D, NW, QB, S, CAUSAL, T>(p, head, qb, smem, pass == 1)) break;
}

}  // namespace fa
