// fa_fwd_fp8.hpp - the exact-attention forward on FP8 (e4m3) Q, K, V for gfx950.
//
// The cited articles name FP8 as one of FlashAttention-3's additions (ai2ai.xin
// flash-attention-principle page, FA-3 section). Q, K and V arrive as e4m3
// bytes with one fp32 dequantisation factor per tensor; the products run on
// v_mfma_scale_f32_32x32x64_f8f6f4 (64-deep contraction, twice the fp16
// rate) with fp32 accumulation, and O is written as fp16 or bf16.
//
// Same tiling as the fp16/bf16 forward (one workgroup per 32*NW query rows,
// K/V tiles of 64 keys streamed HBM -> LDS through an S-stage ring, S^T = K Q^T
// with K rows permuted so accumulator register i of lane l holds key
// 16*(l/32) + i, O^T += V^T P^T with V^T transposed once per tile), with
// these differences:
//   * An operand is 32 bytes per lane. For a 64-deep k-step the lane with
//     l/32 = h supplies bytes whose k slots the hardware pairs by (h, byte):
//     A and B only have to put the same contraction index at the same (h,
//     byte). Q K^T takes d = 64s + 32h .. +31 in both; P V takes the lane's
//     own 32 keys (16h + 0..15 of each 32-key unit) in both.
//   * The reference maximum is the exact running maximum (the row maximum of
//     each tile is taken), and P is formed as 2^(s*c - m + 8) <= 256 before
//     rounding to e4m3: every weight down to 2^-14 of the row maximum is then a
//     normal e4m3 number (3 mantissa bits), and none can reach the e4m3
//     maximum of 448. The row sum is taken in fp32 from the unrounded P;
//     the factor 2^8 cancels in O = acc / l and is taken out of the LSE.
//   * V^T comes from ds_read_b64_tr_b8: lane x of a 16-lane group points at
//     row k0 + x/2, bytes 8*(x%2) of a 16-byte column block and receives
//     rows k0..k0+7 of column x, stored as one 8-byte run of V^T row x.
//   * d = 32 fills half of the 64-deep Q K^T step: the lanes of the second
//     half (h = 1) supply zeros for both operands, so their products add
//     nothing. A 2 KB K (or V) tile is 128 chunks of 16 bytes, so the first
//     half of the waves loads K and the second half V.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fa_device.hpp"
#include "fa_fwd_kernel.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

struct Fp8Params {
  Params b;     // shapes, pointers, work split, c, q_and/q_xor (per byte)
  float v_scale;  // V's dequantisation factor, applied to O
};

// O^T or S^T += A B for e4m3 operands (format code 0 for A and B, unit
// block scales: exponent 127 means 2^0).
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
  i32x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (int)lo[e];
    r[4 + e] = (int)hi[e];
  }
  return r;
}

template <int D, int NW, int S, bool CAUSAL, typename TO>
__global__ __launch_bounds__(NW * 64) void fa_fwd_fp8_kernel(Fp8Params pp) {
  const Params& p = pp.b;
  using MO = Mma<TO>;
  constexpr int BN = 64;                     // keys per tile (two 32-key units)
  constexpr int BM = 32 * NW;                // query rows per workgroup
  constexpr int NT = 64 * NW;
  constexpr int KS = D >= 64 ? D / 64 : 1;   // 64-deep k-steps of Q K^T
  constexpr bool HALF_K = D == 32;            // d = 32: lanes h = 1 supply zeros
  constexpr int NDT = D / 32;                // 32-wide d tiles of O
  constexpr int CPR = D / 16;                // 16-byte chunks per K/V row
  constexpr int TILE = BN * D;               // bytes of a K (or V) tile
  // HBM->LDS loads per thread per tensor; d = 32: K by the first NW/2 waves,
  // V by the others, one load each per tile
  constexpr bool SPLIT = TILE / 16 < NT;
  constexpr int CPT = SPLIT ? 1 : TILE / 16 / NT;
  constexpr int LOADS = SPLIT ? 1 : 2 * CPT;
  constexpr int TBLK = (BN / 8) * (D / 16);  // 8-key x 16-column transpose blocks
  constexpr int TPW = TBLK / (4 * NW);       // transpose reads per wave per tile
  constexpr int PENDING = (S - 3) * LOADS;
  static_assert(D == 32 || D == 64 || D == 128, "fp8 path: d = 32, 64 or 128");
  static_assert(SPLIT ? TILE / 16 * 2 == NT : CPT * NT * 16 == TILE, "tile must split evenly over threads");
  static_assert(TPW >= 1 && TPW * 4 * NW == TBLK, "V transpose must split evenly over waves");
  static_assert(S >= 3 && PENDING < 64, "stage count out of range");

  __shared__ __attribute__((aligned(1024))) char smem[S][2][TILE];
  __shared__ __attribute__((aligned(1024))) char vts[2][TILE];  // V^T: D rows of BN bytes

  int head, qb;
  work_item<CAUSAL>(p, blockIdx.x, head, qb);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int r32 = lane & 31;
  const int Nq = p.Nq, Nk = p.Nk;
  const size_t q_head = (size_t)head * Nq * D;
  const size_t kv_head = (size_t)head * Nk * D;
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)p.q + q_head), (short)0, Nq * D, kBufferFlags);
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)p.k + kv_head), (short)0, Nk * D, kBufferFlags);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint8_t*)p.v + kv_head), (short)0, Nk * D, kBufferFlags);

  const int q_row = qb * BM + 32 * wave + r32;

  // ---- the lane's query row as B operands: d = 64s + 32h .. +31
  i32x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    // d = 32: the second lane half's d range (32..63) is past the row; it
    // reads the next row's bytes and is zeroed (q_and/q_xor masks below)
    u32x4 w0 = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, q_row * D + 64 * s + 32 * half, 0, 0);
    u32x4 w1 = __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, q_row * D + 64 * s + 32 * half + 16, 0, 0);
    const uint32_t keep = (HALF_K && half) ? 0u : 0xffffffffu;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w0[e] = ((w0[e] & p.q_and) ^ p.q_xor) & keep;
      w1[e] = ((w1[e] & p.q_and) ^ p.q_xor) & keep;
    }
    qf[s] = join(w0, w1);
  }

  int kv_end = Nk;
  if (CAUSAL) {
    const int last = qb * BM + BM;
    kv_end = last < Nk ? last : Nk;
  }
  const int ntiles = (kv_end + BN - 1) / BN;
  int first_masked = (Nk % BN == 0) ? ntiles : Nk / BN;
  if (CAUSAL) {
    const int diag = (qb * BM) / BN;
    first_masked = diag < first_masked ? diag : first_masked;
  }
  first_masked = first_masked < ntiles ? first_masked : ntiles;

  f32x16 oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[t][i] = 0.f;
  float m_run = -__builtin_inff();  // exact running maximum (exp2 domain)
  float l_run = 0.f;                // this lane's half of the row sum of 2^8 P
  const float c = p.c;

  // ---- HBM -> LDS (K rows permuted, V rows natural)
  uint32_t k_goff[CPT], v_goff[CPT];
  const int lwave = SPLIT ? wave % (NW / 2) : wave;  // the wave's block within its tensor
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int sl = (lwave * CPT + i) * 64 + lane;
    const int r = sl / CPR;
    const int ch = (lds_off<D>(r, sl % CPR) - r * D) >> 4;
    const int kkey = (r & ~31) | lds_row_to_key(r & 31);
    k_goff[i] = kkey * D + 16 * ch;
    v_goff[i] = r * D + 16 * ch;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&smem[0][0][0];
  constexpr uint32_t kOutOfRange = 0x40000000u;
  auto issue = [&](int t, int st) {  // tile t into ring stage st (= t % S)
    const uint32_t gb = t < ntiles ? (uint32_t)(t * TILE) : kOutOfRange;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const uint32_t blk = (uint32_t)((lwave * CPT + i) * 1024);
      if (!SPLIT || wave < NW / 2)
        dma_to_lds(k_rsrc, __builtin_amdgcn_readfirstlane(lds_base + (2 * st) * TILE + blk), k_goff[i] + gb);
      if (!SPLIT || wave >= NW / 2)
        dma_to_lds(v_rsrc, __builtin_amdgcn_readfirstlane(lds_base + (2 * st + 1) * TILE + blk), v_goff[i] + gb);
    }
  };

  // ---- V tile -> V^T (8 keys x 16 columns per 16-lane group)
  int tr_src[TPW], tr_dst[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int G = (wave * TPW + i) * 4 + (lane >> 4);
    const int k0 = 8 * (G % (BN / 8));
    const int d0 = 16 * (G / (BN / 8));
    const int x = lane & 15;
    tr_src[i] = lds_off<D>(k0 + (x >> 1), d0 >> 4) + 8 * (x & 1);
    tr_dst[i] = lds_off<BN>(d0 + x, k0 >> 4) + (k0 & 15);
  }
  auto transpose_v = [&](int j, int st) {  // tile j, in ring stage st
    const char* src = smem[st][1];
    char* dst = vts[j & 1];
    i32x2 blk[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) blk[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(src + tr_src[i]));
#pragma unroll
    for (int i = 0; i < TPW; ++i) *(i32x2*)(dst + tr_dst[i]) = blk[i];
  };

  // LDS operand offsets: K rows (unit t, k-step s: chunks 4s + 2h, +1) and
  // V^T rows (d tile dt: keys 16h.. of unit 0 and 32 + 16h.. of unit 1).
  int k_off[2][KS];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < KS; ++s) k_off[t][s] = lds_off<D>(32 * t + r32, 4 * s + 2 * half);
  int k_off2[2][KS];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < KS; ++s) k_off2[t][s] = lds_off<D>(32 * t + r32, 4 * s + 2 * half + 1);
  int v_off[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int t = 0; t < 2; ++t) v_off[dt][t] = lds_off<BN>(32 * dt + r32, 2 * t + half);

  auto tile = [&](auto mask_tag, int j, int st) {  // tile j, in ring stage st
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* ks = smem[st][0];
    const char* vt = vts[j & 1];
    f32x16 sacc[2];
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        // d = 32: the second lane half has no K bytes (its Q half is zero)
        const i32x8 a = (HALF_K && half) ? i32x8{}
                                         : join(*(const u32x4*)(ks + k_off[t][s]), *(const u32x4*)(ks + k_off2[t][s]));
        sacc[t] = mfma_fp8(a, qf[s], s == 0 ? f32x16{} : sacc[t]);
      }
    if (MASK) {
      int lim = CAUSAL ? (q_row + 1 < Nk ? q_row + 1 : Nk) : Nk;
      lim -= j * BN + 16 * half;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[t][i] = (i + 32 * t < lim) ? sacc[t][i] : -__builtin_inff();
    }
    // exact row maximum of the tile (both lanes of the row), exp2 domain
    float m4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) m4[e] = vmax(sacc[0][e], sacc[1][e]);
#pragma unroll
    for (int i = 4; i < 16; ++i) m4[i & 3] = vmax(m4[i & 3], vmax(sacc[0][i], sacc[1][i]));
    const float mx = max_with_partner(vmax(vmax(m4[0], m4[1]), vmax(m4[2], m4[3]))) * c;
    if (__any(mx > m_run)) {
      float m_new = vmax(m_run, mx);
      m_new = (m_new == -__builtin_inff()) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    // P' = 2^(s*c - m + 8) in (0, 256], rounded to e4m3 as the B operand:
    // byte j of the lane holds key 32*(j/16) + 16h + j%16
    const float negm = 8.0f - m_run;
    float lsum = 0.f;
    i32x8 pb;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int t = w >> 2, i0 = 4 * (w & 3);
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i0 + 0], c, negm));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i0 + 1], c, negm));
      const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i0 + 2], c, negm));
      const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i0 + 3], c, negm));
      lsum += (p0 + p1) + (p2 + p3);
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
      pb[w] = word;
    }
    l_run += lsum;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const i32x8 a = join(*(const u32x4*)(vt + v_off[dt][0]), *(const u32x4*)(vt + v_off[dt][1]));
      oacc[dt] = mfma_fp8(a, pb, oacc[dt]);
    }
  };

  // prologue: tiles 0..S-2 requested, V^T of tile 0 written
#pragma unroll
  for (int t = 0; t < S - 1; ++t) issue(t, t);
  wait_vmcnt<PENDING>();
  __syncthreads();
  transpose_v(0, 0);
  __syncthreads();
  const auto unmasked = std::integral_constant<bool, false>{};
  const auto masked = std::integral_constant<bool, true>{};
  // Step j (tile j in ring stage st = j % S): request tile j+S-1 into the
  // stage of tile j-1, transpose tile j+1, compute tile j, wait for the next
  // tile and meet at the barrier.
  auto step = [&](auto mask_tag, int j, int st) {
    issue(j + S - 1, (st + S - 1) % S);
    transpose_v(j + 1, (st + 1) % S);
    tile(mask_tag, j, st);
    wait_vmcnt<PENDING>();
    __syncthreads();
  };
  int j = 0;
  // Unmasked tiles S at a time: the ring stages (and V^T buffers) are
  // constants, so LDS operand addresses are per-lane bases plus immediates.
  for (; j + S <= first_masked; j += S)
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (step(unmasked, j + I, I), ...);
    }(std::make_integer_sequence<int, S>{});
  for (; j < first_masked; ++j) step(unmasked, j, j % S);
  // Causal: tiles whose first key comes after this wave's last row add
  // nothing to its rows; the wave only takes its share of their loads,
  // transposes and barriers.
  const int wave_last_row = qb * BM + 32 * wave + 31;
  for (; j < ntiles && !(CAUSAL && j * BN > wave_last_row); ++j) step(masked, j, j % S);
  for (; j < ntiles; ++j) {
    issue(j + S - 1, (j + S - 1) % S);
    transpose_v(j + 1, (j + 1) % S);
    wait_vmcnt<PENDING>();
    __syncthreads();
  }

  // ---- epilogue: O = v_scale * acc / l, LSE = ln2 * (m - 8 + log2 l)
  const float l_tot = sum_with_partner(l_run);
  if (q_row < Nq) {
    const float f = pp.v_scale / l_tot;
    TO* Oh = (TO*)p.o + q_head + (size_t)q_row * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = __builtin_bit_cast(uint32_t, MO::cvt(oacc[dt][4 * g + 0] * f, oacc[dt][4 * g + 1] * f));
        w[1] = __builtin_bit_cast(uint32_t, MO::cvt(oacc[dt][4 * g + 2] * f, oacc[dt][4 * g + 3] * f));
        *(u32x2*)(Oh + 32 * dt + 8 * g + 4 * half) = w;
      }
    if (p.lse != nullptr && half == 0)
      p.lse[(size_t)head * Nq + q_row] = 0.69314718055994531f * (m_run - 8.0f + log2f(l_tot));
  }
}

}  // namespace fa
