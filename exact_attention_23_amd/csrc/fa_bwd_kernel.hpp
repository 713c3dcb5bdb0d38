// fa_bwd_kernel.hpp - the exact-attention backward kernels for gfx950 (CDNA4).
//
// What is computed (the chain rule of the forward definition; the cited articles say
// training keeps the softmax statistics for the backward pass, kwkr.cn YOLO11
// FlashAttention-2 article, section 2.3, and that the backward recomputes the
// weights instead of storing them, "YOLOv12推理速度翻倍秘诀：Flash Attention加持",
// section 1):
//     P = exp(scale * Q K^T - LSE)   rebuilt per tile from the forward's LSE
//     dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
//     dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q
//
// Three kernels, no atomics (every output element is summed in a fixed order):
//   * fa_bwd_pre_kernel: per query row, -D_i and LSE_i * log2(e) into a
//     workspace of 32-row records (rows past Nq get +inf and 0, so that they
//     produce P = 0 downstream without any row masking). The dP products start
//     their accumulation from -D, so dP - D costs no vector instruction.
//   * fa_bwd_dkdv_kernel: one workgroup per block of BN = 32*NW keys; wave w
//     owns 32 keys and keeps their K and V rows in VGPRs as MFMA B operands.
//     It walks the head's query rows in tiles of 32 and accumulates dK and dV
//     in fp32 MFMA accumulators for the whole walk.
//   * fa_bwd_dq_kernel: one workgroup per block of 32*NW query rows, wave w
//     owns 32 rows; it walks the keys in tiles of 64 like the forward and
//     accumulates dQ. It recomputes S and dP (two of the five products once
//     more), which is what removes the atomics a single-pass dQ would need.
//
// gfx950 mapping of the dK/dV kernel, per query tile of 32 rows:
//   * S = Q K^T and dP = dO V^T with v_mfma_f32_32x32x16: the Q (dO) rows are
//     the A operand (16-byte LDS reads of the staged tile), the wave's K (V)
//     rows the B operand from VGPRs. In the accumulator lane l holds key l%32
//     and 16 queries, register i holding query 8(i/4) + 4(l/32) + i%4.
//   * Those registers, rounded in pairs, are directly the A operand (P^T,
//     dS^T: row = key, k = 8 queries) of dV += P^T dO and dK += dS^T Q, with
//     the queries of a k-step taken in that register order. The B operands
//     (dO and Q with the queries along k) come from ds_read_b64_tr_b16
//     transpose reads. At d <= 64 they are read straight from the staged
//     tiles (two transpose reads per operand, each handing a lane 4
//     consecutive queries of its d column). At d = 128, where the direct
//     reads' addresses do not fit in the registers beside the operands,
//     they come from transposed copies, Q^T and dO^T, written once per
//     workgroup per tile, one tile ahead; inside each group of 16 queries the
//     copies store the queries in the order 0-3, 8-11, 4-7, 12-15 (bits 2
//     and 3 swapped), so a lane's eight queries are one 16-byte run.
//   * LSE and D of the 16 queries of a lane are four 16-byte LDS reads each
//     (the lanes of a half read the same address).
//   * Q, dO and the workspace records go HBM -> LDS by buffer_load ... lds
//     through a ring of S stages, as in the forward.
// The dQ kernel is the forward's structure with a different per-unit body:
// S^T = K Q^T and dP^T = V dO^T (K and V rows as A operands from LDS in the
// permuted key order, Q and dO of the wave's rows as B operands in VGPRs),
// then dQ^T += K^T dS^T with dS^T straight from the accumulator registers and
// the K^T operand, like the B operands above, read straight from the K tile
// at d <= 64 and from a copy transposed once per tile at d = 128. Tiles that
// are read directly use the forward's swizzle (tile_off), under which both
// the operand reads and the transpose reads are free of bank conflicts; the
// copy path keeps lds_off, which suits its transposes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fa_device.hpp"

namespace fa {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* aux;    // [B*H][nrec][2][32] fp32: LSE*log2(e) (+inf past Nq), -D (0 past Nq)
  int B, H, Nq, Nk;
  int nrec;      // 32-row records per head: ceil(Nq / 32)
  int nblk;      // blocks per head (key blocks for dK/dV, query blocks for dQ)
  int xcd_q;     // workgroups / 8
  int xcd_r;     // workgroups % 8
  int group;     // heads per scheduling group
  int launch_order;  // nonzero: logical id = workgroup id (no per-XCD ranges)
  float c;       // scale * log2(e)
  float scale;
};

constexpr float kLog2e = 1.4426950408889634f;

// Workgroup id -> (head, block), with the same XCD-contiguous remap (or launch
// order) and head groups as the forward. DESC walks the blocks of a head from the last one (the heaviest
// for causal dQ, whose late query blocks see the most keys); ascending order
// puts the heaviest causal dK/dV blocks (early keys) first.
template <bool DESC>
__device__ __forceinline__ void bwd_work_item(const BwdParams& p, int bid, int& head, int& blk) {
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int L = p.launch_order ? bid : xcd * p.xcd_q + (xcd < p.xcd_r ? xcd : p.xcd_r) + slot;
  const int per_group = p.group * p.nblk;
  const int grp = L / per_group;
  const int rem = L - grp * per_group;
  const int heads_total = p.B * p.H;
  int hig = heads_total - grp * p.group;
  hig = hig < p.group ? hig : p.group;
  const int rank = rem / hig;
  head = grp * p.group + (rem - rank * hig);
  blk = DESC ? (p.nblk - 1 - rank) : rank;
}

// ---------------------------------------------------------------------------
// -D_i = -sum_c dO_ic O_ic and LSE_i * log2(e), per query row, into 32-row
// records. D/8 threads share a row, 16 bytes of O and dO each.
template <int D, typename T>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(BwdParams p) {
  using vec = typename Mma<T>::vec;
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int npad = p.nrec * 32;
  const int64_t rows = (int64_t)p.B * p.H * npad;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int sub = threadIdx.x % TPR;
  const bool in = r < rows;
  int head = 0, row = 0;
  if (in) {
    head = (int)(r / npad);
    row = (int)(r - (int64_t)head * npad);
  }
  const bool valid = in && row < p.Nq;
  float acc = 0.f;
  if (valid) {
    const size_t off = ((size_t)head * p.Nq + row) * D + 8 * sub;
    const f32x8 a = __builtin_convertvector(*(const vec*)((const T*)p.o + off), f32x8);
    const f32x8 b = __builtin_convertvector(*(const vec*)((const T*)p.dout + off), f32x8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(a[e], b[e], acc);
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (in && sub == 0) {
    float* rec = p.aux + ((size_t)head * p.nrec + (row >> 5)) * 64 + (row & 31);
    rec[0] = valid ? p.lse[(size_t)head * p.Nq + row] * kLog2e : __builtin_inff();
    rec[32] = valid ? -acc : 0.f;
  }
}

// ---------------------------------------------------------------------------
// dK and dV for one block of 32*NW keys.
// K rows of the dK/dV kernel in LDS at d = 128 (1) or in VGPRs (0).
#ifndef FA_BWD_K_LDS
#define FA_BWD_K_LDS 1
#endif

// Waves per SIMD the backward kernels are compiled for (register budget).
// d = 32 dQ: capped at four waves (128 registers; it takes about 100). (d = 64 dK/dV capped at three waves ran 2-3% faster but
// its 11 spilled registers added 40% to its HBM traffic; it is not capped.)
constexpr int bwd_dkdv_min_waves(int) { return 1; }
constexpr int bwd_dq_min_waves(int d) { return d == 32 ? 4 : 1; }

template <int D, int NW, int S, bool CAUSAL, typename T>
__global__ __launch_bounds__(NW * 64, bwd_dkdv_min_waves(D)) void fa_bwd_dkdv_kernel(BwdParams p) {
  using M = Mma<T>;
  using vec = typename M::vec;
  constexpr int BM = 32;                     // query rows per tile
  constexpr int BN = 32 * NW;                // keys per workgroup
  constexpr int NT = 64 * NW;
  constexpr int KS = D / 16;                 // k-steps over d
  constexpr int NDT = D / 32;                // 32-wide d tiles of dK, dV
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int TILE = BM * D * 2;           // bytes of a Q (or dO) tile
  constexpr int CPT = 2 * TILE / 16 / NT;    // HBM->LDS loads per thread for Q and dO
  constexpr int AUXB = BM * 8;               // bytes of a tile's LSE and D
  constexpr int AUX_LANES = AUXB / 16 / NW;  // lanes per wave loading them
  constexpr int LOADS = CPT + 1;             // loads per wave per tile
  constexpr bool DIRECT = D <= 64;           // B operands straight from the staged tiles
  constexpr int TBLK = (BM / 4) * (D / 16);  // copy path: 4-row x 16-column blocks per tensor
  constexpr int TPW = 2 * TBLK / (4 * NW);   // copy path: transpose reads per wave per tile
  // Loads left in flight at the end of step j: tile j+1 must have landed
  // (the copy path transposes tile j+1 during step j, so tile j+2 there).
  constexpr int PENDING = (S - (DIRECT ? 2 : 3)) * LOADS;
  static_assert(CPT >= 1 && CPT * NT * 16 == 2 * TILE, "Q and dO tiles must split over threads");
  static_assert(TILE % 1024 == 0, "a 1 KB load block must not straddle Q and dO");
  static_assert(AUX_LANES >= 1 && AUX_LANES * 16 * NW == AUXB, "records must split over waves");
  static_assert(DIRECT || (TPW >= 1 && TPW * 4 * NW == 2 * TBLK), "transposes must split over waves");
  static_assert(DIRECT || TBLK % 4 == 0, "a wave's transpose groups must stay in one tensor");
  static_assert(PENDING >= 0 && PENDING < 64, "stage count out of range");
  auto toff = [](int r, int c) { return DIRECT ? tile_off<2 * D>(r, c) : lds_off<2 * D>(r, c); };

  // Staged tiles ([stage][Q, dO], rows = queries), the copy path's
  // transposes ([parity][Q^T, dO^T], rows = d columns of 32 queries) and the
  // records.
  __shared__ __attribute__((aligned(1024))) char ring[S][2][TILE];
  __shared__ __attribute__((aligned(1024))) char trb[DIRECT ? 1 : 2][2][DIRECT ? 16 : TILE];
  __shared__ __attribute__((aligned(16))) float auxs[S][2 * BM];
  // At d = 128 the wave's K rows live in LDS instead of VGPRs (the registers
  // are full there); each wave reads back only its own 32 rows.
  constexpr bool K_LDS = FA_BWD_K_LDS && D == 128;
  __shared__ __attribute__((aligned(1024))) char kls[K_LDS ? 32 * NW : 1][K_LDS ? 2 * D : 16];
  // At d = 64 a tile computes P, and its dV products, before dP - D: the
  // exponentials then overlap matrix work of the same wave (2.5% faster
  // there; at d = 32 and 128 it ran slower, and at 128 it spills).
  constexpr bool P_FIRST = D == 64;

  int head, kb;
  bwd_work_item<false>(p, blockIdx.x, head, kb);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int r32 = lane & 31;
  const int Nq = p.Nq, Nk = p.Nk;
  const float c = p.c;
  const size_t q_head = (size_t)head * Nq * D;
  const size_t kv_head = (size_t)head * Nk * D;
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.q + q_head), (short)0, Nq * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t do_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.dout + q_head), (short)0, Nq * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.k + kv_head), (short)0, Nk * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.v + kv_head), (short)0, Nk * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t aux_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.aux + (size_t)head * p.nrec * 64), (short)0, p.nrec * 256, kBufferFlags);

  const int n0 = kb * BN;
  const int kw0 = n0 + 32 * wave;  // first key of this wave
  const int key = kw0 + r32;       // this lane's key (keys past Nk read as zero)

  // K and V rows of the lane's key: B operands of S = Q K^T and dP = dO V^T.
  vec kf[K_LDS ? 1 : KS], vf[KS];
  int k_off[K_LDS ? KS : 1];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int off = key * (2 * D) + 2 * (16 * s + 8 * half);
    const vec kv = __builtin_bit_cast(vec, __builtin_amdgcn_raw_buffer_load_b128(k_rsrc, off, 0, 0));
    if constexpr (K_LDS) {
      k_off[s] = lds_off<2 * D>(32 * wave + r32, 2 * s + half);
      *(vec*)(&kls[0][0] + k_off[s]) = kv;  // read back by this lane only
    } else {
      kf[s] = kv;
    }
    vf[s] = __builtin_bit_cast(vec, __builtin_amdgcn_raw_buffer_load_b128(v_rsrc, off, 0, 0));
  }

  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk[t][i] = 0.f;
      dv[t][i] = 0.f;
    }

  // Query tiles: causal rows below n0 see none of these keys.
  const int ntq = (Nq + BM - 1) / BM;
  const int t0 = CAUSAL ? (n0 / BM < ntq ? n0 / BM : ntq) : 0;
  const int ntiles = ntq - t0;
  // Tiles before first_free need the mask: all of them when the block holds
  // keys past Nk, and (causal) those holding a row below the block's last key.
  int first_free = 0;
  if (CAUSAL) {
    const int need = n0 + BN - 1 - t0 * BM;  // rows i < n0+BN-1 see only part of the block
    first_free = need > 0 ? (need + BM - 1) / BM : 0;
  }
  if (n0 + BN > Nk) first_free = ntiles;
  first_free = first_free < ntiles ? first_free : ntiles;

  // ---- HBM -> LDS loads. Load i of this wave fills 1 KB block wave*CPT + i of
  // the [Q | dO] stage; slot sl of a tensor is physical chunk sl % CPR of row
  // sl / CPR, which holds logical chunk (sl % CPR) ^ swizzle(row).
  uint32_t goff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int blk = wave * CPT + i;
    const int tensor = (blk * 1024) / TILE;
    const int sl = (blk * 1024 - tensor * TILE) / 16 + lane;
    const int r = sl / CPR;
    const int ch = (toff(r, sl % CPR) - r * (2 * D)) >> 4;
    goff[i] = r * (2 * D) + 16 * ch;
  }
  const uint32_t lds_ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&ring[0][0][0];
  const uint32_t lds_aux = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&auxs[0][0];
  constexpr uint32_t kOutOfRange = 0x40000000u;
  auto issue = [&](int j, int st) {  // tile j into ring stage st (= j % S)
    const bool live = j < ntiles;
    const uint32_t gb = live ? (uint32_t)((t0 + j) * TILE) : kOutOfRange;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int blk = wave * CPT + i;
      const int tensor = (blk * 1024) / TILE;
      dma_to_lds(tensor ? do_rsrc : q_rsrc,
                 __builtin_amdgcn_readfirstlane(lds_ring + st * (2 * TILE) + blk * 1024), goff[i] + gb);
    }
    const uint32_t ab = live ? (uint32_t)((t0 + j) * AUXB) : kOutOfRange;
    if (lane < AUX_LANES)
      dma_to_lds(aux_rsrc, __builtin_amdgcn_readfirstlane(lds_aux + st * AUXB + wave * (AUX_LANES * 16)),
                 ab + wave * (AUX_LANES * 16) + 16 * lane);
  };

  // ---- copy path: transposes of a staged tile into Q^T / dO^T. Transpose
  // read i of this wave covers, in 16-lane group G, rows q0..q0+3 and columns
  // d0..d0+15 of one tensor; lane x points at row q0 + x/4, columns
  // d0 + 4(x%4) .. +3, receives rows q0..q0+3 of column d0 + x and stores
  // them as one 8-byte run of row d0 + x of the copy, at the position of q0
  // in the bit-2/3-swapped query order.
  int tr_src[DIRECT ? 1 : TPW], tr_dst[DIRECT ? 1 : TPW];
  if constexpr (!DIRECT) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int G = (wave * TPW + i) * 4 + (lane >> 4);
      const int tensor = G / TBLK;
      const int g = G - tensor * TBLK;
      const int q0 = 4 * (g % (BM / 4));
      const int d0 = 16 * (g / (BM / 4));
      const int x = lane & 15;
      const int col = d0 + 4 * (x & 3);
      tr_src[i] = tensor * TILE + lds_off<2 * D>(q0 + (x >> 2), col >> 3) + 2 * (col & 7);
      const int pos = (q0 & ~15) | (((q0 >> 3) & 1) << 2) | (((q0 >> 2) & 1) << 3);
      tr_dst[i] = tensor * TILE + lds_off<2 * BM>(d0 + x, pos >> 3) + 2 * (pos & 7);
    }
  }
  auto transpose = [&](int j) {
    if constexpr (!DIRECT) {
      const char* src = &ring[j % S][0][0];
      char* dst = &trb[j & 1][0][0];
      i16x4 blk[TPW];
#pragma unroll
      for (int i = 0; i < TPW; ++i)
        blk[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + tr_src[i]));
#pragma unroll
      for (int i = 0; i < TPW; ++i) *(i16x4*)(dst + tr_dst[i]) = blk[i];
    }
  };

  // LDS read offsets that do not depend on the tile.
  int a_off[KS];  // Q / dO rows as A operands: row r32, chunk 2s + half
#pragma unroll
  for (int s = 0; s < KS; ++s) a_off[s] = toff(r32, 2 * s + half);
  int b_off[NDT][2];  // copy path: Q^T / dO^T rows 32dt + r32, queries 16c2 + 8half ..
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) b_off[dt][c2] = lds_off<2 * BM>(32 * dt + r32, 2 * c2 + half);
  // Direct path: Q^T / dO^T B operand of d tile dt for k-step c2 (queries 16c2 + 4half +
  // 0..3, then 8 on: the order of the P^T / dS^T registers) straight from
  // the staged tile: two transpose reads, lane x of a 16-lane group pointing
  // at query 16c2 + 4half + x/4 (then + 8), columns d0 + 4(x%4) .. +3 with
  // d0 = 32dt + 16((lane/16)%2), and receiving 4 queries of column d0 + x.
  const int trx = lane & 15;
  const int tr_row = 4 * half + (trx >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (trx & 3);
  auto b_direct = [&](const char* src, int c2, int dt) -> vec {
    const int row = tr_row + 16 * c2;
    const int col = tr_col + 32 * dt;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(src + tile_off<2 * D>(row, col >> 3) + 2 * (col & 7)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(src + tile_off<2 * D>(row + 8, col >> 3) + 2 * (col & 7)));
    const u32x2 wl = __builtin_bit_cast(u32x2, lo), wh = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(vec, u32x4{wl[0], wl[1], wh[0], wh[1]});
  };

  // ---- one query tile
  auto tile = [&](auto mask_tag, int j, int st) {  // tile j, in ring stage st
    constexpr bool MASK = decltype(mask_tag)::value;
    const int i0 = (t0 + j) * BM;
    // Causal: a wave whose first key is after the tile's last row adds zeros.
    if (MASK && CAUSAL && kw0 > i0 + BM - 1) return;
    const char* qs = &ring[st][0][0];
    const char* dos = &ring[st][1][0];
    const float* ax = auxs[st];
    const char* qt = &trb[DIRECT ? 0 : (j & 1)][0][0];
    const char* dot = &trb[DIRECT ? 0 : (j & 1)][1][0];
    f32x16 sa, dpa;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const vec a = *(const vec*)(qs + a_off[s]);
      vec kb;
      if constexpr (K_LDS)
        kb = *(const vec*)(&kls[0][0] + k_off[s]);
      else
        kb = kf[s];
      sa = M::run(a, kb, s == 0 ? f32x16{} : sa);
    }
    if constexpr (P_FIRST) {
      // P first, four queries at a time (LSE*log2(e) of the lane's queries
      // 8a + 4half + 0..3), and dV += P^T dO from it, so that the vector work
      // of P and the matrix work of dP - D and dV can overlap in this wave
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 lz = *(const f32x4*)(ax + 8 * a + 4 * half);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 4 * a + b;
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[i], c, -lz[b]));
          if (MASK) {
            const int qi = i0 + 8 * a + 4 * half + b;
            const bool vis = key < Nk && (!CAUSAL || key <= qi);
            pv = vis ? pv : 0.f;
          }
          sa[i] = pv;
        }
      }
      vec pa[2], da[2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        u32x4 wp;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          wp[m] = __builtin_bit_cast(uint32_t, M::cvt(sa[8 * c2 + 2 * m], sa[8 * c2 + 2 * m + 1]));
        pa[c2] = __builtin_bit_cast(vec, wp);
      }
      // dP - D in one chain: the first dP MFMA starts from -D of the queries
      // its registers hold (register 4a + b: query 8a + 4half + b)
      f32x16 nd;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 dz = *(const f32x4*)(ax + BM + 8 * a + 4 * half);
#pragma unroll
        for (int b = 0; b < 4; ++b) nd[4 * a + b] = dz[b];
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const vec a = *(const vec*)(dos + a_off[s]);
        dpa = M::run(a, vf[s], s == 0 ? nd : dpa);
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const vec bo = DIRECT ? b_direct(dos, c2, dt) : *(const vec*)(dot + b_off[dt][c2]);
          dv[dt] = M::run(pa[c2], bo, dv[dt]);
        }
      // dS = P (dP - D)
#pragma unroll
      for (int i = 0; i < 16; ++i) dpa[i] = sa[i] * dpa[i];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        u32x4 wd;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          wd[m] = __builtin_bit_cast(uint32_t, M::cvt(dpa[8 * c2 + 2 * m], dpa[8 * c2 + 2 * m + 1]));
        da[c2] = __builtin_bit_cast(vec, wd);
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const vec bq = DIRECT ? b_direct(qs, c2, dt) : *(const vec*)(qt + b_off[dt][c2]);
          dk[dt] = M::run(da[c2], bq, dk[dt]);
        }
    } else {
      // dP - D in one chain: the first dP MFMA starts from -D of the queries
      // its registers hold (register 4a + b: query 8a + 4half + b)
      f32x16 nd;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 dz = *(const f32x4*)(ax + BM + 8 * a + 4 * half);
#pragma unroll
        for (int b = 0; b < 4; ++b) nd[4 * a + b] = dz[b];
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const vec a = *(const vec*)(dos + a_off[s]);
        dpa = M::run(a, vf[s], s == 0 ? nd : dpa);
      }
      // P and dS in place of S and dP - D, four queries at a time: LSE*log2(e)
      // of the lane's queries 8a + 4half + 0..3
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 lz = *(const f32x4*)(ax + 8 * a + 4 * half);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 4 * a + b;
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[i], c, -lz[b]));
          if (MASK) {
            const int qi = i0 + 8 * a + 4 * half + b;
            const bool vis = key < Nk && (!CAUSAL || key <= qi);
            pv = vis ? pv : 0.f;
          }
          sa[i] = pv;
          dpa[i] = pv * dpa[i];
        }
      }
      // P^T and dS^T as A operands: k-step c2 takes registers 8c2 .. 8c2+7.
      vec pa[2], da[2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        u32x4 wp, wd;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          wp[m] = __builtin_bit_cast(uint32_t, M::cvt(sa[8 * c2 + 2 * m], sa[8 * c2 + 2 * m + 1]));
          wd[m] = __builtin_bit_cast(uint32_t, M::cvt(dpa[8 * c2 + 2 * m], dpa[8 * c2 + 2 * m + 1]));
        }
        pa[c2] = __builtin_bit_cast(vec, wp);
        da[c2] = __builtin_bit_cast(vec, wd);
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const vec bo = DIRECT ? b_direct(dos, c2, dt) : *(const vec*)(dot + b_off[dt][c2]);
          const vec bq = DIRECT ? b_direct(qs, c2, dt) : *(const vec*)(qt + b_off[dt][c2]);
          dv[dt] = M::run(pa[c2], bo, dv[dt]);
          dk[dt] = M::run(da[c2], bq, dk[dt]);
        }
    }
  };

  if (ntiles > 0) {
    // prologue: tiles 0..S-2 requested; tile 0 landed (copy path: tiles 0
    // and 1, and tile 0 transposed)
#pragma unroll
    for (int t = 0; t < S - 1; ++t) issue(t, t);
    wait_vmcnt<PENDING>();
    __syncthreads();
    if constexpr (!DIRECT) {
      transpose(0);
      __syncthreads();
    }
    const auto unmasked = std::integral_constant<bool, false>{};
    const auto masked = std::integral_constant<bool, true>{};
    // Step j (tile j in ring stage st = j % S): request tile j+S-1 into the
    // stage of tile j-1, (copy path) transpose tile j+1, compute tile j; then
    // wait until the next tile to read has landed and meet at the barrier.
    auto step = [&](auto mask_tag, int j, int st) {
      issue(j + S - 1, (st + S - 1) % S);
      transpose(j + 1);
      tile(mask_tag, j, st);
      wait_vmcnt<PENDING>();
      __syncthreads();
    };
    int j = 0;
    for (; j < first_free; ++j) step(masked, j, j % S);
    // Direct path: unmasked tiles S at a time from a tile in stage 0, so the
    // stages are constants and the LDS operand addresses are per-lane bases
    // plus immediates.
    if constexpr (DIRECT) {
      for (; j < ntiles && j % S != 0; ++j) step(unmasked, j, j % S);
      for (; j + S <= ntiles; j += S)
        [&]<int... I>(std::integer_sequence<int, I...>) {
          (step(unmasked, j + I, I), ...);
        }(std::make_integer_sequence<int, S>{});
    }
    for (; j < ntiles; ++j) step(unmasked, j, j % S);
  }

  // ---- epilogue: dK = scale * acc, dV = acc; lane l holds column 32dt + l%32
  // of keys kw0 + 8(i/4) + 4half + i%4.
  const float scale = p.scale;
  T* dkh = (T*)p.dk + kv_head;
  T* dvh = (T*)p.dv + kv_head;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kr = kw0 + 8 * (i >> 2) + 4 * half + (i & 3);
    if (kr < Nk) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        dkh[(size_t)kr * D + 32 * dt + r32] = (T)(scale * dk[dt][i]);
        dvh[(size_t)kr * D + 32 * dt + r32] = (T)dv[dt][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ for one block of 32*NW query rows.
template <int D, int NW, int S, bool CAUSAL, typename T>
__global__ __launch_bounds__(NW * 64, bwd_dq_min_waves(D)) void fa_bwd_dq_kernel(BwdParams p) {
  using M = Mma<T>;
  using vec = typename M::vec;
  constexpr int BN = 64;               // keys per tile (two units of 32)
  constexpr int BM = 32 * NW;          // query rows per workgroup
  constexpr int NT = 64 * NW;
  constexpr int KS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int CPR = D / 8;
  constexpr int CHUNKS = BN * CPR;     // 16-byte chunks per K (or V) tile
  constexpr int CPT = CHUNKS / NT;
  constexpr int TILE = BN * D * 2;
  constexpr int LOADS = 2 * CPT;
  constexpr bool DIRECT = D <= 64;  // K^T operand straight from the K tile
  constexpr int TBLK = (BN / 4) * (D / 16);
  constexpr int TPW = TBLK / (4 * NW);
  // Loads left in flight at the end of step j: tile j+1 must have landed
  // (the copy path transposes tile j+1 during step j, so tile j+2 there).
  constexpr int PENDING = (S - (DIRECT ? 2 : 3)) * LOADS;
  static_assert(CPT >= 1 && CPT * NT == CHUNKS, "tile must split evenly over threads");
  static_assert(DIRECT || (TPW >= 1 && TPW * 4 * NW == TBLK), "K transpose must split evenly over waves");
  static_assert(PENDING >= 0 && PENDING < 64, "stage count out of range");
  auto toff = [](int r, int c) { return DIRECT ? tile_off<2 * D>(r, c) : lds_off<2 * D>(r, c); };

  // K and V tiles as loaded ([stage][K, V], rows = keys in the permuted
  // order) and, on the copy path, K^T (rows = d, keys in natural order),
  // double-buffered.
  __shared__ __attribute__((aligned(1024))) char smem[S][2][TILE];
  __shared__ __attribute__((aligned(1024))) char kts[DIRECT ? 1 : 2][DIRECT ? 16 : TILE];

  int head, qb;
  bwd_work_item<CAUSAL>(p, blockIdx.x, head, qb);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int r32 = lane & 31;
  const int Nq = p.Nq, Nk = p.Nk;
  const float c = p.c;
  const size_t q_head = (size_t)head * Nq * D;
  const size_t kv_head = (size_t)head * Nk * D;
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.q + q_head), (short)0, Nq * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t do_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.dout + q_head), (short)0, Nq * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.k + kv_head), (short)0, Nk * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const T*)p.v + kv_head), (short)0, Nk * D * 2, kBufferFlags);

  const int q_row = qb * BM + 32 * wave + r32;  // this lane's query row

  // Q and dO rows of the lane's query: B operands of S^T and dP^T.
  vec qf[KS], dof[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int off = q_row * (2 * D) + 2 * (16 * s + 8 * half);
    qf[s] = __builtin_bit_cast(vec, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, off, 0, 0));
    dof[s] = __builtin_bit_cast(vec, __builtin_amdgcn_raw_buffer_load_b128(do_rsrc, off, 0, 0));
  }
  // Its LSE*log2(e) and D; rows past the records are padding (+inf, 0).
  float lse2 = __builtin_inff(), dlt = 0.f;  // dlt: -D
  if (q_row < p.nrec * 32) {
    const float* rec = p.aux + ((size_t)head * p.nrec + (q_row >> 5)) * 64 + (q_row & 31);
    lse2 = rec[0];
    dlt = rec[32];
  }
  f32x16 ndv;  // d = 64: -D in every register, the start of each dP^T chain
#pragma unroll
  for (int i = 0; i < 16; ++i) ndv[i] = dlt;

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

  f32x16 dq[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[t][i] = 0.f;

  // ---- HBM -> LDS: K and V rows both in the permuted key order, so that
  // accumulator register i of lane l holds key 16(l/32) + i of a unit.
  uint32_t goff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int sl = (wave * CPT + i) * 64 + lane;
    const int r = sl / CPR;
    const int ch = (toff(r, sl % CPR) - r * (2 * D)) >> 4;
    const int kkey = (r & ~31) | lds_row_to_key(r & 31);
    goff[i] = kkey * (2 * D) + 16 * ch;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)&smem[0][0][0];
  constexpr uint32_t kOutOfRange = 0x40000000u;
  auto issue = [&](int t, int st) {  // tile t into ring stage st (= t % S)
    const uint32_t gb = t < ntiles ? (uint32_t)(t * TILE) : kOutOfRange;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const uint32_t blk = (uint32_t)((wave * CPT + i) * 1024);
      dma_to_lds(k_rsrc, __builtin_amdgcn_readfirstlane(lds_base + (2 * st) * TILE + blk), goff[i] + gb);
      dma_to_lds(v_rsrc, __builtin_amdgcn_readfirstlane(lds_base + (2 * st + 1) * TILE + blk), goff[i] + gb);
    }
  };

  // ---- copy path: K tile -> K^T. A 4-aligned run of LDS rows holds 4
  // consecutive keys (from key0 on), which the transpose read hands to a
  // lane as one 8-byte run of its d column.
  int tr_src[DIRECT ? 1 : TPW], tr_dst[DIRECT ? 1 : TPW];
  if constexpr (!DIRECT) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int G = (wave * TPW + i) * 4 + (lane >> 4);
      const int r0 = 4 * (G % (BN / 4));
      const int d0 = 16 * (G / (BN / 4));
      const int x = lane & 15;
      const int col = d0 + 4 * (x & 3);
      tr_src[i] = lds_off<2 * D>(r0 + (x >> 2), col >> 3) + 2 * (col & 7);
      const int key0 = (r0 & ~31) | lds_row_to_key(r0 & 31);
      tr_dst[i] = lds_off<2 * BN>(d0 + x, key0 >> 3) + 2 * (key0 & 7);
    }
  }
  auto transpose_k = [&](int j) {
    if constexpr (!DIRECT) {
      const char* src = smem[j % S][0];
      char* dst = kts[j & 1];
      i16x4 blk[TPW];
#pragma unroll
      for (int i = 0; i < TPW; ++i)
        blk[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + tr_src[i]));
#pragma unroll
      for (int i = 0; i < TPW; ++i) *(i16x4*)(dst + tr_dst[i]) = blk[i];
    }
  };

  int a_off[2][KS];  // K / V rows of unit t: row 32t + r32, chunk 2s + half
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < KS; ++s) a_off[t][s] = toff(32 * t + r32, 2 * s + half);
  int kt_off[NDT][2][2];  // copy path: K^T rows 32dt + r32, keys 32t + 16half + 8s2 .. +7
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) kt_off[dt][t][s2] = lds_off<2 * BN>(32 * dt + r32, 4 * t + 2 * half + s2);
  // Direct path: K^T A operand of d tile dt for keys 32t + 16half + 8s2 .. +7 (natural
  // order, the order of the dS^T registers) straight from the K tile. LDS
  // row 16s2 + 4half + 0..3 (+ 32t) holds keys 16half + 8s2 + 0..3 and the
  // rows 8 on hold the next 4 (the permuted order keeps 4-aligned runs of
  // rows consecutive): two transpose reads, lane x of a 16-lane group
  // pointing at row 16s2 + 4half + x/4 (then + 8), columns d0 + 4(x%4) ..
  // +3 with d0 = 32dt + 16((lane/16)%2), and receiving 4 keys of column
  // d0 + x.
  const int trx = lane & 15;
  const int tr_row = 4 * half + (trx >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (trx & 3);
  auto kt_direct = [&](const char* ks, int t, int s2, int dt) -> vec {
    const int row = tr_row + 32 * t + 16 * s2;
    const int col = tr_col + 32 * dt;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(ks + tile_off<2 * D>(row, col >> 3) + 2 * (col & 7)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(ks + tile_off<2 * D>(row + 8, col >> 3) + 2 * (col & 7)));
    const u32x2 wl = __builtin_bit_cast(u32x2, lo), wh = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(vec, u32x4{wl[0], wl[1], wh[0], wh[1]});
  };

  auto unit = [&](auto mask_tag, int j, int t, int st) {  // unit t of tile j, in ring stage st
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* ks = smem[st][0];
    const char* vs = smem[st][1];
    const char* kt = kts[DIRECT ? 0 : (j & 1)];
    f32x16 sa, dpa;
#pragma unroll
    for (int s = 0; s < KS; ++s) sa = M::run(*(const vec*)(ks + a_off[t][s]), qf[s], s == 0 ? f32x16{} : sa);
#pragma unroll
    // d = 64: dP^T - D in one chain, the first MFMA starting from -D (the
    // lane's query, in every register). At d = 32 (four waves per SIMD) and
    // d = 128 the 16 registers of that start do not fit, and -D is added per
    // score.
    for (int s = 0; s < KS; ++s)
      dpa = M::run(*(const vec*)(vs + a_off[t][s]), dof[s], s == 0 ? (D == 64 ? ndv : f32x16{}) : dpa);
    float ds[16];
    // keys j*BN + 32t + 16half + i are visible while i < lim
    int lim = 16;
    if (MASK) {
      lim = CAUSAL ? (q_row + 1 < Nk ? q_row + 1 : Nk) : Nk;
      lim -= j * BN + 32 * t + 16 * half;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[i], c, -lse2));
      if (MASK) pv = (i < lim) ? pv : 0.f;
      ds[i] = D == 64 ? pv * dpa[i] : pv * (dpa[i] + dlt);
    }
    vec b[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4 w;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        w[m] = __builtin_bit_cast(uint32_t, M::cvt(ds[8 * s2 + 2 * m], ds[8 * s2 + 2 * m + 1]));
      b[s2] = __builtin_bit_cast(vec, w);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        dq[dt] = M::run(DIRECT ? kt_direct(ks, t, s2, dt) : *(const vec*)(kt + kt_off[dt][t][s2]), b[s2], dq[dt]);
  };

  // prologue: tiles 0..S-2 requested, tile 0 landed (copy path: tiles 0
  // and 1, and K^T of tile 0 written)
#pragma unroll
  for (int t = 0; t < S - 1; ++t) issue(t, t);
  wait_vmcnt<PENDING>();
  __syncthreads();
  if constexpr (!DIRECT) {
    transpose_k(0);
    __syncthreads();
  }
  const auto unmasked = std::integral_constant<bool, false>{};
  const auto masked = std::integral_constant<bool, true>{};
  // Step j (tile j in ring stage st = j % S), as in the dK/dV kernel.
  auto step = [&](auto mask_tag, int j, int st) {
    issue(j + S - 1, (st + S - 1) % S);
    transpose_k(j + 1);
    unit(mask_tag, j, 0, st);
    unit(mask_tag, j, 1, st);
    wait_vmcnt<PENDING>();
    __syncthreads();
  };
  int j = 0;
  // d = 32: unmasked tiles S at a time, ring stages as constants (at d = 64
  // the unrolled loop ran 4% slower).
  if constexpr (D == 32)
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
    transpose_k(j + 1);
    wait_vmcnt<PENDING>();
    __syncthreads();
  }

  // ---- epilogue: dQ = scale * acc. Lane l holds row q_row, columns
  // 32dt + 8g + 4half + 0..3 in registers 4g .. 4g+3.
  if (q_row < Nq) {
    const float scale = p.scale;
    T* dqh = (T*)p.dq + q_head + (size_t)q_row * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = __builtin_bit_cast(uint32_t, M::cvt(scale * dq[dt][4 * g + 0], scale * dq[dt][4 * g + 1]));
        w[1] = __builtin_bit_cast(uint32_t, M::cvt(scale * dq[dt][4 * g + 2], scale * dq[dt][4 * g + 3]));
        *(u32x2*)(dqh + 32 * dt + 8 * g + 4 * half) = w;
      }
  }
}

}  // namespace fa
