// fa_fwd_kernel.hpp - the exact-attention forward block on 32x32x16 matrix
// instructions for gfx950 (CDNA4), and the definitions the forward kernels
// share (Params, Strides, work_item). The tiled forward now runs on the
// 16x16x32 form (fa_fwd16.hpp); this block serves the persistent form
// (fa_fwd_stream.hpp), which cuts a query block's key range into pieces.
//
// Method (kwkr.cn YOLO11 FlashAttention-2 article, section 1.2; "FlashAttention
// 深度解读", section 原理 items 1-2 and the precision-handling paragraph;
// ai2ai.xin flash-attention-principle page, section on block computation):
// one workgroup owns a block of query rows of one (batch, head); it streams the
// head's K and V in tiles of BN keys through LDS, and for each tile computes
// the scores on the matrix cores, folds them into a running row maximum and a
// running exponential sum, rescales the output accumulator when the maximum
// grows, and adds P V. The score matrix lives only in registers.
//
// gfx950 mapping
//   * A wave owns RB blocks of 32 query rows. Scores are formed transposed,
//     S^T = K Q^T, with v_mfma_f32_32x32x16_{f16,bf16}: K rows are the A
//     operand (16-byte LDS reads), the wave's Q rows are the B operand and stay
//     in VGPRs for the whole kernel. One K fragment feeds the RB row blocks.
//     In the 32x32 accumulator layout lane l holds column l%32 (its query) and
//     16 rows (keys), so a query's scores sit in two lanes (l and l^32) and the
//     row reductions are in-register plus one exchange with the partner lane.
//   * K rows are placed in LDS in a permuted order so that accumulator
//     register i of lane l holds key 16*(l/32)+i of its 32-key subtile. Those
//     registers, rounded to fp16/bf16 in pairs (v_cvt_pk_*), are directly the
//     B operand (P^T) of O^T += V^T P^T. The V^T operands come from the V
//     tile itself, two ds_read_b64_tr_b16 transpose reads per operand (VT = 0),
//     or from a copy transposed once per workgroup, one tile ahead (VT = 1).
//   * O^T accumulates in fp32 MFMA accumulators: lane l holds d/2 elements of
//     its query's output row.
//   * Global reads are buffer loads whose range is one head's tensor, so rows
//     and keys past the end read as zero without branches. K/V tiles go from
//     HBM straight into LDS (buffer_load ... lds, 16 bytes per lane) through a
//     ring of S stages, S-1 tiles ahead of the math, with no staging
//     registers; each wave waits on its own loads (vmcnt) and one barrier per
//     tile publishes a stage to the workgroup. LDS rows are XOR-swizzled in
//     16-byte chunks (tile_off) against bank conflicts.
//   * exp is v_exp_f32 (2^x) on scores scaled by scale*log2(e), folded into one
//     FMA with the reference maximum. The row sum that normalises O is taken
//     from the same rounded P that enters the P V product, so the
//     normalisation matches the weights actually applied: for fp16 on the
//     matrix cores (a 16x16x32 MFMA against a 0/1 selector, sparing the
//     vector units), for bf16 on the vector units (one dot2 per pair). fp16
//     takes its log-sum-exp from that sum too; bf16 also sums the fp32 P
//     before rounding for the log-sum-exp, since 8-bit rounding would move it
//     by up to 2^-8.
//   * The reference maximum lags the true running maximum: P of a tile is
//     formed against it first, and only when that tile's row sum exceeds 2^15
//     (or is not finite, as on a row's first tile) is the maximum of the tile
//     taken, O and the row sum rescaled and P redone. The row sum bounds every
//     P of the row, so P always stays finite in fp16 and keeps full relative
//     precision; the result is unchanged in exact arithmetic because O and the
//     row sum carry the same reference. The common path thus needs no row
//     maximum at all: per score it is one FMA, one exp2 and half a conversion.
//   * The block first runs optimistically: the reference comes
//     from its first tile and is never tested again, so no unit waits for its
//     row sums. A P too large for its type then shows as a non-finite row
//     sum or output at the end, and the workgroup redoes the block with the
//     tests (scores that rise far along the keys; rare for real data).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fa_device.hpp"

namespace fa {

// Element strides of one [B, H, N, d] tensor: batch, head and row (the d
// elements of a row are contiguous). Contiguous tensors have (H*N*d, N*d, d).
struct Strides {
  int64_t b, h;
  int n;
};

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Nq, Nk;
  int num_qb;     // query blocks per head
  int total;      // workgroups = B*H*num_qb
  int xcd_q;      // total / 8
  int xcd_r;      // total % 8
  int group;      // heads per scheduling group
  int launch_order;  // nonzero: logical id = workgroup id (no per-XCD ranges)
  float c;        // |scale| * log2(e), or 1 when scale == 0
  uint32_t q_and; // applied to each 32-bit word of Q: ~0 normally, 0 when scale == 0
  uint32_t q_xor; // 0x80008000 flips both halves' sign when scale < 0
  int nkt;        // short-range kernel: 64-key tiles (= waves) per workgroup
  Strides sq, sk, sv, so;  // layouts of q, k, v and o
};

// First element of head (b, h) of a tensor, and the bytes a buffer resource
// over its n rows must cover (rows past n then read as zero).
template <typename T>
__device__ __forceinline__ T* head_base(const void* base, const Strides& s, int b, int h) {
  return (T*)base + (int64_t)b * s.b + (int64_t)h * s.h;
}
template <int D>
__device__ __forceinline__ int head_bytes(int n, const Strides& s) {
  return ((n - 1) * s.n + D) * 2;
}

// Largest tile row sum, relative to the reference maximum, that is accepted
// without raising the maximum (see the file comment). Every P of the tile is
// at most its row sum, so each stays below 2^15 and is finite in fp16.
constexpr float kTileSumLimit = 32768.0f;

// Workgroup id -> (head, query block). Workgroups are dispatched round-robin
// over the 8 XCDs; the remap gives each XCD a contiguous range of logical ids
// so the query blocks of one head share that XCD's L2 for its K/V. Inside the
// range, heads are taken in groups; for causal masks the heaviest query
// blocks (most key tiles) of a group go first.
template <bool CAUSAL>
__device__ __forceinline__ void work_item(const Params& p, int bid, int& head, int& qb) {
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int L = p.launch_order ? bid : xcd * p.xcd_q + (xcd < p.xcd_r ? xcd : p.xcd_r) + slot;
  const int per_group = p.group * p.num_qb;
  const int grp = L / per_group;
  const int rem = L - grp * per_group;
  const int heads_total = p.B * p.H;
  int hig = heads_total - grp * p.group;
  hig = hig < p.group ? hig : p.group;
  const int rank = rem / hig;
  head = grp * p.group + (rem - rank * hig);
  qb = CAUSAL ? (p.num_qb - 1 - rank) : rank;
}

// One query block (head, qb) over key tiles [t_lo, t_hi) (clipped to the
// tiles the block sees). part == nullptr: the block's whole key range, so O
// and LSE are written. Otherwise a piece of it: the unnormalised O^T
// ([D][BM] fp32), the reference maximum, the log-sum-exp's row sum and the
// normaliser's row sum (each [BM] fp32) go to part, to be merged with the
// block's other pieces.
//
// strict = false is the optimistic pass: the reference maximum is set from
// the block's first tile (first unit, when pipelined) and never raised after,
// so no later unit waits for its row sums before P V. A P more than 2^16
// above the reference overflows fp16 (bf16: far beyond, the fp32 row sum or
// output) and shows as a non-finite row sum or output at the end; then
// nothing is stored and false is returned (the same for every wave of the
// workgroup), and the caller runs the block again with strict = true, which
// raises the reference whenever a unit's row sum exceeds 2^15 or is not
// finite, so P never overflows. (A runtime flag, not a template parameter:
// one copy of the loop serves both passes.)
//
// VT = 1: each V tile is transposed once per workgroup into a double-buffered
// V^T tile (vts, 2 x BN*D*2 bytes), which the waves read with 16-byte reads.
// VT = 0: no V^T buffer (vts unused); every wave reads its V^T operands from
// the V tile itself with transpose reads (two per operand), which saves the
// transpose step, its barrier distance and its LDS, so the ring can be
// shorter (S >= 2, or 3 with PIPE).
template <int D, int BN, int NW, int RB, int S, bool PIPE, int VT, bool CAUSAL, typename T>
__device__ __forceinline__ bool fa_fwd_block(const Params& p, int head, int qb, int t_lo, int t_hi,
                                             float* part, char (&smem)[S][2][BN * D * 2],
                                             char* vts, bool strict = true) {
  using M = Mma<T>;
  using vec = typename M::vec;
  using pair = typename M::pair;
  constexpr int WR = 32 * RB;          // query rows per wave
  constexpr int BM = WR * NW;          // query rows per workgroup
  constexpr int NT = 64 * NW;          // threads per workgroup
  constexpr int KS = D / 16;           // k-steps of the QK^T contraction
  constexpr int NSUB = BN / 32;        // 32-key subtiles per tile
  constexpr int NDT = D / 32;          // 32-wide d tiles of O
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int CHUNKS = BN * CPR;     // chunks per K (or V) tile
  constexpr int CPT = CHUNKS / NT;     // 16-byte chunks per thread per tensor
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int LOADS = 2 * CPT;       // LDS loads per thread per tile (K and V)
  constexpr int TBLK = (BN / 4) * (D / 16);  // 4-key x 16-d blocks of a V tile
  constexpr int TPW = TBLK / (4 * NW);       // transpose reads per wave per tile
  static_assert(CPT >= 1 && CPT * NT == CHUNKS, "tile must split evenly over threads");
  static_assert(TPW >= 1 && TPW * 4 * NW == TBLK, "V transpose must split evenly over waves");
  static_assert(BM % BN == 0, "a query block must cover whole key tiles");
  // Loads left in flight at the end of an iteration. VT = 1: the next
  // iteration reads K of tile j+1 (and, pipelined, of j+2) and transposes V
  // of tile j+2, so tiles up to j+2 must have landed. VT = 0: it reads K and
  // V of tile j+1 (pipelined: also K of j+2).
  constexpr int AHEAD = VT ? 3 : (PIPE ? 3 : 2);
  constexpr int PENDING = (S - AHEAD) * LOADS;
  static_assert(S >= AHEAD && PENDING < 64, "stage count out of range");

  int tid = threadIdx.x;
  // Opaque to the optimiser, so the address arithmetic below is redone in
  // each pass instead of being hoisted out of the caller's pass loop and
  // held in registers through both.
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  // Wave index in a scalar register: every per-wave condition below (which
  // row blocks see a tile) must compile to a scalar branch, never to an
  // EXEC mask, because MFMA instructions ignore EXEC.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;  // which 16-key half of a subtile this lane holds
  const int r32 = lane & 31;   // this lane's query within a 32-row block

  const int Nq = p.Nq, Nk = p.Nk;
  const int hb = head / p.H, hh = head - hb * p.H;
  const int qrs = 2 * p.sq.n, krs = 2 * p.sk.n, vrs = 2 * p.sv.n;  // row strides in bytes
  const __amdgpu_buffer_rsrc_t q_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)head_base<const T>(p.q, p.sq, hb, hh), (short)0, head_bytes<D>(Nq, p.sq), kBufferFlags);
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)head_base<const T>(p.k, p.sk, hb, hh), (short)0, head_bytes<D>(Nk, p.sk), kBufferFlags);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)head_base<const T>(p.v, p.sv, hb, hh), (short)0, head_bytes<D>(Nk, p.sv), kBufferFlags);

  const int wave_q0 = qb * BM + wave * WR;

  // ---- this lane's query rows as B-operand fragments (8 elements per k-step)
  vec qf[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = wave_q0 + 32 * rb + r32;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
          q_rsrc, row * qrs + 2 * (16 * s + 8 * half), 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (w[e] & p.q_and) ^ p.q_xor;
      qf[rb][s] = __builtin_bit_cast(vec, w);
    }
  }

  int kv_end = Nk;
  if (CAUSAL) {
    const int last = qb * BM + BM;  // keys < last can be visible to this block
    kv_end = last < Nk ? last : Nk;
  }
  const int ntiles = (kv_end + BN - 1) / BN;
  t_hi = t_hi < ntiles ? t_hi : ntiles;  // tiles of this call: [t_lo, t_hi)

  f32x16 oacc[RB][NDT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[rb][t][i] = 0.f;
  // Running reference maximum (exp2 domain) and row sums relative to it:
  // l_run, the whole row's sum of the rounded P (the normaliser of O, and for
  // fp16 also the log-sum-exp's), and for bf16 l32_run, the sum of the
  // unrounded fp32 P over the lane's half of the keys (the log-sum-exp's;
  // combined with the partner lane at the end).
  float m_run[RB], l_run[RB], l32_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -__builtin_inff();
    l_run[rb] = 0.f;
    l32_run[rb] = 0.f;
  }
  // A operand of the row-sum MFMA (16x16x32): lane l holds row l%16 of the
  // 16x32 selector, for k group l/16. Row m picks the k groups of its own
  // query: A[m][k] = 1 iff (m/4)%2 == (k/8)%2. With B = the P operand (lane l
  // supplies k group l/16 of column l%16, i.e. 8 keys of query l%32), output
  // row m of column n sums the 16 keys of query n + 16*((m/4)%2), and the
  // 16x16 output layout puts rows 4*(l/16)..+3 of column l%16 in lane l: the
  // lane's own query l%32.
  const vec row_sel = M::selector((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1));
  const float c = p.c;

  // ---- tile loads (HBM -> LDS). Load i of this wave fills the 1 KB block
  // (wave*CPT + i) of a tile: 16-byte slot sl = 64*block + lane is physical
  // chunk sl % CPR of tile row sl / CPR, which holds logical chunk
  // (sl % CPR) ^ swizzle(row). K rows are fetched in the permuted key order,
  // V rows in natural order.
  uint32_t k_goff[CPT], v_goff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int sl = (wave * CPT + i) * 64 + lane;
    const int r = sl / CPR;
    const int ch = (tile_off<2 * D>(r, sl % CPR) - r * (2 * D)) >> 4;  // logical chunk
    const int kkey = (r & ~31) | lds_row_to_key(r & 31);
    k_goff[i] = kkey * krs + 16 * ch;
    v_goff[i] = r * vrs + 16 * ch;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  // Offsets of tiles past the end are pushed beyond every buffer's range:
  // those loads only write zeros to LDS and touch no memory.
  constexpr uint32_t kOutOfRange = 0x40000000u;
  // Tile t goes to ring stage st = (t - t_lo) % S; the callers pass st, a
  // constant where the loop is unrolled over the ring.
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

  // LDS read offsets (bytes) that do not depend on the tile.
  // K A-operand: row 32t + r32, chunk 2s + half.
  int k_roff[NSUB][KS];
#pragma unroll
  for (int t = 0; t < NSUB; ++t)
#pragma unroll
    for (int s = 0; s < KS; ++s) k_roff[t][s] = tile_off<2 * D>(32 * t + r32, 2 * s + half);
  // V transpose (once per tile per workgroup): transpose read i of this wave
  // covers, in 16-lane group g, the block of keys k0..k0+3 and d columns
  // d0..d0+15 of the V tile; lane x points at key k0 + x/4, columns
  // d0 + 4*(x%4) .. +3, and receives keys k0..k0+3 of column d0 + x, which it
  // writes as one 8-byte run into V^T row d0 + x.
  int tr_src[TPW], tr_dst[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int G = (wave * TPW + i) * 4 + (lane >> 4);
    const int k0 = 4 * (G % (BN / 4)), d0 = 16 * (G / (BN / 4));
    const int x = lane & 15;
    const int col = d0 + 4 * (x & 3);
    tr_src[i] = tile_off<2 * D>(k0 + (x >> 2), col >> 3) + 2 * (col & 7);
    tr_dst[i] = lds_off<2 * BN>(d0 + x, k0 >> 3) + 2 * (k0 & 7);
  }
  // V^T A-operand: row 32*dt + r32 (a d column), keys 32t + 16*half + 8*s2
  // .. +7, i.e. chunk 4t + 2*half + s2: one 16-byte read.
  int v_roff[NDT][NSUB][2];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int t = 0; t < NSUB; ++t)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        v_roff[dt][t][s2] = lds_off<2 * BN>(32 * dt + r32, 4 * t + 2 * half + s2);

  // V tile j (as loaded, in stage st) -> V^T buffer j % 2 (VT = 1 only)
  auto transpose_v = [&](int j, int st) {
    if constexpr (VT != 0) {
      const char* vsrc = smem[st][1];
      char* vdst = vts + ((j - t_lo) & 1) * TILE_BYTES;
      i16x4 blk[TPW];
#pragma unroll
      for (int i = 0; i < TPW; ++i)
        blk[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vsrc + tr_src[i]));
#pragma unroll
      for (int i = 0; i < TPW; ++i) *(i16x4*)(vdst + tr_dst[i]) = blk[i];
    }
  };
  // VT = 0: the V^T operand for d tile dt and keys k0 .. k0+7 (k0 = 32t +
  // 16*half + 8*s2) straight from the V tile: two transpose reads, each
  // handing lane x of a 16-lane group keys k0..k0+3 (then k0+4..k0+7) of d
  // column 32dt + 16*((lane/16)%2) + x while pointing at key k0 + x/4,
  // columns d0 + 4*(x%4)..+3 (all lanes of a group share k0 and d0).
  const int trx = lane & 15;
  const int tr_row = 16 * half + (trx >> 2);                    // key row of the first read, t = s2 = 0
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (trx & 3);    // d column, dt = 0
  auto vt_direct = [&](const char* vs, int t, int s2, int dt) -> vec {
    const int row = tr_row + 32 * t + 8 * s2;
    const int col = tr_col + 32 * dt;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(vs + tile_off<2 * D>(row, col >> 3) + 2 * (col & 7)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(vs + tile_off<2 * D>(row + 4, col >> 3) + 2 * (col & 7)));
    const u32x2 wl = __builtin_bit_cast(u32x2, lo), wh = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(vec, u32x4{wl[0], wl[1], wh[0], wh[1]});
  };

  // The work is a sequence of units, one per 32-key subtile t of tile j
  // (unit u = 2j + t). Registers per unit: its scores, its P (B operands) and
  // its row sums (rounded; bf16 also fp32), double-buffered by t.
  static_assert(NSUB == 2, "a tile is two 32-key units");
  f32x16 sacc[2][RB];
  vec pf[2][RB][2];
  float psum[2][RB], ps32[2][RB];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      psum[b][rb] = 0.f;
      ps32[b][rb] = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) pf[b][rb][s2] = vec{};
    }

  // LDS operands of one unit: K rows of subtile t of tile j (A operands of
  // S^T = K Q^T, one per k-step) and V^T of subtile t of tile j (A operands
  // of O^T += V^T P^T, per 16-key half s2 and 32-wide d tile).
  auto load_k = [&](int st, int t, vec (&kf)[KS]) {
    const char* ks = smem[st][0];
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = *(const vec*)(ks + k_roff[t][s]);
  };
  auto load_v = [&](int j, int st, int t, vec (&vf)[2][NDT]) {
    if constexpr (VT != 0) {
      const char* vs = vts + ((j - t_lo) & 1) * TILE_BYTES;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vf[s2][dt] = *(const vec*)(vs + v_roff[dt][t][s2]);
    } else {
      const char* vs = smem[st][1];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vf[s2][dt] = vt_direct(vs, t, s2, dt);
    }
  };
  auto qk = [&](const vec (&kf)[KS], f32x16 (&out)[RB]) {
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) out[rb] = M::run(kf[s], qf[rb][s], s == 0 ? f32x16{} : out[rb]);
  };
  auto pv = [&](const vec (&vf)[2][NDT], const vec (&pr)[RB][2]) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) oacc[rb][dt] = M::run(vf[s2][dt], pr[rb][s2], oacc[rb][dt]);
  };

  // Scores of keys past Nk, and (causal) of keys after the row, -> -inf.
  // Rows past a causal row block's last row are masked too, so such tiles
  // add exact zeros.
  auto mask_unit = [&](int j, int t, f32x16 (&sr)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // keys j*BN + 32t + 16*half + i are visible while i < lim
      const int q_row = wave_q0 + 32 * rb + r32;
      int lim = CAUSAL ? (q_row + 1 < Nk ? q_row + 1 : Nk) : Nk;
      lim -= j * BN + 32 * t + 16 * half;
#pragma unroll
      for (int i = 0; i < 16; ++i) sr[rb][i] = (i < lim) ? sr[rb][i] : -__builtin_inff();
    }
  };

  // Row sum of a unit's rounded P: two 16x16x32 MFMAs of the selector
  // against the P operands (each lane gets its own query's sum).
  auto sub_sum = [&](const vec (&pr)[2]) -> float {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) acc = M::sel_sum(row_sel, pr[s2], acc);
    return acc[0];
  };

  // P = 2^(S*c - m) of one row block's unit, rounded in pairs into its two B
  // operands; returns its row sum of the rounded P, and in l32 (bf16) the
  // lane's fp32 sum of the unrounded P.
  auto exp_unit = [&](const f32x16& sr, float negm, vec (&pr)[2], float& l32) {
    float lsum = 0.f, lrnd = 0.f;
    u32x4 w[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sr[2 * i], c, negm));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sr[2 * i + 1], c, negm));
      const pair pp = M::cvt(p0, p1);
      lsum = M::lse_sum(p0, p1, lsum);
      lrnd = M::rnd_sum(pp, lrnd);
      w[i >> 2][i & 3] = __builtin_bit_cast(uint32_t, pp);
    }
    pr[0] = __builtin_bit_cast(vec, w[0]);
    pr[1] = __builtin_bit_cast(vec, w[1]);
    l32 = lsum;
    if constexpr (M::kVecRowSum) return lrnd;
    return sub_sum(pr);
  };

  // Row maximum of a unit's scores, in the exp2 domain (both lanes of the
  // row take part).
  auto unit_max = [&](const f32x16& sr) -> float {
    float m4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) m4[k] = sr[k];
#pragma unroll
    for (int i = 4; i < 16; ++i) m4[i & 3] = vmax(m4[i & 3], sr[i]);
    return max_with_partner(vmax(vmax(m4[0], m4[1]), vmax(m4[2], m4[3]))) * c;
  };
  // Raise row block rb's reference maximum to cover mx: O and l are rescaled
  // by 2^(m_old - m_new). A row with no visible key yet keeps 0.
  auto raise_max = [&](int rb, float mx) {
    float m_new = vmax(m_run[rb], mx);
    m_new = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[rb][dt][i] *= alpha;
    l_run[rb] *= alpha;
    l32_run[rb] *= alpha;
    m_run[rb] = m_new;
  };
  // A unit's row sum bounds every P of the row, so a sum within
  // kTileSumLimit means its P is finite in fp16 and was formed against a
  // usable reference (no maximum is needed for that). Otherwise (a row's
  // first unit, where m_run = -inf, or scores grown past the reference by
  // about 2^15) the reference is raised and P redone.
  auto unit_ok = [&](const float (&ps)[RB]) {
    bool ok = true;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) ok &= (ps[rb] <= kTileSumLimit);
    return ok;
  };

  // Tiles from `first_masked` on need masking: the tile holding key Nk-1 when
  // Nk is not a multiple of BN, and (causal) every tile that reaches past the
  // first row of the workgroup.
  int first_masked = (Nk % BN == 0) ? ntiles : Nk / BN;
  if (CAUSAL) {
    const int diag = (qb * BM) / BN;  // first tile with a key > row qb*BM
    first_masked = diag < first_masked ? diag : first_masked;
  }
  first_masked = first_masked < ntiles ? first_masked : ntiles;

  // Start of tile j (both loops): request tile j+S-1 into the stage of tile
  // j-1 (free since the last barrier) and write V^T of tile j+1 (its stage
  // has landed). End of tile j: wait until tile j+2 has landed (this wave's
  // own loads) and meet the other waves at the barrier. Past the last tile
  // the stages hold zeros from out-of-range loads.
  auto tile_start = [&](int j, int st) {
    issue(j + S - 1, (st + S - 1) % S);
    transpose_v(j + 1, (st + 1) % S);
  };
  auto tile_end = [&]() {
    wait_vmcnt<PENDING>();
    __syncthreads();
  };

  // ---- the steps of a tile: Q K^T of both units; mask, P and row sums with
  // one acceptance test for the tile (raising the reference to the tile's
  // maximum when it fails); P V.
  auto qk_step = [&](int st) {
    // k-step outer, unit inner: consecutive MFMAs feed different accumulators
    const char* ks = smem[st][0];
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const vec a = *(const vec*)(ks + k_roff[t][s]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sacc[t][rb] = M::run(a, qf[rb][s], s == 0 ? f32x16{} : sacc[t][rb]);
      }
  };
  auto softmax_step = [&](auto mask_tag, int j) {
    if (decltype(mask_tag)::value) {
      mask_unit(j, 0, sacc[0]);
      mask_unit(j, 1, sacc[1]);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        psum[t][rb] = exp_unit(sacc[t][rb], -m_run[rb], pf[t][rb], ps32[t][rb]);
    if ((strict || j == t_lo) && __any(!(unit_ok(psum[0]) && unit_ok(psum[1])))) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        raise_max(rb, vmax(unit_max(sacc[0][rb]), unit_max(sacc[1][rb])));
#pragma unroll
        for (int t = 0; t < 2; ++t)
          psum[t][rb] = exp_unit(sacc[t][rb], -m_run[rb], pf[t][rb], ps32[t][rb]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l_run[rb] += psum[0][rb] + psum[1][rb];
      if constexpr (M::kLse32) l32_run[rb] += ps32[0][rb] + ps32[1][rb];
    }
  };
  auto pv_step = [&](int j, int st) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      vec vf[2][NDT];
      load_v(j, st, t, vf);
      pv(vf, pf[t]);
    }
  };

  // ---- the plain loop: one tile at a time, all waves in step.
  auto plain_tile = [&](auto mask_tag, int j, int st) {
    qk_step(st);
    softmax_step(mask_tag, j);
    pv_step(j, st);
    tile_end();
  };

  // ---- the pipelined loop: Q K^T runs one unit ahead. Unit u forms its P
  // on the vector units while the matrix cores compute the scores of unit
  // u+1; the order is written out (each MFMA, then its share of the P pairs,
  // fenced so that the compiler keeps the interleaving). Then come unit u's
  // row sums on the matrix cores, its acceptance test (raising the reference
  // and redoing P when it fails) and its P V. Only the scores cross from one
  // unit to the next.
  constexpr int NMF = RB * KS;  // Q K^T MFMAs of a unit
  constexpr int NPR = RB * 8;   // P pairs of a unit
  auto piped_unit = [&](auto mask_tag, int j, int t, f32x16 (&sr)[RB], vec (&pr)[RB][2],
                        float (&ps)[RB], float (&p32)[RB], const vec (&kf)[KS], f32x16 (&sn)[RB],
                        int st) {
    if (decltype(mask_tag)::value) mask_unit(j, t, sr);
    float negm[RB], lsum[RB], lrnd[RB];
    u32x4 w[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      negm[rb] = -m_run[rb];
      lsum[rb] = 0.f;
      lrnd[rb] = 0.f;
    }
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (
          [&] {
            constexpr int m = I;
            constexpr int s = m / RB, rb = m % RB;
            sn[rb] = M::run(kf[s], qf[rb][s], s == 0 ? f32x16{} : sn[rb]);
#pragma unroll
            for (int q = m * NPR / NMF; q < (m + 1) * NPR / NMF; ++q) {
              const int rq = q / 8, i = q % 8;
              const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sr[rq][2 * i], c, negm[rq]));
              const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sr[rq][2 * i + 1], c, negm[rq]));
              const pair pq = M::cvt(p0, p1);
              lsum[rq] = M::lse_sum(p0, p1, lsum[rq]);
              lrnd[rq] = M::rnd_sum(pq, lrnd[rq]);
              w[rq][i >> 2][i & 3] = __builtin_bit_cast(uint32_t, pq);
            }
            __builtin_amdgcn_sched_barrier(0);
          }(),
          ...);
    }(std::make_integer_sequence<int, NMF>{});
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      pr[rb][0] = __builtin_bit_cast(vec, w[rb][0]);
      pr[rb][1] = __builtin_bit_cast(vec, w[rb][1]);
      if constexpr (M::kVecRowSum)
        ps[rb] = lrnd[rb];
      else
        ps[rb] = sub_sum(pr[rb]);
      p32[rb] = lsum[rb];
    }
    vec vf[2][NDT];
    load_v(j, st, t, vf);
    if ((strict || (j == t_lo && t == 0)) && __any(!unit_ok(ps))) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        raise_max(rb, unit_max(sr[rb]));
        ps[rb] = exp_unit(sr[rb], -m_run[rb], pr[rb], p32[rb]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l_run[rb] += ps[rb];
      if constexpr (M::kLse32) l32_run[rb] += p32[rb];
    }
    pv(vf, pr);
  };
  auto piped_tile = [&](auto mask_tag, int j, int st) {
    {  // unit (j, 0), with Q K^T of unit (j, 1)
      vec kf[KS];
      load_k(st, 1, kf);
      piped_unit(mask_tag, j, 0, sacc[0], pf[0], psum[0], ps32[0], kf, sacc[1], st);
    }
    {  // unit (j, 1), with Q K^T of unit (j+1, 0)
      vec kf[KS];
      load_k((st + 1) % S, 0, kf);
      piped_unit(mask_tag, j, 1, sacc[1], pf[1], psum[1], ps32[1], kf, sacc[0], st);
    }
    tile_end();
  };

  // ---- prologue: tiles t_lo..t_lo+S-2 requested, V^T of tile t_lo written.
#pragma unroll
  for (int t = 0; t < S - 1; ++t) issue(t_lo + t, t);
  wait_vmcnt<PENDING>();
  __syncthreads();
  if constexpr (VT != 0) {
    transpose_v(t_lo, 0);
    __syncthreads();
  }

  // Causal: a tile whose first key comes after this wave's last row adds
  // nothing to any of its rows, and neither does any later tile. The test is
  // wave-uniform; the scores a pipelined wave carries into such a tile are
  // never used.
  auto beyond_rows = [&](int j) { return CAUSAL && j * BN > wave_q0 + WR - 1; };
  const auto unmasked = std::integral_constant<bool, false>{};
  const auto masked = std::integral_constant<bool, true>{};
  const int j_free = first_masked < t_hi ? first_masked : t_hi;
  int j = t_lo;
  auto stage = [&](int jj) { return (jj - t_lo) % S; };
  // The unmasked tiles run S at a time from t_lo, so that the ring stage of
  // each is a constant and every LDS operand address is a per-lane base plus
  // an immediate offset; the rest (fewer than S unmasked tiles, and the
  // masked ones) take the stage at run time. At d = 128 the per-lane bases
  // of all K and V^T reads (24 registers) do not fit beside the operands,
  // and every tile takes the stage at run time.
  constexpr bool kRingUnroll = D <= 64;
  auto ring_steps = [&](auto body) {
    if constexpr (kRingUnroll)
      for (; j + S <= j_free; j += S)
      [&]<int... I>(std::integer_sequence<int, I...>) {
        (body(j + I, I), ...);
      }(std::make_integer_sequence<int, S>{});
  };
  if constexpr (PIPE) {
    // Scores of the first unit before the loop; its test raises the
    // reference from -inf.
    {
      vec kf[KS];
      load_k(0, 0, kf);
      qk(kf, sacc[0]);
    }
    ring_steps([&](int jj, int st) {
      tile_start(jj, st);
      piped_tile(unmasked, jj, st);
    });
    for (; j < j_free; ++j) {
      tile_start(j, stage(j));
      piped_tile(unmasked, j, stage(j));
    }
    for (; j < t_hi && !beyond_rows(j); ++j) {
      tile_start(j, stage(j));
      piped_tile(masked, j, stage(j));
    }
  }
  if constexpr (!PIPE) {
    ring_steps([&](int jj, int st) {
      tile_start(jj, st);
      plain_tile(unmasked, jj, st);
    });
    for (; j < j_free; ++j) {
      tile_start(j, stage(j));
      plain_tile(unmasked, j, stage(j));
    }
    for (; j < t_hi && !beyond_rows(j); ++j) {
      tile_start(j, stage(j));
      plain_tile(masked, j, stage(j));
    }
  }

  // Causal tiles past this wave's rows: only its share of the loads,
  // transposes and barriers.
  for (; j < t_hi; ++j) {
    tile_start(j, stage(j));
    tile_end();
  }

  if (!strict) {
    // Every row sum finite, or the workgroup redoes the block. The ring is
    // drained first: the loads past the last tile (zeros) may still be in
    // flight, and a second pass refills the same stages. Each wave leaves its
    // verdict in a word of the drained ring.
    bool bad = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float l_tot = l_run[rb] + (M::kLse32 ? l32_run[rb] : 0.f);  // finiteness only
      float om = 0.f;  // bf16 P reaches 2^127 before the row sum overflows: check O too
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) om = vmax(om, __builtin_fabsf(oacc[rb][dt][i]));
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
      __syncthreads();  // every wave has read the verdicts before the ring refills
      return false;
    }
  }

  if (part != nullptr) {
    // ---- a piece of the key range: unnormalised O^T, reference, row sum
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = wave * WR + 32 * rb + r32;  // row within the block
      const float l_nrm = M::kVecRowSum ? sum_with_partner(l_run[rb]) : l_run[rb];
      const float l_lse = M::kLse32 ? sum_with_partner(l32_run[rb]) : l_nrm;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          part[(32 * dt + 8 * (i >> 2) + 4 * half + (i & 3)) * BM + row] = oacc[rb][dt][i];
      if (half == 0) {
        part[D * BM + row] = m_run[rb];
        part[D * BM + BM + row] = l_lse;
        part[D * BM + 2 * BM + row] = l_nrm;
      }
    }
    return true;
  }

  // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int q_row = wave_q0 + 32 * rb + r32;
    const float l_nrm = M::kVecRowSum ? sum_with_partner(l_run[rb]) : l_run[rb];
    const float l_lse = M::kLse32 ? sum_with_partner(l32_run[rb]) : l_nrm;
    const float inv = 1.0f / l_nrm;
    if (q_row < Nq) {
      T* Oh = head_base<T>(p.o, p.so, hb, hh) + (int64_t)q_row * p.so.n;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = __builtin_bit_cast(uint32_t, M::cvt(oacc[rb][dt][4 * g + 0] * inv,
                                                     oacc[rb][dt][4 * g + 1] * inv));
          w[1] = __builtin_bit_cast(uint32_t, M::cvt(oacc[rb][dt][4 * g + 2] * inv,
                                                     oacc[rb][dt][4 * g + 3] * inv));
          *(u32x2*)(Oh + 32 * dt + 8 * g + 4 * half) = w;
        }
      if (p.lse != nullptr && half == 0)
        p.lse[(size_t)head * Nq + q_row] = 0.69314718055994531f * (m_run[rb] + log2f(l_lse));
    }
  }
  return true;
}

// Waves per SIMD the register allocation must allow. At d = 64 with a V^T
// copy, two workgroups share a CU by LDS (80 KB each), and the bf16 form would
// otherwise take a few registers more than half the file; capped at two
// waves it spills a dozen registers and runs 15% faster. Reading V^T
// directly, three workgroups share a CU (32 KB each with the 2-stage ring)
// and the cap is three waves (one 32-row block per wave needs about 150
// registers).
#ifndef FA_FWD_MIN_WAVES_D64_DIRECT
#define FA_FWD_MIN_WAVES_D64_DIRECT 3
#endif
constexpr int fwd_min_waves(int d, int vt) {
  return d == 64 ? (vt ? 2 : FA_FWD_MIN_WAVES_D64_DIRECT) : 1;
}

template <int D, int BN, int NW, int RB, int S, bool PIPE, int VT, bool CAUSAL, typename T>
__global__ __launch_bounds__(NW * 64, fwd_min_waves(D, VT)) void fa_fwd_kernel(Params p) {
  // K and V tiles as loaded ([stage][K,V], rows = keys), and (VT = 1) V^T
  // tiles (rows = d, BN keys each) for the P V operand, double-buffered:
  // while tile j runs, V^T of tile j+1 is written.
  __shared__ __attribute__((aligned(1024))) char smem[S][2][BN * D * 2];
  int head, qb;
  work_item<CAUSAL>(p, blockIdx.x, head, qb);
  char* vts = nullptr;
  if constexpr (VT != 0) {
    __shared__ __attribute__((aligned(1024))) char vt_buf[2][BN * D * 2];
    vts = &vt_buf[0][0];
  }
  // the optimistic pass, then (rarely) the strict one
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass)
    if (fa_fwd_block<D, BN, NW, RB, S, PIPE, VT, CAUSAL, T>(p, head, qb, 0, 0x7fffffff, nullptr, smem,
                                                            vts, pass == 1))
      break;
}

}  // namespace fa
