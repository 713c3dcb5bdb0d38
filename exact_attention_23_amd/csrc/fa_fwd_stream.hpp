// fa_fwd_stream.hpp - the forward with the work split evenly over a persistent
// grid, and the merge of query blocks whose key range was split.
//
// The tiled forward gives every workgroup one query block. When the blocks
// outnumber the resident workgroups by a non-integer factor, the last round
// runs partly empty (1600 equal blocks on 512 resident workgroups take 4
// rounds of work for 3.125 rounds' worth). Here a grid of exactly the
// resident workgroups walks the flattened (query block, key tile) sequence:
// workgroup w takes tiles [w*T/G, (w+1)*T/G) of the T tiles, so every
// workgroup does the same number of tiles (to within one). A query block cut
// by such a boundary is computed in pieces, each over its own key range; a
// piece leaves its unnormalised O, its reference maximum and its row sums
// (the normaliser's, n_p, and the log-sum-exp's, l_p; the same sum for
// fp16), and the combine kernel merges the pieces of a block exactly: with m
// the largest reference, O = sum_p 2^(m_p - m) O_p / sum_p 2^(m_p - m) n_p
// and LSE = ln2 (m + log2 sum_p 2^(m_p - m) l_p). This is the
// same rescaling the online softmax applies between tiles (kwkr.cn YOLO11
// FlashAttention-2 article, section 1.2), applied across workgroups.
//
// Full masks only (every block has the same number of tiles). Workspace per
// workgroup: two piece slots of BM * (D + 3) floats ([D][BM] O^T, then the
// BM references, the BM log-sum-exp row sums and the BM normaliser row
// sums); a workgroup's first and last segments are the only ones that can be
// pieces.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_fwd_kernel.hpp"

namespace fa {

struct StreamParams {
  float* part;    // [G][2][BM * (D + 3)] fp32 piece slots
  int64_t total;  // T: tiles over all blocks (blocks * ntb)
  int ntb;        // key tiles per query block
  int nblocks;    // B * H * query blocks per head
  int G;          // workgroups of the persistent grid
  int gq, gr;     // G / 8, G % 8 (XCD-contiguous numbering)
};

// First tile of logical workgroup w.
__device__ __forceinline__ int64_t stream_start(const StreamParams& sp, int w) {
  return (int64_t)w * sp.total / sp.G;
}

template <int D, int BN, int NW, int RB, int S, bool PIPE, int VT, typename T>
__global__ __launch_bounds__(NW * 64, 2) void fa_fwd_stream_kernel(Params p, StreamParams sp) {
  constexpr int BM = 32 * RB * NW;
  __shared__ __attribute__((aligned(1024))) char smem[S][2][BN * D * 2];
  char* vts = nullptr;
  if constexpr (VT != 0) {
    __shared__ __attribute__((aligned(1024))) char vt_buf[2][BN * D * 2];
    vts = &vt_buf[0][0];
  }
  // Logical numbering: workgroups are dispatched round-robin over the 8
  // XCDs; consecutive logical ranges (the blocks of one head) stay on one
  // XCD and share its L2 for the head's K and V.
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int w = xcd * sp.gq + (xcd < sp.gr ? xcd : sp.gr) + slot;
  const int64_t g_hi = stream_start(sp, w + 1);
  int64_t g = stream_start(sp, w);
  bool first = true;
  while (g < g_hi) {
    const int bid = (int)(g / sp.ntb);
    const int t0 = (int)(g - (int64_t)bid * sp.ntb);
    const int64_t left = g_hi - g;
    const int t1 = left < sp.ntb - t0 ? t0 + (int)left : sp.ntb;
    const int head = bid / p.num_qb;
    const int qb = bid - head * p.num_qb;
    float* part = nullptr;
    if (t0 != 0 || t1 != sp.ntb)
      part = sp.part + ((size_t)w * 2 + (first ? 0 : 1)) * (size_t)(BM * (D + 3));
    fa_fwd_block<D, BN, NW, RB, S, PIPE, VT, false, T>(p, head, qb, t0, t1, part, smem, vts);
    g += t1 - t0;
    first = false;
    if (g < g_hi) {
      // the next segment reuses the LDS ring: let every load of this one
      // land and every wave leave it first
      wait_vmcnt<0>();
      __syncthreads();
    }
  }
}

// One workgroup per boundary between workgroup ranges: the workgroup of
// boundary b (b = 1..G-1) merges the query block that boundary cuts, unless
// the boundary falls on a block edge or an earlier boundary cuts the same
// block. Thread r merges row r of the block's pieces.
template <int D, int BM, typename T>
__global__ __launch_bounds__(256) void fa_fwd_combine_kernel(Params p, StreamParams sp) {
  using M = Mma<T>;
  using pair = typename M::pair;
  constexpr int MAXP = 8;  // pieces whose weights are kept in registers
  const int b = blockIdx.x + 1;
  if (b >= sp.G) return;
  const int64_t gb = stream_start(sp, b);
  if (gb >= sp.total || gb % sp.ntb == 0) return;  // not inside a block
  const int bid = (int)(gb / sp.ntb);
  const int64_t g_first = (int64_t)bid * sp.ntb;
  const int64_t g_last = g_first + sp.ntb - 1;
  if (stream_start(sp, b - 1) > g_first) return;  // an earlier boundary merges this block
  auto owner = [&](int64_t g) {
    int w = (int)(g * sp.G / sp.total);
    while (w + 1 < sp.G && stream_start(sp, w + 1) <= g) ++w;
    while (w > 0 && stream_start(sp, w) > g) --w;
    return w;
  };
  const int wa = owner(g_first), wb = owner(g_last);
  const int head = bid / p.num_qb;
  const int qb = bid - head * p.num_qb;
  const int hb = head / p.H, hh = head - hb * p.H;
  // Workgroups with an empty range (fewer tiles than workgroups) wrote nothing.
  auto has_work = [&](int w) { return stream_start(sp, w + 1) > stream_start(sp, w); };
  // The block is the last segment of wa (its first, slot 0, if wa's range
  // starts at the block's first tile) and the first segment (slot 0) of
  // every later workgroup up to wb.
  auto piece = [&](int w) -> const float* {
    const int s = (w == wa && stream_start(sp, wa) < g_first) ? 1 : 0;
    return sp.part + ((size_t)w * 2 + s) * (size_t)(BM * (D + 3));
  };
  for (int r = threadIdx.x; r < BM; r += 256) {
    const int q_row = qb * BM + r;
    if (q_row >= p.Nq) continue;
    float m = -__builtin_inff();
    for (int w = wa; w <= wb; ++w)
      if (has_work(w)) m = vmax(m, piece(w)[D * BM + r]);
    float l = 0.f, n = 0.f;
    float f[MAXP];
    int np = 0;
    for (int w = wa; w <= wb; ++w) {
      if (!has_work(w)) continue;
      const float* pc = piece(w);
      const float fw = __builtin_amdgcn_exp2f(pc[D * BM + r] - m);
      if (np < MAXP) f[np] = fw;
      ++np;
      l += fw * pc[D * BM + BM + r];
      n += fw * pc[D * BM + 2 * BM + r];
    }
    const float inv = 1.0f / n;
    T* Oh = head_base<T>(p.o, p.so, hb, hh) + (int64_t)q_row * p.so.n;
    for (int d = 0; d < D; d += 2) {
      float a0 = 0.f, a1 = 0.f;
      int ip = 0;
      for (int w = wa; w <= wb; ++w) {
        if (!has_work(w)) continue;
        const float* pc = piece(w);
        const float fw = ip < MAXP ? f[ip] : __builtin_amdgcn_exp2f(pc[D * BM + r] - m);
        ++ip;
        a0 += fw * pc[d * BM + r];
        a1 += fw * pc[(d + 1) * BM + r];
      }
      *(pair*)(Oh + d) = M::cvt(a0 * inv, a1 * inv);
    }
    if (p.lse != nullptr) p.lse[(size_t)head * p.Nq + q_row] = 0.69314718055994531f * (m + log2f(l));
  }
}

}  // namespace fa
