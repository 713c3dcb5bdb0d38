// fa_fwd_kernel.hpp - the exact-attention forward kernel for gfx950 (CDNA4).
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
//   * A wave owns 32 query rows. Scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{f16,bf16}: K rows are the A operand (read from
//     LDS), the wave's Q rows are the B operand and stay in VGPRs for the
//     whole kernel. In the 32x32 accumulator layout lane l holds column l%32
//     (its query) and 16 rows (keys), so a query's scores sit in two lanes
//     (l and l^32) and the row reductions are in-register plus one
//     cross-lane exchange with the partner lane.
//   * K rows are written to LDS in a permuted order so that accumulator
//     register i of lane l holds key 16*(l/32)+i of its 32-key subtile. Those
//     registers, rounded to fp16/bf16, are directly the B operand (P^T) of the
//     P V product O^T += V^T P^T; V is stored transposed in LDS (Vt[d][key])
//     so each lane's A operand is one 16-byte LDS read.
//   * O^T accumulates in fp32 MFMA accumulators: lane l holds d/2 elements of
//     its query's output row.
//   * K/V tiles are fetched with 128-bit global loads into registers one tile
//     ahead and written into the other half of a double-buffered LDS, so the
//     fetch of tile j+1 overlaps the math of tile j; one barrier per tile.
//   * exp is v_exp_f32 (2^x) on scores pre-multiplied by scale*log2(e), folded
//     into one FMA with the running maximum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
  float c;        // |scale| * log2(e), or 1 when scale == 0
  uint32_t q_and; // applied to each 32-bit word of Q: ~0 normally, 0 when scale == 0
  uint32_t q_xor; // 0x80008000 flips both halves' sign when scale < 0
};

template <typename T> struct Mma;
template <> struct Mma<_Float16> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    _Float16 a = (_Float16)lo, b = (_Float16)hi;  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
};
template <> struct Mma<__bf16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
};

// Inverse of the key permutation inside a 32-key subtile: key x = 16*g + i is
// stored in LDS row 8*(i/4) + 4*g + i%4, which is the accumulator row that
// register i of a lane in half g covers.
__device__ __forceinline__ int key_to_lds_row(int x) {
  return ((x & 15) >> 2) * 8 + (x >> 4) * 4 + (x & 3);
}

// Partner-lane (l ^ 32) combine through ds_bpermute.
__device__ __forceinline__ float partner(float x) {
  const int src = ((int)__lane_id() ^ 32) << 2;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, x)));
}
__device__ __forceinline__ float max_with_partner(float x) { return fmaxf(x, partner(x)); }
__device__ __forceinline__ float sum_with_partner(float x) { return x + partner(x); }

// Workgroup id -> (head, query block). Workgroups are dispatched round-robin
// over the 8 XCDs; the remap gives each XCD a contiguous range of logical ids
// so the query blocks of one head share that XCD's L2 for its K/V. Inside the
// range, heads are taken in groups; for causal masks the heaviest query
// blocks (most key tiles) of a group go first.
template <bool CAUSAL>
__device__ __forceinline__ void work_item(const Params& p, int bid, int& head, int& qb) {
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int L = xcd * p.xcd_q + (xcd < p.xcd_r ? xcd : p.xcd_r) + slot;
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

template <int D, int BN, int NW, bool CAUSAL, typename T>
__global__ __launch_bounds__(NW * 64) void fa_fwd_kernel(Params p) {
  using M = Mma<T>;
  using vec = typename M::vec;
  constexpr int BM = 32 * NW;        // query rows per workgroup
  constexpr int NT = 64 * NW;        // threads per workgroup
  constexpr int KS = D / 16;         // k-steps of the QK^T contraction
  constexpr int NSUB = BN / 32;      // 32-key subtiles per tile
  constexpr int NDT = D / 32;        // 32-wide d tiles of O
  constexpr int KSTR = D + 8;        // LDS row stride of K (elements), 16 B pad
  constexpr int VSTR = BN + 8;       // LDS row stride of V^T (elements), 16 B pad
  constexpr int KCHUNKS = BN * D / 8;          // 16-byte K chunks per tile
  constexpr int VUNITS = (BN / 4) * (D / 8);   // 4-key x 8-d V blocks per tile
  constexpr int KCH = (KCHUNKS + NT - 1) / NT; // per thread (the last may be partial)
  constexpr int VUN = (VUNITS + NT - 1) / NT;
  static_assert(KCHUNKS % NT == 0 || KCHUNKS < NT, "K tile must split evenly");
  static_assert(VUNITS % NT == 0 || VUNITS < NT, "V tile must split evenly");

  __shared__ __attribute__((aligned(16))) T smem_k[2][BN * KSTR];
  __shared__ __attribute__((aligned(16))) T smem_v[2][D * VSTR];

  int head, qb;
  work_item<CAUSAL>(p, blockIdx.x, head, qb);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;  // which 16-key half of a subtile this lane holds
  const int r32 = lane & 31;   // this lane's query within the wave

  const int Nq = p.Nq, Nk = p.Nk;
  const T* __restrict__ Qh = (const T*)p.q + (size_t)head * Nq * D;
  const T* __restrict__ Kh = (const T*)p.k + (size_t)head * Nk * D;
  const T* __restrict__ Vh = (const T*)p.v + (size_t)head * Nk * D;

  const int wave_q0 = qb * BM + wave * 32;
  const int q_row = wave_q0 + r32;

  // ---- this lane's query row as B-operand fragments (8 elements per k-step)
  vec qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (q_row < Nq) w = *(const u32x4*)(Qh + (size_t)q_row * D + 16 * s + 8 * half);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (w[e] & p.q_and) ^ p.q_xor;
    qf[s] = __builtin_bit_cast(vec, w);
  }

  int kv_end = Nk;
  if (CAUSAL) {
    const int last = qb * BM + BM;  // keys < last can be visible to this block
    kv_end = last < Nk ? last : Nk;
  }
  const int ntiles = (kv_end + BN - 1) / BN;

  f32x16 oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[t][i] = 0.f;
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float c = p.c;

  // ---- tile fetch (global -> registers) and store (registers -> LDS)
  u32x4 kreg[KCH];
  u32x4 vreg[VUN][4];
  auto fetch = [&](int j) {
    const int kb = j * BN;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + NT * i;
      const int row = ch / (D / 8), col = ch % (D / 8);
      const int key = kb + row;
      u32x4 w = {0u, 0u, 0u, 0u};
      if ((KCHUNKS >= NT || ch < KCHUNKS) && key < Nk)
        w = *(const u32x4*)(Kh + (size_t)key * D + col * 8);
      kreg[i] = w;
    }
#pragma unroll
    for (int i = 0; i < VUN; ++i) {
      const int u = tid + NT * i;
      const int g4 = u % (BN / 4), c8 = u / (BN / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + 4 * g4 + r;
        u32x4 w = {0u, 0u, 0u, 0u};
        if ((VUNITS >= NT || u < VUNITS) && key < Nk)
          w = *(const u32x4*)(Vh + (size_t)key * D + c8 * 8);
        vreg[i][r] = w;
      }
    }
  };
  auto store = [&](int buf) {
    T* ks = smem_k[buf];
    T* vs = smem_v[buf];
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + NT * i;
      if (KCHUNKS < NT && ch >= KCHUNKS) continue;
      const int row = ch / (D / 8), col = ch % (D / 8);
      const int lrow = (row & ~31) | key_to_lds_row(row & 31);
      *(u32x4*)(ks + lrow * KSTR + col * 8) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VUN; ++i) {
      const int u = tid + NT * i;
      if (VUNITS < NT && u >= VUNITS) continue;
      const int g4 = u % (BN / 4), c8 = u / (BN / 4);
      // transpose 4 keys x 8 d into 8 rows of Vt holding 4 keys each
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const uint32_t a0 = vreg[i][0][w2], a1 = vreg[i][1][w2];
        const uint32_t a2 = vreg[i][2][w2], a3 = vreg[i][3][w2];
        u32x2 lo, hi;  // d = 8*c8 + 2*w2 (low halves) and + 1 (high halves)
        lo[0] = (a0 & 0xffffu) | (a1 << 16);
        lo[1] = (a2 & 0xffffu) | (a3 << 16);
        hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
        hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        const int d0 = 8 * c8 + 2 * w2;
        *(u32x2*)(vs + d0 * VSTR + 4 * g4) = lo;
        *(u32x2*)(vs + (d0 + 1) * VSTR + 4 * g4) = hi;
      }
    }
  };

  fetch(0);
  store(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) fetch(j + 1);
    const int kb = j * BN;
    // A tile whose first key lies after every row of this wave is fully
    // masked for it; the wave only helps move data.
    const bool active = !CAUSAL || kb <= wave_q0 + 31;
    if (active) {
      const T* ks = smem_k[buf];
      const T* vs = smem_v[buf];
      // ---- S^T = K Q^T for the BN keys of this tile
      f32x16 sacc[NSUB];
#pragma unroll
      for (int t = 0; t < NSUB; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[t][i] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const vec a = *(const vec*)(ks + (32 * t + r32) * KSTR + 16 * s + 8 * half);
          sacc[t] = M::run(a, qf[s], sacc[t]);
        }
      }
      // ---- tail / causal masking (only on boundary tiles)
      const bool tail = kb + BN > Nk;
      const bool diag = CAUSAL && (kb + BN - 1 > wave_q0);
      if (tail || diag) {
#pragma unroll
        for (int t = 0; t < NSUB; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb + 32 * t + 16 * half + i;
            const bool vis = key < Nk && (!CAUSAL || key <= q_row);
            sacc[t][i] = vis ? sacc[t][i] : -__builtin_inff();
          }
      }
      // ---- online softmax update
      float mx = sacc[0][0];
#pragma unroll
      for (int t = 0; t < NSUB; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[t][i]);
      mx = max_with_partner(mx);
      float m_new = fmaxf(m_run, mx * c);
      m_new = (m_new == -__builtin_inff()) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      if (__any(m_new > m_run)) {
#pragma unroll
        for (int t = 0; t < NDT; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[t][i] *= alpha;
      }
      l_run *= alpha;
      m_run = m_new;
      const float negm = -m_new;
      vec pf[NSUB][2];
#pragma unroll
      for (int t = 0; t < NSUB; ++t) {
        u32x4 w0, w1;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i], c, negm));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i + 1], c, negm));
          const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i + 8], c, negm));
          const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i + 9], c, negm));
          l_run += (p0 + p1) + (p2 + p3);
          w0[i / 2] = M::pack(p0, p1);
          w1[i / 2] = M::pack(p2, p3);
        }
        pf[t][0] = __builtin_bit_cast(vec, w0);
        pf[t][1] = __builtin_bit_cast(vec, w1);
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int t = 0; t < NSUB; ++t)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const vec a = *(const vec*)(vs + (32 * dt + r32) * VSTR + 32 * t + 16 * half + 8 * s2);
            oacc[dt] = M::run(a, pf[t][s2], oacc[dt]);
          }
    }
    if (j + 1 < ntiles) store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l)
  const float l_tot = sum_with_partner(l_run);
  const float inv = 1.0f / l_tot;
  if (q_row < Nq) {
    T* Oh = (T*)p.o + (size_t)head * Nq * D + (size_t)q_row * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = M::pack(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv);
        w[1] = M::pack(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
        *(u32x2*)(Oh + 32 * dt + 8 * g + 4 * half) = w;
      }
    if (p.lse != nullptr && half == 0)
      p.lse[(size_t)head * Nq + q_row] = 0.69314718055994531f * (m_run + log2f(l_tot));
  }
}

}  // namespace fa
