// fa_device.hpp - gfx950 (CDNA4) device helpers shared by the attention
// kernels: vector types, the MFMA wrappers per element type, the swizzled LDS
// layout, HBM-to-LDS buffer loads, wait counters and partner-lane exchanges.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Word 3 of a raw buffer resource on gfx9: 32-bit data format, no swizzle.
constexpr int kBufferFlags = 0x00020000;

// Row sums of P. O is divided by the sum of the P values the P V product
// actually used (P rounded to the input type): for fp16 taken on the matrix
// cores, a 16x16x32 MFMA of a 0/1 selector against the P operand (see the
// kernels' row_sel); for bf16 on the vector units (kVecRowSum). Rounding
// errors of the individual weights then cancel against the same errors in
// the normaliser, so a row dominated by one key returns that key's V row to
// within the output's own rounding. For fp16 the log-sum-exp comes from the
// same sum (11 bits: ln of it moves by at most 2^-11); bf16 keeps 8 bits, so
// its log-sum-exp takes a second sum of the unrounded fp32 values (kLse32),
// accumulated per lane while P is formed.
template <typename T> struct Mma;
template <> struct Mma<_Float16> {
  typedef f16x8 vec;
  typedef f16x2 pair;
  static __device__ __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  // round two floats to nearest-even halves in one v_cvt_pk_f16_f32
  static __device__ __forceinline__ pair cvt(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_convertvector(f, pair);
  }
  static __device__ __forceinline__ vec selector(bool on) {
    const _Float16 x = on ? (_Float16)1.0f : (_Float16)0.0f;
    return vec{x, x, x, x, x, x, x, x};
  }
  static __device__ __forceinline__ f32x4 sel_sum(vec sel, vec pr, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(sel, pr, acc, 0, 0, 0);
  }
  static constexpr bool kLse32 = false;
  static __device__ __forceinline__ float lse_sum(float, float, float acc) { return acc; }
  static constexpr bool kVecRowSum = false;
  static __device__ __forceinline__ float rnd_sum(pair, float acc) { return acc; }
};
template <> struct Mma<__bf16> {
  typedef bf16x8 vec;
  typedef bf16x2 pair;
  static __device__ __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ pair cvt(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_convertvector(f, pair);
  }
  static __device__ __forceinline__ vec selector(bool on) {
    const __bf16 x = on ? (__bf16)1.0f : (__bf16)0.0f;
    return vec{x, x, x, x, x, x, x, x};
  }
  static __device__ __forceinline__ f32x4 sel_sum(vec sel, vec pr, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pr, acc, 0, 0, 0);
  }
  static constexpr bool kLse32 = true;
  static __device__ __forceinline__ float lse_sum(float p0, float p1, float acc) {
    return acc + (p0 + p1);
  }
  // The rounded sum is taken on the vector units instead, one v_dot2c_f32_bf16
  // per pair into a per-lane sum (measured 1-2% faster at d = 128 than the
  // selector MFMA, whose cycles the matrix cores there cannot spare).
  static constexpr bool kVecRowSum = true;
  static __device__ __forceinline__ float rnd_sum(pair pp, float acc) {
    const pair one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(pp, one, acc, false);
  }
};

// Key permutation inside a 32-key subtile: LDS row r holds key
// 16*((r/4)%2) + 4*(r/8) + r%4, which is the key that accumulator register
// i = 4*(r/8) + r%4 of a lane in half (r/4)%2 covers.
__device__ __forceinline__ int lds_row_to_key(int r) {
  return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}

// Byte offset of 16-byte chunk c of row r in an LDS tile with ROW_BYTES per
// row (32, 64, 128 or 256). Chunks are XOR-swizzled per row so that every read
// pattern of the kernel touches 16 distinct 16-byte bank groups of a
// 256-byte window per 16 lanes: one chunk of 16 consecutive rows (the MFMA
// A operands) and 2 adjacent chunks of 4 consecutive rows starting at a
// multiple of 4 (the transpose reads).
template <int ROW_BYTES>
__device__ __forceinline__ int lds_off(int r, int c) {
  static_assert(ROW_BYTES == 32 || ROW_BYTES == 64 || ROW_BYTES == 128 || ROW_BYTES == 256, "row size");
  int swz;
  if (ROW_BYTES == 256) swz = ((r & 7) << 1) | ((r >> 3) & 1);             // 1 row per window
  else if (ROW_BYTES == 128) swz = (((r >> 1) & 3) << 1) | ((r >> 3) & 1);  // 2 rows
  else if (ROW_BYTES == 64) swz = (r >> 2) & 3;                             // 4 rows
  else swz = (r >> 3) & 1;  // 8 rows of 2 chunks: rows r and r+8 swap chunks
  return r * ROW_BYTES + 16 * (c ^ swz);
}

// Byte offset of chunk c of row r in the forward's K and V tiles (rows of 2d
// bytes). Besides one chunk of 16 consecutive rows per 16 lanes (the K
// operand reads), the transpose reads of V^T straight from the V tile fetch 4
// chunks of each of 4 consecutive rows (from a multiple of 4) per 32 lanes;
// the swizzle puts those 4 rows in different 64-byte bank blocks of the
// 256-byte window, which lds_off does not for 128- and 256-byte rows.
template <int ROW_BYTES>
__device__ __forceinline__ int tile_off(int r, int c) {
  if constexpr (ROW_BYTES == 256) {
    const int swz = ((r & 3) << 2) | ((r >> 2) & 3);  // rows r..r+3: blocks 0..3
    return r * ROW_BYTES + 16 * (c ^ swz);
  } else if constexpr (ROW_BYTES == 128) {
    // two rows per window; rows r and r+2 take different 64-byte halves
    const int swz = (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
    return r * ROW_BYTES + 16 * (c ^ swz);
  } else {
    return lds_off<ROW_BYTES>(r, c);
  }
}

// One 16-byte-per-lane buffer load straight into LDS: lane l's bytes land at
// LDS address lds_addr + 16*l. Written as inline asm so that the compiler does
// not guard every LDS read with a wait for all such loads in flight; the
// kernel waits for them itself (wait_vmcnt) before the barrier that publishes
// a stage. M0 is set inside the same asm block; the load has no register
// result. M0 is a reserved register the compiler does not save around the
// block (hipcc warns about the clobber); that is safe here because nothing
// else in these kernels reads M0: in their gfx950 assembly every M0 write is
// one of these blocks' own, and no instruction that uses M0 (indirect
// register indexing, LDS-direct or GWS operations, messages) appears.
__device__ __forceinline__ void dma_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr,
                                           uint32_t voffset) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voffset), "s"(rsrc)
      : "memory", "m0");
}

// s_waitcnt for vector-memory count <= N only (other counters untouched).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Combine a value with the partner lane's (l ^ 32) through v_permlane32_swap,
// which swaps the upper 32 lanes of its first operand with the lower 32 lanes
// of its second: with both holding x, every lane ends up with x and x[l ^ 32]
// in the two registers. (Written as inline asm because the compiler builtin
// for this instruction drops its second result.) The s_nop pairs give the
// wait states around the cross-lane move.
__device__ __forceinline__ void swap_with_partner(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// IEEE maximum (v_maximum*_f32): unlike fmaxf it needs no canonicalising of
// its operands. Scores are never NaN for finite inputs.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max_with_partner(float x) {
  float a = x, b = x;
  swap_with_partner(a, b);
  return vmax(a, b);
}
__device__ __forceinline__ float sum_with_partner(float x) {
  float a = x, b = x;
  swap_with_partner(a, b);
  return a + b;
}

}  // namespace fa
