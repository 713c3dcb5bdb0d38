// fa_fp8.hip - the FP8 forward entry point of libfa.so: argument checks, grid
// computation and the launch of the gfx950 e4m3 forward kernel.
//
// The declarations and the contract live in include/fa.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_fwd_fp8.hpp"
#include "fa_host.hpp"

namespace {

typedef void (*Fp8Fn)(fa::Fp8Params);

// 4 waves of 32 query rows, 64-key tiles, a 4-stage ring (20 KB of LDS at
// d = 32, 40 KB at d = 64, 80 KB at d = 128).
template <int D, typename TO>
Fp8Fn pick_d(bool causal) {
  return causal ? fa::fa_fwd_fp8_kernel<D, 4, 4, true, TO> : fa::fa_fwd_fp8_kernel<D, 4, 4, false, TO>;
}
template <typename TO>
Fp8Fn pick_fp8(int64_t d, bool causal) {
  return d == 32 ? pick_d<32, TO>(causal) : (d == 64 ? pick_d<64, TO>(causal) : pick_d<128, TO>(causal));
}
constexpr int kRows = 128;  // query rows per workgroup
constexpr int kThreads = 256;

}  // namespace

extern "C" {

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
               float q_descale, float k_descale, float v_descale, int causal, int out_dtype,
               void* stream) {
  // ---- every check happens before the first HIP call
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FA_ERR_NULLPTR;
  if (out_dtype != FA_DTYPE_FP16 && out_dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 32 && d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  const int64_t lim = (int64_t)1 << 31;
  const int64_t head_lim = (int64_t)1 << 29;
  if (Nq > head_lim || Nk > head_lim || Nq * d >= head_lim || Nk * d >= head_lim) return FA_ERR_SHAPE;
  if (B > lim || H > lim || B * H >= lim) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
  if (!isfinite(scale) || !isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale) ||
      !(q_descale > 0.0f) || !(k_descale > 0.0f) || !(v_descale > 0.0f))
    return FA_ERR_SCALE;
  const float qk = scale * q_descale * k_descale;  // factor of the integer-grid scores
  if (!isfinite(qk)) return FA_ERR_SCALE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
  if (((uintptr_t)lse) & 3u) return FA_ERR_ALIGN;

  const int64_t num_qb = (Nq + kRows - 1) / kRows;
  const int64_t total = B * H * num_qb;
  if (total >= lim) return FA_ERR_SHAPE;
  const size_t q_bytes = (size_t)(B * H) * (size_t)(Nq * d);
  const size_t kv_bytes = (size_t)(B * H) * (size_t)(Nk * d);
  const size_t o_bytes = 2 * q_bytes;
  const size_t lse_bytes = (size_t)(B * H) * (size_t)Nq * 4;
  if (fa::overlaps(o, o_bytes, q, q_bytes) || fa::overlaps(o, o_bytes, k, kv_bytes) ||
      fa::overlaps(o, o_bytes, v, kv_bytes))
    return FA_ERR_ALIAS;
  if (lse != nullptr &&
      (fa::overlaps(lse, lse_bytes, q, q_bytes) || fa::overlaps(lse, lse_bytes, k, kv_bytes) ||
       fa::overlaps(lse, lse_bytes, v, kv_bytes) || fa::overlaps(lse, lse_bytes, o, o_bytes)))
    return FA_ERR_ALIAS;

  fa::Fp8Params pp;
  fa::Params& p = pp.b;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = (int)B;
  p.H = (int)H;
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.num_qb = (int)num_qb;
  p.total = (int)total;
  p.xcd_q = fa::xcd_split(total).q;
  p.xcd_r = fa::xcd_split(total).r;
  if (causal) {  // the order of the 16-bit forward of the same shape
    const fa::CausalOrder co = fa::causal_order(B * H, 2 * Nk * d * 2);
    p.group = co.group;
    p.launch_order = co.launch_order;
  } else {
    p.group = 1;
    p.launch_order = 0;
  }
  p.nkt = 0;
  if (qk == 0.0f) {  // every score is 0: zero Q, any positive factor works
    p.c = 1.0f;
    p.q_and = 0u;
    p.q_xor = 0u;
  } else {  // a negative factor is carried by Q's sign bits (one per byte)
    p.c = fabsf(qk) * 1.4426950408889634f;
    p.q_and = 0xffffffffu;
    p.q_xor = qk < 0.0f ? 0x80808080u : 0u;
  }
  pp.v_scale = v_descale;

  const Fp8Fn fn = out_dtype == FA_DTYPE_FP16 ? pick_fp8<_Float16>(d, causal != 0)
                                              : pick_fp8<__bf16>(d, causal != 0);
  void* args[] = {&pp};
  const hipError_t e = hipLaunchKernel((const void*)fn, dim3((unsigned)total), dim3(kThreads), args, 0,
                                       (hipStream_t)stream);
  return fa::launch_status(e);
}

}  // extern "C"
