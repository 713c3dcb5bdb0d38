// fa_std.hip - entry points of the standard (unfused) attention baseline:
// argument checks and the launch of the three kernels of fa_std_kernel.hpp.
//
// The declarations and the contract live in include/fa.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_host.hpp"
#include "fa_std_kernel.hpp"

namespace {

typedef void (*StdFn)(fa::StdParams);

template <typename T>
StdFn scores_fn(int64_t d) {
  return d == 32 ? fa::fa_std_scores_kernel<32, T>
                 : (d == 64 ? fa::fa_std_scores_kernel<64, T> : fa::fa_std_scores_kernel<128, T>);
}
template <typename T>
StdFn pv_fn(int64_t d) {
  return d == 32 ? fa::fa_std_pv_kernel<32, T>
                 : (d == 64 ? fa::fa_std_pv_kernel<64, T> : fa::fa_std_pv_kernel<128, T>);
}
// The softmax variant keeping a row of NkP keys in registers (4-key groups
// per thread: 1, 2, 4, 8 or 16), or the streaming one past 16384 keys.
template <typename T>
StdFn softmax_fn(int64_t nkp) {
  const int64_t groups = (nkp / 4 + 255) / 256;
  if (groups <= 1) return fa::fa_std_softmax_kernel<1, T>;
  if (groups <= 2) return fa::fa_std_softmax_kernel<2, T>;
  if (groups <= 4) return fa::fa_std_softmax_kernel<4, T>;
  if (groups <= 8) return fa::fa_std_softmax_kernel<8, T>;
  if (groups <= 16) return fa::fa_std_softmax_kernel<16, T>;
  return fa::fa_std_softmax_kernel<0, T>;
}

}  // namespace

extern "C" {

int64_t fa_std_row_stride(int64_t Nk) {
  if (Nk < 1 || Nk > ((int64_t)1 << 29)) return -1;
  return (Nk + 63) / 64 * 64;
}

int fa_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse, float* s, void* p,
               int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
               int dtype, void* stream) {
  // ---- every check happens before the first HIP call
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || s == nullptr || p == nullptr)
    return FA_ERR_NULLPTR;
  if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 32 && d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  const int64_t head_lim = (int64_t)1 << 29;
  if (Nq > head_lim || Nk > head_lim || Nq * d >= head_lim || Nk * d >= head_lim) return FA_ERR_SHAPE;
  const int64_t nkp = (Nk + 63) / 64 * 64;
  // one head's S and P are addressed with 32-bit offsets: Nq * NkP < 2^29
  if (Nq * nkp >= head_lim) return FA_ERR_SHAPE;
  const int64_t lim = (int64_t)1 << 31;
  if (B > lim || H > lim || B * H >= lim) return FA_ERR_SHAPE;
  const int64_t nqb = (Nq + 127) / 128, nkb = (Nk + 63) / 64;
  if (B * H * nqb * nkb >= lim || B * H * Nq >= lim) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)s | (uintptr_t)p) & 15u)
    return FA_ERR_ALIGN;
  if (((uintptr_t)lse) & 3u) return FA_ERR_ALIGN;
  const size_t qo_bytes = (size_t)(B * H * Nq * d * 2), kv_bytes = (size_t)(B * H * Nk * d * 2);
  const size_t s_bytes = (size_t)(B * H * Nq) * (size_t)nkp * 4, p_bytes = s_bytes / 2;
  const size_t lse_bytes = (size_t)(B * H * Nq) * 4;
  struct Span {
    const void* a;
    size_t n;
  } in[3] = {{q, qo_bytes}, {k, kv_bytes}, {v, kv_bytes}},
    out[4] = {{o, qo_bytes}, {s, s_bytes}, {p, p_bytes}, {lse, lse_bytes}};
  for (int i = 0; i < 4; ++i) {
    if (out[i].a == nullptr) continue;
    for (int j = 0; j < 3; ++j)
      if (fa::overlaps(out[i].a, out[i].n, in[j].a, in[j].n)) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (out[j].a != nullptr && fa::overlaps(out[i].a, out[i].n, out[j].a, out[j].n)) return FA_ERR_ALIAS;
  }

  fa::StdParams sp;
  sp.q = q;
  sp.k = k;
  sp.v = v;
  sp.o = o;
  sp.lse = lse;
  sp.s = s;
  sp.p = p;
  sp.B = (int)B;
  sp.H = (int)H;
  sp.Nq = (int)Nq;
  sp.Nk = (int)Nk;
  sp.NkP = (int)nkp;
  sp.scale = scale;
  sp.causal = causal;
  sp.nqb = (int)nqb;
  sp.nkb = (int)nkb;
  const bool f16 = dtype == FA_DTYPE_FP16;
  const StdFn k1 = f16 ? scores_fn<_Float16>(d) : scores_fn<__bf16>(d);
  const StdFn k2 = f16 ? softmax_fn<_Float16>(nkp) : softmax_fn<__bf16>(nkp);
  const StdFn k3 = f16 ? pv_fn<_Float16>(d) : pv_fn<__bf16>(d);
  void* args[] = {&sp};
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipLaunchKernel((const void*)k1, dim3((unsigned)(B * H * nqb * nkb)), dim3(256), args, 0, st);
  if (e == hipSuccess)
    e = hipLaunchKernel((const void*)k2, dim3((unsigned)(B * H * Nq)), dim3(256), args, 0, st);
  if (e == hipSuccess)
    e = hipLaunchKernel((const void*)k3, dim3((unsigned)(B * H * nqb)), dim3(256), args, 0, st);
  return fa::launch_status(e);
}

}  // extern "C"
