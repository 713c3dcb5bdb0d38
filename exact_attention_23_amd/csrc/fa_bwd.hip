// fa_bwd.hip - the backward entry points of libfa.so: argument checks, grid
// computation and the launch of the three gfx950 backward kernels.
//
// The declarations and the contract live in include/fa.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <atomic>

#include "../../include/fa.h"
#include "fa_bwd_kernel.hpp"
#include "fa_host.hpp"

namespace {

typedef void (*BwdFn)(fa::BwdParams);

struct BwdKernels {
  BwdFn pre, dkdv, dq;
  int pre_rows;      // query rows per workgroup of the D/LSE kernel
  int dkdv_threads;  // threads per dK/dV workgroup
  int dkdv_bn;       // keys per dK/dV workgroup
  int dq_threads;    // threads per dQ workgroup
  int dq_bm;         // query rows per dQ workgroup
};

// Waves per workgroup and ring stages: 4 waves of 32 keys (dK/dV) or 32 query
// rows (dQ). At d = 128 the operand and accumulator registers would leave one
// 4-wave workgroup per CU, one wave per SIMD; both kernels take 8 waves there
// instead (two per SIMD, each staged tile shared by twice as many waves), at
// the price of a few spilled registers, which measured 29-30% faster. The
// dQ ring has 3 stages at d = 128 to fit LDS.
#ifndef FA_BWD_SA
#define FA_BWD_SA 3
#endif
#ifndef FA_BWD_SB128
#define FA_BWD_SB128 4
#endif
template <int D, bool C, typename T>
BwdKernels make_bwd() {
  constexpr int NWA = D == 128 ? 8 : 4, SA = FA_BWD_SA;
  constexpr int NWB = D == 128 ? 8 : 4;
  constexpr int SB = D == 128 ? FA_BWD_SB128 : 4;
  return {fa::fa_bwd_pre_kernel<D, T>,
          fa::fa_bwd_dkdv_kernel<D, NWA, SA, C, T>,
          fa::fa_bwd_dq_kernel<D, NWB, SB, C, T>,
          256 / (D / 8),
          64 * NWA,
          32 * NWA,
          64 * NWB,
          32 * NWB};
}

template <typename T>
BwdKernels pick_bwd(int64_t d, bool causal) {
  switch (d) {
    case 32: return causal ? make_bwd<32, true, T>() : make_bwd<32, false, T>();
    case 64: return causal ? make_bwd<64, true, T>() : make_bwd<64, false, T>();
    default: return causal ? make_bwd<128, true, T>() : make_bwd<128, false, T>();
  }
}

// The checks of fa_bwd_ex that do not involve the workspace.
int check_args(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Nq,
               int64_t Nk, int64_t d, float scale, int causal, int dtype) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || dout == nullptr ||
      lse == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return FA_ERR_NULLPTR;
  if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 32 && d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  const int64_t lim = (int64_t)1 << 31;
  const int64_t head_lim = (int64_t)1 << 29;
  if (Nq > head_lim || Nk > head_lim || Nq * d >= head_lim || Nk * d >= head_lim) return FA_ERR_SHAPE;
  if (B > lim || H > lim || B * H >= lim) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
       (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15u)
    return FA_ERR_ALIGN;
  if (((uintptr_t)lse) & 3u) return FA_ERR_ALIGN;
  return FA_OK;
}

// Outputs and the workspace (when not null) are written: none may overlap an
// input, and they may not overlap each other.
int check_alias(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, const void* workspace,
                int64_t ws_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d) {
  const size_t q_bytes = (size_t)(B * H) * (size_t)(Nq * d) * 2;
  const size_t kv_bytes = (size_t)(B * H) * (size_t)(Nk * d) * 2;
  const size_t lse_bytes = (size_t)(B * H) * (size_t)Nq * 4;
  struct Range {
    const void* p;
    size_t n;
  };
  const Range inputs[] = {{q, q_bytes}, {k, kv_bytes}, {v, kv_bytes}, {o, q_bytes},
                          {dout, q_bytes}, {lse, lse_bytes}};
  const Range written[] = {{dq, q_bytes}, {dk, kv_bytes}, {dv, kv_bytes},
                           {workspace, workspace != nullptr ? (size_t)ws_bytes : 0}};
  for (const Range& w : written) {
    for (const Range& in : inputs)
      if (fa::overlaps(w.p, w.n, in.p, in.n)) return FA_ERR_ALIAS;
    for (const Range& w2 : written)
      if (&w2 != &w && fa::overlaps(w.p, w.n, w2.p, w2.n)) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

hipError_t launch(BwdFn fn, int64_t grid, int threads, fa::BwdParams& p, hipStream_t stream) {
  void* args[] = {&p};
  return hipLaunchKernel((const void*)fn, dim3((unsigned)grid), dim3((unsigned)threads), args, 0, stream);
}

}  // namespace

extern "C" {

int64_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Nq) {
  if (B < 1 || H < 1 || Nq < 1) return -1;
  const int64_t lim = (int64_t)1 << 31;
  if (B >= lim || H >= lim || B * H >= lim || Nq > ((int64_t)1 << 29)) return -1;
  return B * H * ((Nq + 31) / 32) * 256;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace,
           int64_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
           float scale, int causal, int dtype, void* stream) {
  return fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, Nq, Nk, d,
                   scale, causal, dtype, FA_BWD_ALL, stream);
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, void* dq, void* dk, void* dv, void* workspace,
              int64_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
              float scale, int causal, int dtype, int kernels, void* stream) {
  // ---- every check happens before the first HIP call
  const int st0 = check_args(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, d, scale, causal, dtype);
  if (st0 != FA_OK) return st0;
  const int64_t lim = (int64_t)1 << 31;
  const int64_t ws_need = fa_bwd_workspace_bytes(B, H, Nq);
  if (workspace == nullptr || ((uintptr_t)workspace & 15u) || ws_need < 0 || workspace_bytes < ws_need)
    return FA_ERR_WORKSPACE;

  const BwdKernels ker = dtype == FA_DTYPE_FP16 ? pick_bwd<_Float16>(d, causal != 0)
                                                : pick_bwd<__bf16>(d, causal != 0);
  const int64_t nrec = (Nq + 31) / 32;
  const int64_t pre_grid = (B * H * nrec * 32 + ker.pre_rows - 1) / ker.pre_rows;
  const int64_t nkb = (Nk + ker.dkdv_bn - 1) / ker.dkdv_bn;
  const int64_t nqb = (Nq + ker.dq_bm - 1) / ker.dq_bm;
  const int64_t dkdv_grid = B * H * nkb;
  const int64_t dq_grid = B * H * nqb;
  if (pre_grid >= lim || dkdv_grid >= lim || dq_grid >= lim) return FA_ERR_SHAPE;

  const int st1 = check_alias(q, k, v, o, dout, lse, dq, dk, dv, workspace, ws_need, B, H, Nq, Nk, d);
  if (st1 != FA_OK) return st1;

  if (kernels < 1 || kernels > FA_BWD_ALL) return FA_ERR_PATH;

  fa::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.aux = (float*)workspace;
  p.B = (int)B;
  p.H = (int)H;
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.nrec = (int)nrec;
  // Causal blocks in the forward's order (fa::causal_order): a dK/dV block
  // streams its head's Q and dO, a dQ block its head's K and V.
  if (causal) {
    const fa::CausalOrder co = fa::causal_order(B * H, 2 * Nq * d * 2);
    p.group = co.group;
    p.launch_order = co.launch_order;
  } else {
    p.group = 1;
    p.launch_order = 0;
  }
  p.c = scale * fa::kLog2e;
  p.scale = scale;
  hipStream_t st = (hipStream_t)stream;

  hipError_t e = hipSuccess;
  if (kernels & FA_BWD_PRE) {
    p.nblk = 0;
    p.xcd_q = p.xcd_r = 0;
    e = launch(ker.pre, pre_grid, 256, p, st);
    if (e != hipSuccess) return fa::launch_status(e);
  }
  if (kernels & FA_BWD_DKDV) {
    p.nblk = (int)nkb;
    p.xcd_q = fa::xcd_split(dkdv_grid).q;
    p.xcd_r = fa::xcd_split(dkdv_grid).r;
    e = launch(ker.dkdv, dkdv_grid, ker.dkdv_threads, p, st);
    if (e != hipSuccess) return fa::launch_status(e);
  }
  if (kernels & FA_BWD_DQ) {
    p.nblk = (int)nqb;
    p.xcd_q = fa::xcd_split(dq_grid).q;
    p.xcd_r = fa::xcd_split(dq_grid).r;
    e = launch(ker.dq, dq_grid, ker.dq_threads, p, st);
  }
  return fa::launch_status(e);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// fa_bwd_noalloc: fa_bwd with its D/LSE records in a file-scope device array
// instead of a caller's workspace, for callers that cannot allocate.
namespace {

constexpr int64_t kScratchBytes = FA_BWD_NOALLOC_SCRATCH_BYTES;

// One copy per GPU the library runs on, held until the process ends. In host
// code `scratch` only names the symbol; its device address (per device) comes
// from hipGetSymbolAddress and is the only form passed to kernels.
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call on each device, with that device current), or null on failure.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch[dev].store(ptr, std::memory_order_release);  // the same address for every caller
  }
  return ptr;
}

}  // namespace

extern "C" {

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Nq,
                   int64_t Nk, int64_t d, float scale, int causal, int dtype, void* stream) {
  // ---- every check happens before the first HIP call
  const int st0 = check_args(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, d, scale, causal, dtype);
  if (st0 != FA_OK) return st0;
  const int64_t need = fa_bwd_workspace_bytes(B, H, Nq);
  if (need < 0 || need > kScratchBytes) return FA_ERR_SCRATCH;
  const int st1 = check_alias(q, k, v, o, dout, lse, dq, dk, dv, nullptr, 0, B, H, Nq, Nk, d);
  if (st1 != FA_OK) return st1;
  void* ptr = scratch_ptr();
  if (ptr == nullptr) return fa::launch_status(hipErrorInvalidSymbol);
  // The D/LSE pass rewrites every record the other two kernels read (padding
  // rows included), so nothing left by an earlier call needs clearing.
  return fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, ptr, kScratchBytes, B, H, Nq, Nk, d, scale,
                   causal, dtype, FA_BWD_ALL, stream);
}

}  // extern "C"
