// fa_api.hip - the forward entry points of libfa.so: argument checks, tile
// selection, grid computation and the launch of the gfx950 forward kernels.
//
// The declarations and the contract live in include/fa.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_host.hpp"
#include "fa_fwd16.hpp"
#include "fa_fwd_kernel.hpp"
#include "fa_fwd_short.hpp"
#include "fa_fwd_stream.hpp"

namespace {

typedef void (*KernelFn)(fa::Params);

struct Variant {
  KernelFn fn;
  int bm;       // query rows per workgroup
  int threads;  // threads per workgroup
};

// Tile shapes per head width: NW waves of RB 32-row blocks, BN keys per tile,
// S LDS stages, whether the software-pipelined loop is used, and whether V^T
// goes through a transposed LDS copy (VT = 1) or is read from the V tile
// directly (VT = 0).
template <int D, int BN, int NW, int RB, int S, bool PIPE, int VT, typename T>
Variant make_variant(bool causal) {
  Variant v;
  v.fn = causal ? fa::fa_fwd_kernel<D, BN, NW, RB, S, PIPE, VT, true, T>
                : fa::fa_fwd_kernel<D, BN, NW, RB, S, PIPE, VT, false, T>;
  v.bm = 32 * RB * NW;
  v.threads = 64 * NW;
  return v;
}

// Tile configuration per head width as (D, BN, NW, RB, S, PIPE, VT). A build
// can override them with -DFA_TILES_D32=... etc. to compare configurations.
// All three read V^T straight from the V tiles (VT = 0); measured against the
// transposed copy (same box, interleaved): 470 vs 480 us (yolo80b16), 2129
// vs 2148 us (long16k). At d = 64 the smaller LDS footprint lets three
// 4-wave workgroups of one 32-row block per wave share a CU (155
// registers): 409 vs 417 us on seq2048 with a 3-stage ring (48 KB), 393 vs
// 402 us with a 2-stage ring (32 KB). Measured and not kept: the pipelined
// loop at d = 64 (408 vs 402) and d = 128 (2138 vs 2087), one row block per
// wave at d = 32 (four workgroups per CU: 467 vs 461).
#ifndef FA_TILES_D32
#define FA_TILES_D32 32, 64, 4, 2, 4, true, 0
#endif
#ifndef FA_TILES_D64
#define FA_TILES_D64 64, 64, 4, 1, 2, false, 0
#endif
#ifndef FA_TILES_D128
#define FA_TILES_D128 128, 64, 8, 1, 4, false, 0
#endif

// The tiled forward (fa_fwd16.hpp): 16x16x32 matrix instructions, NW waves of
// QB 16-row query blocks, S LDS stages, per head width as (D, NW, QB, S); a
// build can override them with -DFA_TILES16_D32=... etc. Against the 32x32x16
// kernel above (fa_fwd_kernel.hpp, which the persistent form still uses),
// same box, interleaved: 432 vs 438 us (yolo80b16), 353 vs 364 us (seq2048),
// 2019 vs 2055 us (long16k). Measured and not kept: four query blocks per
// wave (d = 32: 452 vs 442 us; d = 64, two waves per SIMD: 361 vs 355 us), a
// 2-stage ring at d = 32 (432 vs 430) and a 3-stage one at d = 64 (365 vs
// 352), constant ring stages at d = 128 (2057 vs 2019).
#ifndef FA_TILES16_D32
#define FA_TILES16_D32 32, 4, 2, 4
#endif
#ifndef FA_TILES16_D64
#define FA_TILES16_D64 64, 4, 2, 2
#endif
#ifndef FA_TILES16_D128
#define FA_TILES16_D128 128, 8, 2, 4
#endif
template <int D, int NW, int QB, int S, typename T>
Variant make_variant16(bool causal) {
  Variant v;
  v.fn = causal ? fa::fa_fwd16_kernel<D, NW, QB, S, true, T> : fa::fa_fwd16_kernel<D, NW, QB, S, false, T>;
  v.bm = 16 * QB * NW;
  v.threads = 64 * NW;
  return v;
}

template <typename T>
Variant pick(int64_t d, bool causal) {
  switch (d) {
    case 32: return make_variant16<FA_TILES16_D32, T>(causal);
    case 64: return make_variant16<FA_TILES16_D64, T>(causal);
    default: return make_variant16<FA_TILES16_D128, T>(causal);
  }
}

// The persistent (stream) form of the same tile shapes, full masks only.
typedef void (*StreamFn)(fa::Params, fa::StreamParams);
struct StreamVariant {
  StreamFn fn, combine;
  int bm, threads;
};
template <int D, int BN, int NW, int RB, int S, bool PIPE, int VT, typename T>
StreamVariant make_stream() {
  return {fa::fa_fwd_stream_kernel<D, BN, NW, RB, S, PIPE, VT, T>,
          fa::fa_fwd_combine_kernel<D, 32 * RB * NW, T>, 32 * RB * NW, 64 * NW};
}
template <typename T>
StreamVariant pick_stream(int64_t d) {
  switch (d) {
    case 32: return make_stream<FA_TILES_D32, T>();
    case 64: return make_stream<FA_TILES_D64, T>();
    default: return make_stream<FA_TILES_D128, T>();
  }
}
StreamVariant pick_stream_dt(int dtype, int64_t d) {
  return dtype == FA_DTYPE_FP16 ? pick_stream<_Float16>(d) : pick_stream<__bf16>(d);
}

// Resident workgroups of the stream kernel on the current device (0 if the
// query fails).
int64_t stream_grid(const StreamVariant& sv) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)sv.fn, sv.threads, 0) !=
          hipSuccess ||
      per_cu < 1)
    return 0;
  return (int64_t)per_cu * fa::device_cus();
}

// The short-range kernel for one head width and tile count: its launch
// function and how many of its workgroups a compute unit holds (LDS for
// NWMAX waves, at most 16 waves).
template <typename T>
struct ShortVariant {
  KernelFn fn;
  int per_cu;
};
template <int D, int NWMAX, int QB, typename T>
ShortVariant<T> short_of(bool causal) {
  constexpr int lds = NWMAX * fa::kShortRegion<D, QB> + 3 * NWMAX * 16 * QB * 4;
  constexpr int by_lds = (160 * 1024) / lds;
  constexpr int by_waves = 16 / NWMAX;
  constexpr int per_cu = by_lds < by_waves ? by_lds : by_waves;
  return {causal ? fa::fa_fwd_short_kernel<D, NWMAX, QB, true, T> : fa::fa_fwd_short_kernel<D, NWMAX, QB, false, T>,
          per_cu < 1 ? 1 : per_cu};
}
template <int D, int QB, typename T>
ShortVariant<T> make_short_qb(bool causal, int64_t tiles) {
  if constexpr (D == 128) {
    return short_of<128, fa::kShortMaxWaves<128>, QB, T>(causal);
  } else {
    if (tiles <= 8) return short_of<D, 8, QB, T>(causal);
    return short_of<D, 16, QB, T>(causal);
  }
}
template <int D, typename T>
ShortVariant<T> make_short(bool causal, int64_t tiles, int qb) {
  return qb == 1 ? make_short_qb<D, 1, T>(causal, tiles) : make_short_qb<D, 2, T>(causal, tiles);
}
template <typename T>
ShortVariant<T> pick_short(int64_t d, bool causal, int64_t tiles, int qb) {
  switch (d) {
    case 32: return make_short<32, T>(causal, tiles, qb);
    case 64: return make_short<64, T>(causal, tiles, qb);
    default: return make_short<128, T>(causal, tiles, qb);
  }
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
           float scale, int causal, int dtype, void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, FA_PATH_AUTO, stream);
}

}  // extern "C"

namespace {

// One tensor's layout as the caller gives it (element strides; d contiguous).
struct Layout {
  int64_t b, h, n;
};

// Bytes from a tensor's first element to one past its last.
int64_t span_bytes(const Layout& s, int64_t B, int64_t H, int64_t N, int64_t d) {
  return ((B - 1) * s.b + (H - 1) * s.h + (N - 1) * s.n + d) * 2;
}

// A layout the kernels can address: 16-byte aligned rows and heads, rows at
// least d apart, per-head spans within 32-bit byte offsets (with room for a
// tile read past the last row).
bool layout_ok(const Layout& s, int64_t N, int64_t d) {
  if (s.b < 0 || s.h < 0 || s.n < d) return false;
  if ((s.b | s.h | s.n) & 7) return false;
  const int64_t lim = (int64_t)1 << 30;
  if (s.n >= lim || (N - 1) * s.n + d >= lim / 2 || (N + 256) * s.n * 2 >= 2 * lim) return false;
  return true;
}

// No two elements of an output share an address: sorted by stride, every
// dimension of extent > 1 must step past everything the inner ones cover.
bool injective(const Layout& s, int64_t B, int64_t H, int64_t N, int64_t d) {
  int64_t dims[3][2] = {{s.b, B}, {s.h, H}, {s.n, N}};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (dims[j][0] < dims[i][0]) {
        for (int c = 0; c < 2; ++c) {
          const int64_t t = dims[i][c];
          dims[i][c] = dims[j][c];
          dims[j][c] = t;
        }
      }
  int64_t extent = d;
  for (int i = 0; i < 3; ++i) {
    if (dims[i][1] <= 1) continue;
    if (dims[i][0] < extent) return false;
    extent = dims[i][0] * (dims[i][1] - 1) + extent;
  }
  return true;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
             float scale, int causal, int dtype, int path, bool strided, const int64_t* strides,
             bool persistent, void* workspace, int64_t workspace_bytes, void* stream) {
  // ---- every check happens before the first HIP call
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FA_ERR_NULLPTR;
  if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (d != 32 && d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  // Per-head tensors are addressed with 32-bit byte offsets (buffer loads):
  // keep them below 2^30 bytes so no offset computed in the kernel can wrap.
  const int64_t lim = (int64_t)1 << 31;
  const int64_t head_lim = (int64_t)1 << 29;
  if (Nq > head_lim || Nk > head_lim || Nq * d >= head_lim || Nk * d >= head_lim) return FA_ERR_SHAPE;
  if (B > lim || H > lim || B * H >= lim) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
  if (((uintptr_t)lse) & 3u) return FA_ERR_ALIGN;

  // Layouts: the given element strides, or contiguous [B, H, N, d].
  Layout sq{H * Nq * d, Nq * d, d}, sk{H * Nk * d, Nk * d, d}, sv = sk, so = sq;
  if (strided) {
    if (strides == nullptr) return FA_ERR_STRIDE;
    sq = {strides[0], strides[1], strides[2]};
    sk = {strides[3], strides[4], strides[5]};
    sv = {strides[6], strides[7], strides[8]};
    so = {strides[9], strides[10], strides[11]};
    if (!layout_ok(sq, Nq, d) || !layout_ok(sk, Nk, d) || !layout_ok(sv, Nk, d) ||
        !layout_ok(so, Nq, d) || !injective(so, B, H, Nq, d))
      return FA_ERR_STRIDE;
  }

  const Variant var = dtype == FA_DTYPE_FP16 ? pick<_Float16>(d, causal != 0)
                                             : pick<__bf16>(d, causal != 0);
  const int64_t num_qb = (Nq + var.bm - 1) / var.bm;
  const int64_t total = B * H * num_qb;
  if (total >= lim) return FA_ERR_SHAPE;

  // o and lse are written: neither may overlap an input or the other (byte
  // spans from first to last element, so interleaved layouts count as
  // overlapping).
  const size_t q_bytes = (size_t)span_bytes(sq, B, H, Nq, d);
  const size_t k_bytes = (size_t)span_bytes(sk, B, H, Nk, d);
  const size_t v_bytes = (size_t)span_bytes(sv, B, H, Nk, d);
  const size_t o_bytes = (size_t)span_bytes(so, B, H, Nq, d);
  const size_t lse_bytes = (size_t)(B * H) * (size_t)Nq * 4;
  if (fa::overlaps(o, o_bytes, q, q_bytes) || fa::overlaps(o, o_bytes, k, k_bytes) ||
      fa::overlaps(o, o_bytes, v, v_bytes))
    return FA_ERR_ALIAS;
  if (lse != nullptr &&
      (fa::overlaps(lse, lse_bytes, q, q_bytes) || fa::overlaps(lse, lse_bytes, k, k_bytes) ||
       fa::overlaps(lse, lse_bytes, v, v_bytes) || fa::overlaps(lse, lse_bytes, o, o_bytes)))
    return FA_ERR_ALIAS;
  if (path != FA_PATH_AUTO && path != FA_PATH_TILED && path != FA_PATH_SHORT) return FA_ERR_PATH;
  if (persistent) {
    // the stream form: full masks only, and a workspace for the pieces
    if (causal) return FA_ERR_PATH;
    if (workspace == nullptr || ((uintptr_t)workspace & 15u)) return FA_ERR_WORKSPACE;
  }
  const int64_t key_tiles = (Nk + 63) / 64;
  const int short_max = d == 128 ? fa::kShortMaxWaves<128> : fa::kShortMaxWaves<64>;
  const bool short_fits = key_tiles <= short_max;
  if (path == FA_PATH_SHORT && !short_fits) return FA_ERR_PATH;
  // Latency-bound sizes take the short path when its workgroups all run at
  // once: one 16-row block per workgroup when those fit one per compute
  // unit, else two blocks per workgroup (one per unit, or as many as their
  // LDS lets a unit hold). An explicit short path takes the same choice and
  // runs in rounds when needed.
  const int64_t short_t1 = B * H * ((Nq + 15) / 16), short_t2 = B * H * ((Nq + 31) / 32);
  if (path == FA_PATH_SHORT && short_t2 >= lim) return FA_ERR_SHAPE;
  int short_qb = 0;  // 0: the tiled path
  if (short_fits && path != FA_PATH_TILED) {
    const int64_t cus = fa::device_cus();
    const int per_cu2 = dtype == FA_DTYPE_FP16 ? pick_short<_Float16>(d, causal != 0, key_tiles, 2).per_cu
                                               : pick_short<__bf16>(d, causal != 0, key_tiles, 2).per_cu;
    if (short_t1 <= cus)
      short_qb = 1;
    else if (path == FA_PATH_SHORT || short_t2 <= (int64_t)per_cu2 * cus)
      short_qb = 2;
  }
  const bool use_short = short_qb != 0;  // its workgroup count is below lim (checked or bounded by the CUs)
  const int64_t short_total = short_qb == 1 ? short_t1 : short_t2;

  fa::Params p;
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
  p.xcd_q = (int)(total / 8);
  p.xcd_r = (int)(total % 8);
  // Heads per scheduling group and the per-XCD numbering (see work_item and
  // fa::causal_order). Without a mask every block has the same work and
  // grouping only widens the set of heads in flight (N = 6400, d = 32 in
  // groups of 2 read 11% more from HBM), so each head is its own group.
  if (causal) {
    const fa::CausalOrder co = fa::causal_order(B * H, 2 * Nk * d * 2);
    p.group = co.group;
    p.launch_order = co.launch_order;
  } else {
    p.group = 1;
    p.launch_order = 0;
  }
  p.nkt = (int)key_tiles;
  p.sq = {sq.b, sq.h, (int)sq.n};
  p.sk = {sk.b, sk.h, (int)sk.n};
  p.sv = {sv.b, sv.h, (int)sv.n};
  p.so = {so.b, so.h, (int)so.n};
  if (scale == 0.0f) {  // every logit is 0: zero Q, any positive factor works
    p.c = 1.0f;
    p.q_and = 0u;
    p.q_xor = 0u;
  } else {  // a negative scale is carried by Q's sign so the factor stays > 0
    p.c = fabsf(scale) * 1.4426950408889634f;
    p.q_and = 0xffffffffu;
    p.q_xor = scale < 0.0f ? 0x80008000u : 0u;
  }

  if (persistent) {
    const StreamVariant sv = pick_stream_dt(dtype, d);
    const int64_t G = stream_grid(sv);
    const int64_t nblocks = B * H * ((Nq + sv.bm - 1) / sv.bm);
    const int64_t need = G * 2 * (int64_t)sv.bm * (d + 3) * 4;
    if (G < 1) return fa::launch_status(hipErrorInvalidDeviceFunction);
    if (workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (fa::overlaps(workspace, (size_t)need, q, q_bytes) || fa::overlaps(workspace, (size_t)need, k, k_bytes) ||
        fa::overlaps(workspace, (size_t)need, v, v_bytes) || fa::overlaps(workspace, (size_t)need, o, o_bytes) ||
        (lse != nullptr && fa::overlaps(workspace, (size_t)need, lse, lse_bytes)))
      return FA_ERR_ALIAS;
    if (nblocks >= lim) return FA_ERR_SHAPE;
    fa::StreamParams sp;
    sp.part = (float*)workspace;
    sp.ntb = (int)((Nk + 63) / 64);
    sp.nblocks = (int)nblocks;
    sp.total = nblocks * sp.ntb;
    sp.G = (int)G;
    sp.gq = (int)(G / 8);
    sp.gr = (int)(G % 8);
    p.num_qb = (int)((Nq + sv.bm - 1) / sv.bm);
    void* sargs[] = {&p, &sp};
    hipError_t e = hipLaunchKernel((const void*)sv.fn, dim3((unsigned)G), dim3((unsigned)sv.threads), sargs,
                                   0, (hipStream_t)stream);
    if (e == hipSuccess && G > 1)  // one workgroup per boundary between ranges
      e = hipLaunchKernel((const void*)sv.combine, dim3((unsigned)(G - 1)), dim3(256), sargs, 0,
                          (hipStream_t)stream);
    return fa::launch_status(e);
  }

  void* args[] = {&p};
  hipError_t e;
  if (use_short) {
    const KernelFn fn = dtype == FA_DTYPE_FP16 ? pick_short<_Float16>(d, causal != 0, key_tiles, short_qb).fn
                                               : pick_short<__bf16>(d, causal != 0, key_tiles, short_qb).fn;
    p.num_qb = (int)((Nq + 16 * short_qb - 1) / (16 * short_qb));
    p.total = (int)short_total;
    p.xcd_q = (int)(short_total / 8);
    p.xcd_r = (int)(short_total % 8);
    e = hipLaunchKernel((const void*)fn, dim3((unsigned)short_total), dim3((unsigned)(64 * key_tiles)),
                        args, 0, (hipStream_t)stream);
  } else {
    e = hipLaunchKernel((const void*)var.fn, dim3((unsigned)total), dim3(var.threads), args, 0,
                        (hipStream_t)stream);
  }
  return fa::launch_status(e);
}

}  // namespace

extern "C" {

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
              float scale, int causal, int dtype, int path, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, path, false, nullptr,
                  false, nullptr, 0, stream);
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                   const int64_t* strides, float scale, int causal, int dtype, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, FA_PATH_AUTO, true,
                  strides, false, nullptr, 0, stream);
}

int64_t fa_fwd_stream_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                      int dtype) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (d != 32 && d != 64 && d != 128) ||
      (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16))
    return -1;
  const StreamVariant sv = pick_stream_dt(dtype, d);
  const int64_t G = stream_grid(sv);
  if (G < 1) return -1;
  return G * 2 * (int64_t)sv.bm * (d + 3) * 4;
}

int fa_fwd_stream_advised(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int dtype,
                          int causal) {
  if (causal != 0 || B < 1 || H < 1 || Nq < 1 || Nk < 1 || (d != 32 && d != 64 && d != 128) ||
      (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16))
    return 0;
  const StreamVariant sv = pick_stream_dt(dtype, d);
  const int64_t G = stream_grid(sv);
  if (G < 1) return 0;
  const int64_t blocks = B * H * ((Nq + sv.bm - 1) / sv.bm);
  // Measured on the MI355X: the stream form wins (8-13%) when the tiled
  // kernel's last round holds at most a quarter of the resident workgroups
  // after one or two full rounds; after three full rounds (1600 blocks on
  // 512) the merge costs more than the short last round saves (a workgroup
  // alone on its compute unit runs close to twice as fast as two sharing it).
  const int64_t full = blocks / G, rest = blocks % G;
  return full >= 1 && full <= 2 && rest > 0 && rest * 4 <= G ? 1 : 0;
}

int fa_fwd_stream(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                  int dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, FA_PATH_AUTO, false,
                  nullptr, true, workspace, workspace_bytes, stream);
}

}  // extern "C"
