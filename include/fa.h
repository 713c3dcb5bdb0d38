/*
 * fa.h - C ABI of the MI355X (gfx950) exact-attention library, libfa.so.
 *
 * Forward operation: for every batch b and head h,
 *
 *     S   = scale * Q K^T                    (Nq x Nk)
 *     S_ij = -inf where causal and j > i     (top-left aligned)
 *     O   = softmax_rows(S) V                (Nq x d)
 *     LSE_i = ln sum_j exp(S_ij)             (natural log)
 *
 * This is the attention formula of "FlashAttention 深度解读" (coreui.cn), section
 * 背景, and the three-step definition in the kwkr.cn YOLO11 FlashAttention-2
 * article, section 1.1. The library computes it the way those articles (section 原理
 * of the former, section 1.2 of the latter) describe: K and V are streamed in
 * tiles through on-chip memory and each tile updates a running row maximum,
 * a running exponential sum and a rescaled output accumulator, so the score
 * matrix S never reaches device memory. Work is spread over (batch, head,
 * query block), as the kwkr.cn article, section 1.2, says FlashAttention-2
 * does. The arguments follow scaled_dot_product_attention(q, k, v,
 * is_causal, scale) as called in that article, section 2.2, with no mask
 * tensor and no dropout; LSE is the softmax statistic it says training keeps
 * (section 2.3).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (HBM of the current HIP device),
 *     owned and allocated by the caller. The library never allocates, frees
 *     or synchronises; it enqueues work on `stream` and returns.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream
 *     of the current device.
 *   - Every argument is checked before any HIP call is made. A failed check
 *     returns a positive status and enqueues nothing. There is no fallback to
 *     another algorithm: an unsupported request is an error.
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by fa_fwd. */
enum fa_status {
  FA_OK = 0,
  FA_ERR_NULLPTR = 1, /* a tensor argument is NULL (lse may be NULL in fa_fwd)   */
  FA_ERR_SHAPE = 2,   /* B, H, Nq or Nk < 1, or an index product too large     */
  FA_ERR_HEADDIM = 3, /* d not in {32, 64, 128}                                 */
  FA_ERR_DTYPE = 4,   /* dtype not FA_DTYPE_FP16 or FA_DTYPE_BF16               */
  FA_ERR_SCALE = 5,   /* scale is NaN or infinite                               */
  FA_ERR_CAUSAL = 6,  /* causal not 0 or 1                                      */
  FA_ERR_ALIGN = 7,   /* a tensor not 16-byte aligned, or lse not 4-byte        */
  FA_ERR_ALIAS = 8,   /* an output overlaps an input, another output or the     */
                      /* workspace                                              */
  FA_ERR_LAUNCH = 9,  /* the kernel launch itself failed (its return value)     */
  FA_ERR_PATH = 10,   /* fa_fwd_ex: unknown path, or FA_PATH_SHORT with Nk too  */
                      /* large for it; fa_bwd_ex: kernel mask not in 1..7       */
  FA_ERR_WORKSPACE = 11, /* fa_bwd: workspace NULL, not 16-byte aligned, or     */
                         /* smaller than fa_bwd_workspace_bytes                 */
  FA_ERR_STRIDE = 12, /* fa_fwd_strided: strides NULL, or a layout the kernels  */
                      /* cannot address (see fa_fwd_strided)                    */
  FA_ERR_SCRATCH = 13 /* fa_bwd_noalloc: the sizes need more than the library's */
                      /* static scratch (FA_BWD_NOALLOC_SCRATCH_BYTES)          */
};

/* Element types of q, k, v and o (all four share one type). Accumulation is
 * always fp32. */
enum fa_dtype { FA_DTYPE_FP16 = 0, FA_DTYPE_BF16 = 1 };

/*
 * fa_fwd - exact attention forward, O and (optionally) LSE.
 *
 *   q      [B, H, Nq, d]  contiguous, row-major, d fastest; dtype elements
 *   k, v   [B, H, Nk, d]  same layout
 *   o      [B, H, Nq, d]  output, same layout and dtype; must not overlap
 *                         q, k, v or lse
 *   lse    [B, H, Nq]     fp32 output, natural-log log-sum-exp of the scaled,
 *                         masked scores of each query row; NULL skips it
 *   B, H   batch and head counts, >= 1
 *   Nq, Nk query and key/value sequence lengths, >= 1, any value (no multiple
 *          of 8 or of a tile size is required; the tail is masked). Nq*d and
 *          Nk*d must stay below 2^29 elements per head (1 GiB of fp16), and
 *          B*H below 2^31.
 *   d      head width: 32, 64 or 128
 *   scale  multiplier of Q K^T; any finite value (0 gives uniform weights).
 *          Callers wanting the usual default pass 1/sqrt(d).
 *   causal 0: every key is visible; 1: key j is visible to query i iff j <= i
 *          (top-left alignment, so no row is ever empty)
 *   dtype  FA_DTYPE_FP16 or FA_DTYPE_BF16
 *   stream hipStream_t (as void*) the kernel is enqueued on
 *
 * Returns FA_OK once the kernel is enqueued, otherwise an fa_status code.
 * Results are deterministic: the same inputs and arguments give bitwise-equal
 * outputs (no atomics, fixed reduction order).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
           float scale, int causal, int dtype, void* stream);

/* Kernel choice for fa_fwd_ex. Both compute the same operation; they differ
 * in how the key range of a head is walked.
 *   FA_PATH_TILED  one workgroup per block of query rows streams the head's
 *                  keys tile after tile through LDS, updating the running
 *                  maximum, sum and output as in the online softmax of the
 *                  kwkr.cn YOLO11 FlashAttention-2 article, section 1.2.
 *   FA_PATH_SHORT  for short key ranges: one workgroup per 16 query rows
 *                  (B*H*ceil(Nq/16) workgroups when those are no more than
 *                  the GPU's compute units, else one per 32 rows) takes every
 *                  64-key tile at once, one wave per tile, and combines the
 *                  per-tile maxima, sums and outputs exactly (the same
 *                  rescaling, applied across tiles in parallel). Requires
 *                  ceil(Nk / 64) <= 16 for d = 32 and 64, <= 9 for d = 128
 *                  (Nk <= 1024 or 576).
 *   FA_PATH_AUTO   FA_PATH_SHORT when it applies and its workgroups all run
 *                  at once (16-row workgroups at most one per compute unit,
 *                  or 32-row ones as many as the units' LDS holds:
 *                  latency-bound sizes); FA_PATH_TILED otherwise. */
enum fa_path { FA_PATH_AUTO = 0, FA_PATH_TILED = 1, FA_PATH_SHORT = 2 };

/*
 * fa_fwd_ex - fa_fwd with an explicit kernel choice (fa_path). All other
 * arguments, the results and the error behaviour are those of fa_fwd; an
 * unknown path, or FA_PATH_SHORT beyond its key-range limit, returns
 * FA_ERR_PATH after the other checks and before any HIP call.
 * fa_fwd(...) is fa_fwd_ex(..., FA_PATH_AUTO, stream).
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
              float scale, int causal, int dtype, int path, void* stream);

/*
 * fa_fwd_strided - fa_fwd on tensors in any [B, H, N, d] layout whose d
 * elements are contiguous: for example [B, N, H, d] (sequence-major, the
 * layout of a projection's output reshaped into heads) or q, k, v as views
 * of one fused [B, N, 3, H, d] projection output. The layout and fusion
 * variants of the kwkr.cn YOLO11 FlashAttention-2 article, section 2.2 (the
 * transposes around the attention call) and of "FlashAttention 深度解读",
 * section 实现 2 (fused operator), are then read in place, with no copies.
 *
 *   strides  host array of 12 int64 element strides, in the order
 *            q: batch, head, row;  k: batch, head, row;
 *            v: batch, head, row;  o: batch, head, row.
 *            Element (b, h, n, c) of q is at q + b*s0 + h*s1 + n*s2 + c.
 *            Every stride is a multiple of 8 elements (16 bytes) and >= 0;
 *            row strides are >= d; one head's rows span fewer than 2^29
 *            elements. o's layout must map distinct elements to distinct
 *            addresses. Violations return FA_ERR_STRIDE.
 *   lse      stays contiguous [B, H, Nq] fp32 (or NULL).
 * Everything else (arguments, results, error behaviour) is as in fa_fwd; the
 * kernel choice is FA_PATH_AUTO. Overlap checks use each tensor's byte span
 * from its first to its last element, so o interleaved with an input counts
 * as overlapping (FA_ERR_ALIAS).
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                   const int64_t* strides, float scale, int causal, int dtype, void* stream);

/*
 * Persistent ("stream") form of the forward, for full masks. fa_fwd gives
 * every workgroup one block of query rows; when the blocks outnumber the
 * workgroups the GPU holds at once by a non-integer factor, the last round
 * runs partly empty. fa_fwd_stream launches exactly the resident workgroups
 * and gives each an equal share of the (query block, key tile) work; a query
 * block whose key range is cut between two workgroups is computed in pieces
 * (each with its own running maximum, sum and output, as in the online
 * softmax of the kwkr.cn YOLO11 FlashAttention-2 article, section 1.2) and a
 * second kernel merges the pieces exactly.
 *
 * fa_fwd_stream_workspace_bytes - workspace bytes fa_fwd_stream needs on the
 * current device for these sizes (it depends on how many workgroups the
 * device holds at once); -1 for invalid arguments or a failed device query.
 *
 * fa_fwd_stream_advised - 1 when the stream form is expected to beat fa_fwd
 * for these arguments on the current device: full mask, and query blocks
 * filling one or two rounds of the resident workgroups plus at most a
 * quarter of another (fa_fwd then runs a mostly empty last round); else 0.
 * Never fails.
 *
 * fa_fwd_stream - fa_fwd (contiguous tensors, same arguments, results and
 * checks) on the stream form. causal = 1 returns FA_ERR_PATH. workspace:
 * device memory of at least fa_fwd_stream_workspace_bytes bytes, 16-byte
 * aligned, caller-owned, not overlapping any tensor (FA_ERR_WORKSPACE,
 * FA_ERR_ALIAS); its contents on entry do not matter. Two kernels are
 * enqueued on `stream`. Deterministic (fixed split and merge order).
 * The one exception to "every check before any HIP call": the workspace
 * size and overlap checks need the number of resident workgroups, which
 * comes from an occupancy query of the current device (a HIP call that
 * enqueues nothing); every other check runs before it.
 */
int64_t fa_fwd_stream_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                      int dtype);
int fa_fwd_stream_advised(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int dtype,
                          int causal);
int fa_fwd_stream(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                  int dtype, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * fa_fwd_fp8 - exact attention forward on FP8 inputs (FlashAttention-3's FP8
 * variant, ai2ai.xin flash-attention-principle page, FA-3 section).
 *
 *   q, k, v    [B, H, N, d] contiguous, one byte per element: OCP e4m3 ("fn":
 *              no infinities; bytes 0x7f and 0xff are NaN and must not occur)
 *   q_descale, k_descale, v_descale
 *              per-tensor dequantisation factors (> 0, finite): element x of q
 *              stands for q_descale * e4m3(x), and likewise for k and v
 *   o          [B, H, Nq, d] contiguous output in out_dtype (FA_DTYPE_FP16 or
 *              FA_DTYPE_BF16)
 *   lse, B, H, Nq, Nk, scale, causal, stream: as in fa_fwd
 *   d          32, 64 or 128 (d = 32 fills half of each 64-deep Q K^T step)
 * Computes the forward of the dequantised tensors: S = scale * q_descale *
 * k_descale * (Q K^T on the e4m3 values, fp32 accumulation), O = softmax(S) V.
 * The attention weights are rounded to e4m3 (after scaling so that the
 * largest weight of a row is 2^8) for the P V product on the FP8 matrix cores;
 * the row sum and the LSE use the unrounded fp32 weights. Errors: FA_ERR_DTYPE
 * for out_dtype, FA_ERR_HEADDIM for d = 32, FA_ERR_SCALE for a descale factor
 * that is not finite and positive or a product with scale that overflows;
 * otherwise as fa_fwd. Deterministic (no atomics).
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
               float q_descale, float k_descale, float v_descale, int causal, int out_dtype,
               void* stream);

/*
 * Backward pass. For an upstream gradient dO of the forward's output O, the
 * gradients of the scalar sum(O * dO) with respect to Q, K and V, per (b, h):
 *
 *     P   = softmax_rows(scale * Q K^T [causal mask])   recomputed from LSE
 *     dV  = P^T dO
 *     dP  = dO V^T
 *     D_i = sum_c dO_ic O_ic         (= sum_j P_ij dP_ij)
 *     dS  = P * (dP - D)             (elementwise, D broadcast along rows)
 *     dQ  = scale * dS K
 *     dK  = scale * dS^T Q
 *
 * The cited articles state that training keeps the forward's softmax statistics for
 * the backward pass (kwkr.cn YOLO11 FlashAttention-2 article, section 2.3) and
 * that the backward recomputes the attention weights rather than storing them
 * ("YOLOv12推理速度翻倍秘诀：Flash Attention加持", section 1); the formulas are the
 * chain rule of the forward definition above. P is rebuilt tile by tile from
 * Q, K and the forward's LSE as P = exp(scale * q.k - LSE), so no Nq x Nk
 * matrix reaches device memory here either.
 */

/*
 * fa_bwd_workspace_bytes - bytes of device workspace fa_bwd needs for B*H
 * heads of Nq query rows: 256 * B * H * ceil(Nq / 32) (two fp32 values per
 * query row, rows padded to a multiple of 32). Returns -1 when B, H or Nq is
 * below 1 or the size does not fit in int64_t.
 */
int64_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Nq);

/*
 * fa_bwd - gradients dQ, dK, dV of exact attention.
 *
 *   q, k, v    the forward's inputs, layouts and dtype as in fa_fwd
 *   o          [B, H, Nq, d] the forward's output O for these inputs
 *   dout       [B, H, Nq, d] upstream gradient dO, same dtype
 *   lse        [B, H, Nq] fp32, the forward's LSE (natural log) for the same
 *              q, k, scale and causal; the weights are rebuilt from it, so an
 *              LSE from other inputs gives meaningless gradients
 *   dq         [B, H, Nq, d] output, dtype of q
 *   dk, dv     [B, H, Nk, d] outputs, dtype of q
 *   workspace  device memory of at least fa_bwd_workspace_bytes(B, H, Nq)
 *              bytes, 16-byte aligned, owned by the caller; its contents on
 *              entry do not matter and are overwritten. It must not overlap
 *              any tensor argument.
 *   workspace_bytes  its size in bytes
 *   B, H, Nq, Nk, d, scale, causal, dtype, stream: as in fa_fwd
 *
 * dq, dk and dv must not overlap each other, any input or the workspace.
 * Work is enqueued on `stream` as three kernels (per-row -D and the scaled
 * LSE into the workspace; dK and dV per block of keys; dQ per block of
 * query rows), so the workspace must stay allocated until they have run.
 * Returns FA_OK once enqueued, otherwise an fa_status code (all checks are
 * made before any HIP call). Accumulation is fp32; every output element is
 * summed in a fixed order, so results are deterministic (no atomics).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace,
           int64_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
           float scale, int causal, int dtype, void* stream);

/* Kernel selection for fa_bwd_ex, a bit mask. fa_bwd runs all three in this
 * order on one stream. FA_BWD_PRE fills the workspace (per-row -D and the
 * scaled LSE); FA_BWD_DKDV and FA_BWD_DQ read it and are independent of each
 * other, so a caller may enqueue PRE, then DKDV and DQ on two streams that
 * both wait for PRE. */
enum fa_bwd_kernels { FA_BWD_PRE = 1, FA_BWD_DKDV = 2, FA_BWD_DQ = 4, FA_BWD_ALL = 7 };

/*
 * fa_bwd_ex - fa_bwd enqueuing only the kernels selected in `kernels`
 * (fa_bwd_kernels bits). Arguments, checks and results are those of fa_bwd;
 * a mask outside 1..FA_BWD_ALL returns FA_ERR_PATH after the other checks.
 * DKDV and DQ read the workspace as the last PRE with the same o, dout, lse
 * and sizes left it: the caller orders them after that PRE.
 * fa_bwd(...) is fa_bwd_ex(..., FA_BWD_ALL, stream).
 */
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, void* dq, void* dk, void* dv, void* workspace,
              int64_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
              float scale, int causal, int dtype, int kernels, void* stream);

/*
 * fa_bwd_noalloc - fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same gradients from the same kernels, with the D/LSE
 * records kept in a scratch array inside the library instead of a
 * caller-provided workspace. Arguments, results and checks are fa_bwd's
 * without workspace and workspace_bytes. The caller still provides every
 * tensor; the library allocates and frees nothing (no hipMalloc, no
 * allocating library routine).
 *
 * The scratch is a static device array of FA_BWD_NOALLOC_SCRATCH_BYTES
 * (16 MiB), one copy on each GPU the library runs on, held until the process
 * ends; its address on a device is looked up on the first call on that
 * device. Sizes with fa_bwd_workspace_bytes(B, H, Nq) above it return
 * FA_ERR_SCRATCH (e.g. B*H*ceil(Nq/32) > 65536), before any HIP call.
 * Every call on one GPU shares that GPU's copy: calls that overlap in time
 * on one GPU (on different streams, or from different threads without
 * ordering) race and give wrong gradients; calls ordered on one stream are
 * safe. Nothing in the scratch needs clearing between calls (each call
 * rewrites every record it reads).
 */
#define FA_BWD_NOALLOC_SCRATCH_BYTES (16LL << 20)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Nq,
                   int64_t Nk, int64_t d, float scale, int causal, int dtype, void* stream);

/*
 * Standard (unfused) attention: the baseline the fused forward is measured
 * against. The cited articles contrast FlashAttention with attention computed
 * the standard way ("FlashAttention 深度解读", section 背景: the score matrix
 * is written to device memory, read back for the softmax, the probabilities
 * are written and read back again for the product with V; ai2ai.xin
 * flash-attention-principle page, the five-step list of the self-attention
 * bottleneck; kwkr.cn YOLO11 FlashAttention-2 article, section 1.1). This
 * computes the same O and LSE as fa_fwd that way, in three kernels, each a
 * full pass over an Nq x Nk matrix in HBM:
 *   1. S = scale * Q K^T      written to s (fp32)
 *   2. P = softmax_rows(S)    s read, causal mask applied (top-left, as in
 *                             fa_fwd), p written in dtype, lse written
 *   3. O = P V                p read
 * Both products run over the whole Nq x Nk square (causal too), as a
 * standard implementation does.
 *
 * fa_std_row_stride - NkP, the row stride (in elements) of s and p: Nk
 * rounded up to a multiple of 64; -1 for Nk < 1 or Nk > 2^29.
 *
 * fa_std_fwd - arguments as fa_fwd, plus
 *   s   [B, H, Nq, NkP] fp32, caller-owned device memory, 16-byte aligned:
 *       s[b,h,i,j] = scale * q_i . k_j for j < Nk (masked entries included);
 *       columns j >= Nk are not written
 *   p   [B, H, Nq, NkP] in dtype, caller-owned, 16-byte aligned: the
 *       normalised attention weights softmax(S) (0 where masked and for
 *       columns j >= Nk), rounded to dtype; the product with V uses them
 *       as stored
 * o, s, p and lse must not overlap an input or each other (FA_ERR_ALIAS).
 * Additional size limit: Nq * NkP < 2^29 per head (FA_ERR_SHAPE). Three
 * kernels are enqueued on `stream`. Every check runs before any HIP call.
 */
int64_t fa_std_row_stride(int64_t Nk);
int fa_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse, float* s, void* p,
               int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
               int dtype, void* stream);

/* A static, human-readable description of a status code (never NULL). */
const char* fa_status_str(int status);

/* HIP's description of the error behind the calling thread's last
 * FA_ERR_LAUNCH (static string, "" if none). */
const char* fa_last_launch_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
