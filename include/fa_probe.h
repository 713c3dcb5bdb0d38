/*
 * fa_probe.h - C ABI of libfa_probe.so, a measurement aid that is not part of
 * the attention library: the vector-unit throughput of the instructions the
 * forward's softmax step spends its time on (exp2 and fused multiply-add, the
 * per-score work of the online softmax in "FlashAttention 深度解读", section
 * 原理 2, and the kwkr.cn YOLO11 FlashAttention-2 article, section 1.2), the
 * rate of its matrix instruction, and how far the two kinds of work overlap
 * when different waves of one SIMD, or one wave, issue them. The benchmark turns the
 * measured rates into a vector-unit bound for the forward next to its
 * matrix-core bound.
 *
 * fa_probe_vector_rate - enqueue one kernel on `stream` that runs `iters`
 * iterations of `chains` independent dependency chains per thread, each
 * iteration one instruction per chain of the kind `op` selects:
 *   FA_PROBE_EXP2 (0)  v_exp_f32 (2^x)
 *   FA_PROBE_FMA  (1)  v_fma_f32
 *   FA_PROBE_MIX  (2)  one v_fma_f32 feeding one v_exp_f32 (the softmax's
 *                      pair per score; counted as one pair)
 * over `blocks` workgroups of 256 threads. Each thread writes one float of
 * its final values to out[blocks * 256] (device memory, caller-owned), so
 * nothing is optimised away. The instruction count is blocks * 256 * iters *
 * chains. Returns 0, or 1 for invalid arguments (op outside 0..2, blocks or
 * iters < 1, chains not 8, out NULL), or 2 when the launch fails. Time it
 * with events on `stream`.
 *
 * fa_probe_matrix_rate - enqueue one kernel of `blocks` workgroups of 256
 * threads (4 waves); each wave runs `iters` steps of independent matrix
 * instruction chains with accumulators in vector registers: shape 0, 4 chains
 * of v_mfma_f32_32x32x16_f16 (32768 FLOP each); shape 1, 8 chains of
 * v_mfma_f32_16x16x32_f16 (16384 FLOP each, the tiled forward's
 * instruction). Either way a step is 131072 FLOP per wave, blocks * 4 * iters
 * steps in all. Each thread writes one float to out[blocks * 256]
 * (caller-owned device memory). Returns 0, 1 for invalid arguments (shape
 * not 0 or 1, blocks or iters < 1, out NULL), or 2 when the launch fails.
 *
 * fa_probe_coexec - enqueue one kernel of `blocks` workgroups of 512 threads
 * (8 waves, two per SIMD). With bit 0 of `roles` set, waves 0-3 (one per
 * SIMD) run `matrix_iters` steps of the matrix chains above; with bit 1 set,
 * waves 4-7 run `vector_iters` steps of softmax-shaped vector work (32 values
 * per lane, each step one v_fma_f32 and one v_exp_f32 per value and one
 * v_cvt_pk_f16_f32 per pair). Timing roles 1, 2 and 3 shows whether the
 * SIMDs overlap the two kinds of work (time of 3 near the larger of 1 and 2)
 * or take them in turn (near their sum). Each thread writes one float to
 * out[blocks * 512]. Returns 0, 1 for invalid arguments (roles outside 1..3,
 * blocks or either count < 1, out NULL), or 2 when the launch fails.
 *
 * fa_probe_coissue - enqueue one kernel of `blocks` workgroups of 256
 * threads (4 waves, one per SIMD when blocks does not exceed the CUs; with
 * 2x or 4x as many blocks, two or four waves share each SIMD). Each wave
 * runs `iters` steps; a step holds, by `mode`: 1, 16 v_mfma_f32_16x16x32_f16
 * (8 independent chains); 2, the vector work of one fa_probe_coexec vector
 * step; 3, both in one wave, in the compiler's order; 4, both in one wave,
 * the instruction stream interleaved one matrix instruction to five vector
 * instructions. Timing modes 1-4 shows how far one wave's own matrix and
 * vector instructions overlap, and how that compares with several waves
 * sharing a SIMD. Each thread writes one float to out[blocks * 256]
 * (caller-owned device memory). Returns 0, 1 for invalid arguments (mode
 * outside 1..4, blocks or iters < 1, out NULL), or 2 when the launch fails.
 */
#ifndef FA_PROBE_H_
#define FA_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_probe_op { FA_PROBE_EXP2 = 0, FA_PROBE_FMA = 1, FA_PROBE_MIX = 2 };

int fa_probe_vector_rate(int op, int blocks, int iters, int chains, float* out, void* stream);
int fa_probe_matrix_rate(int shape, int blocks, int iters, float* out, void* stream);
int fa_probe_coexec(int roles, int blocks, int matrix_iters, int vector_iters, float* out, void* stream);
int fa_probe_coissue(int mode, int blocks, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H_ */
