/* Measurement probes for MI355X (gfx950): a plain streaming read,
 * matrix-instruction throughput loops and vector-ALU throughput loops. They set the practical ceilings that
 * the attention kernels' throughputs are compared against (HBM bandwidth
 * for decode, matrix rates for prefill and dense attention); they are not
 * part of the attention computation.
 *
 * Conventions: device pointers owned by the caller; every call is
 * asynchronous on `stream` (NULL: the default stream); the return value is
 * 0 on success, 1 for an invalid argument (checked on the host before any
 * HIP call), 4 for a launch error. */
#ifndef QA_PROBE_H
#define QA_PROBE_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16) at `src` with 16-byte loads, grid-stride,
 * in `wgs` workgroups of 256 threads (1 <= wgs <= 65535), and writes one int
 * per workgroup to `sink[wgs]` so that the reads are not elided. */
int qa_probe_stream_read(const void* src, size_t bytes, int wgs, int* sink, hipStream_t stream);

/* Matrix-instruction throughput: every wave of `wgs` workgroups (4 waves
 * each, one per SIMD; 1 <= wgs <= 65535) issues `iters` (>= 1) rounds of
 * independent accumulations with operands held in registers:
 *   kind 0: 4 x v_mfma_i32_32x32x32_i8          (4 x 65536 ops per round)
 *   kind 1: 4 x v_mfma_f32_32x32x16_f16         (4 x 32768 flops per round)
 *   kind 2: 8 x v_mfma_i32_16x16x64_i8          (8 x 32768 ops per round)
 *   kind 3: 8 x v_mfma_f32_16x16x32_f16         (8 x 16384 flops per round)
 *   kind 4: 16 x v_mfma_i32_16x16x64_i8         (16 x 32768)
 *   kind 5: 16 x v_mfma_f32_16x16x32_f16        (16 x 16384)
 *   kind 6: 4 x v_mfma_i32_16x16x64_i8          (4 x 32768)
 *   kind 7: 4 x v_mfma_f32_16x16x32_f16         (4 x 16384)
 *   kind 8: 4 x v_mfma_f32_32x32x64_f8f6f4, E4M3 (4 x 131072)
 * Total work = per-round ops x iters x 4 x wgs; wgs = 256 k puts k waves on
 * every SIMD of the 256 compute units. One float per thread (the sum of all
 * accumulator elements) goes to `sink[wgs * 256]`. */
int qa_probe_mfma(int kind, int iters, int wgs, float* sink, hipStream_t stream);

/* Vector-ALU throughput: every lane of `wgs` workgroups of 256 threads
 * (1 <= wgs <= 65535) runs `iters` (>= 1) rounds of 8 independent
 * single-operation chains:
 *   kind 0: v_exp_f32 (the base-2 exponential of the softmax)
 *   kind 1: v_fma_f32
 * Total lane operations = 8 x iters x 256 x wgs. One float per thread goes
 * to `sink[wgs * 256]`. */
int qa_probe_valu(int kind, int iters, int wgs, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QA_PROBE_H */
