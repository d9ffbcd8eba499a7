/* tlsl_measure.h -- measurement aids of libtlsl.so (gfx950).
 *
 * None of these compute any part of the token-selection method.  They exist
 * so that a benchmark can time one kernel of a multi-kernel entry point with
 * HIP events on the stream that kernel is launched on, and can calibrate the
 * roofline it reports against: a streaming copy (achievable HBM bandwidth,
 * and the scale of the HBM byte counters for a transfer of known size) and a
 * matrix-core loop (achievable dense MFMA rate).
 *
 * Same error codes and thread-local message as tlsl.h.
 */
#ifndef TLSL_MEASURE_H
#define TLSL_MEASURE_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Arms the kernel timer for the kernel named `kernel` (its function name
 * without namespace or template arguments, e.g. "prefill_score_kernel",
 * "decode_scan_kernel", "sparse_attn_kernel", "topk_filter_kernel").  From
 * then on, each launch of that kernel by any entry point is bracketed by a
 * pair of HIP events recorded on the launch stream, for at most
 * `max_launches` (1..65536) launches; later launches are not timed.  Events
 * are created here (not in the entry points).  Arming again discards what
 * the previous arming recorded.  Process-wide state: arm and collect from
 * one host thread while no other thread launches through the library.
 * Errors: TLSL_ERR_NULL (kernel NULL), TLSL_ERR_SHAPE (max_launches out of
 * range), TLSL_ERR_HIP (event creation failed). */
int tlsl_timer_arm(const char* kernel, int max_launches);

/* Waits for the last recorded event, writes the number of timed launches and
 * the total, minimum and maximum event time per launch in milliseconds (any
 * output pointer may be NULL; times are 0 when nothing was timed) and
 * disarms the timer.  Errors: TLSL_ERR_SHAPE (not armed), TLSL_ERR_HIP. */
int tlsl_timer_collect(int* launches, double* total_ms, double* min_ms, double* max_ms);

/* Streaming copy of `bytes` bytes (a multiple of 16) from src to dst
 * (device pointers, 16-byte aligned, not overlapping) with 16-byte vector
 * loads and stores: reads `bytes` and writes `bytes` of HBM once each.
 * Asynchronous on `stream`.  Errors: TLSL_ERR_NULL, TLSL_ERR_SHAPE
 * (bytes == 0 or not a multiple of 16), TLSL_ERR_ALIGN, TLSL_ERR_HIP. */
int tlsl_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Dense matrix-core loop: `blocks` workgroups of 256 threads, each wave
 * issuing `iters` rounds of 8 independent 16x16 MFMAs of type `dt`
 * (TLSL_BF16: 16x16x32 bf16; TLSL_FP8_E4M3: 16x16x128 fp8) on register
 * operands, then storing one float per thread to `sink` (device, blocks*256
 * floats) so the work is live.  *flops receives the algorithmic flop count of
 * the launch (2*16*16*K per MFMA).  Asynchronous on `stream`.
 * Errors: TLSL_ERR_NULL, TLSL_ERR_SHAPE (blocks <= 0, iters <= 0 or odd),
 * TLSL_ERR_UNSUPPORTED (other dtypes), TLSL_ERR_HIP. */
int tlsl_calib_mfma(int dt, int blocks, int iters, float* sink, double* flops, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TLSL_MEASURE_H */
