/*
 * sa_peaks.h — achievable-peak probes shipped with libsa (measurement only).
 *
 * The hot path is bound either by the bf16 matrix cores (the block-sparse and
 * vertical-slash forward, the indexer) or by HBM (the gathered decode).  These
 * two calls enqueue a kernel that does nothing but that unit's work, so a
 * benchmark can time them beside the real kernels and report each kernel's
 * rate against the spec peak and against the rate this chip sustains at the
 * clock it runs during the measurement.  Neither is part of the method.
 *
 * Conventions as in sa.h: device pointers owned by the caller, asynchronous on
 * `stream` (a hipStream_t), return 0 on success, 1 for a bad argument, 7 when
 * HIP reports a launch error.  The caller times the launch (HIP events).
 */
#ifndef SA_PEAKS_H_
#define SA_PEAKS_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core loop: waves_per_cu (a multiple of 4) waves on every CU each run
 * 4 independent chains of `iters` v_mfma_f32_32x32x16_bf16.  *flop receives
 * the floating-point operations the launch performs (2 per multiply-add).
 * sink: any device buffer of >= 1 KB (written only under a condition the data
 * never meets). */
int sa_peak_mfma_bf16(float* sink, int iters, int waves_per_cu, double* flop, void* stream);

/* Streaming read of `bytes` (16-byte aligned, read in 16-byte elements) `reps`
 * times by 8 workgroups of 256 threads per CU.  *bytes_read receives the
 * bytes the launch reads.  sink: any device buffer of >= 4 KB. */
int sa_peak_read(const void* buf, size_t bytes, int reps, void* sink, double* bytes_read, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SA_PEAKS_H_ */
