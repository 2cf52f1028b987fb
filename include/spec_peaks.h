/*
 * spec_peaks.h - C ABI of the peak probes (libspec_peaks.so), a measurement
 * aid kept apart from the speculation library: the attainable HBM read and
 * copy bandwidth and the attainable dense bf16 MFMA rate of the GPU they run
 * on, the denominators that kernel timings are reported against beside the
 * published peaks.  None of these calls is part of a speculation step.
 *
 * Conventions: pointers are DEVICE memory owned by the caller; `stream` is a
 * hipStream_t (NULL = default stream); every call only enqueues one kernel
 * and returns 0, or -1 for a bad argument (nothing launched), or the HIP
 * error code of the launch.  The caller times the launch (e.g. with events
 * on the same stream).
 */
#ifndef SPEC_PEAKS_H
#define SPEC_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a positive multiple of 16; src 16-byte aligned) once with
 * 16-byte loads, `blocks` workgroups of 512 threads striding over the buffer,
 * four loads in flight per thread.  The XOR of everything read is folded
 * into sink[0] (4 bytes) only in the unlikely case that it equals a fixed
 * constant, so the kernel writes (almost) nothing. */
int32_t spec_peak_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks,
                       void* stream);

/* dst[0:bytes) = src[0:bytes) with 16-byte loads and stores (bytes a positive
 * multiple of 16, both pointers 16-byte aligned, no overlap); traffic is
 * 2 * bytes. */
int32_t spec_peak_copy(void* dst, const void* src, int64_t bytes, int32_t blocks, void* stream);

/* `blocks` workgroups of 256 threads; every wave runs `iters` rounds of 8
 * independent v_mfma_f32_16x16x32_bf16 (16 x 16 x 32 multiply-adds each) on
 * register operands, then writes its accumulators' sum per thread to
 * sink[blocks * 256] (float32).  Work: blocks * 4 * iters * 8 * 16384 flops
 * (spec_peak_mfma_flops). */
int32_t spec_peak_mfma(int32_t iters, float* sink, int32_t blocks, void* stream);
double spec_peak_mfma_flops(int32_t iters, int32_t blocks);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_PEAKS_H */
