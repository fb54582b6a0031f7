/*
 * uno_probe.h -- measurement probes of the gfx950 GPU (not part of the decode
 * step): the ceilings that the decode kernels' rates are compared with besides
 * the vendor peaks.  Built into libuno_probe.so, beside libuno.so.
 *
 * Every probe enqueues on `stream` (a hipStream_t; NULL = the default stream)
 * and returns 0, or -1 for a bad argument (nothing enqueued) and -2 for a
 * launch failure.  Buffers are device pointers owned by the caller.
 */
#ifndef UNO_PROBE_H
#define UNO_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` (a multiple of 16 * 256) from `src`, 16-byte
 * loads, `n_wg` workgroups of 256 threads striding over the buffer.  mode:
 * bit 0 marks the loads non-temporal; bit 1 keeps eight loads in flight per
 * lane instead of four.  Each workgroup writes one float (a reduction of what
 * it read) to sink[wg]. */
int uno_probe_read(const void *src, size_t bytes, int mode, int n_wg, float *sink,
                   void *stream);

/* Copy of `bytes` (a multiple of 16 * 256) from src to dst with 16-byte loads
 * and stores, `n_wg` workgroups of 256 threads striding over the buffer. */
int uno_probe_copy(const void *src, void *dst, size_t bytes, int n_wg, void *stream);

/* Register-only bf16 matrix-core loop: `n_wg` workgroups of 256 threads, each
 * wave issuing `iters` rounds of four independent v_mfma_f32_32x32x16_bf16
 * (2 * 32 * 32 * 16 flops each); sink[wg] receives one accumulator value.
 * Flops = n_wg * 4 waves * iters * 4 * 32768. */
int uno_probe_mfma(int iters, int n_wg, float *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* UNO_PROBE_H */
