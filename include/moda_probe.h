/*
 * moda_probe.h -- C ABI of libmoda_probe.so: measurement kernels that give the
 * attainable peaks the MoDA kernels are compared with (bf16 matrix-core rate,
 * HBM copy and read bandwidth) on the GPU the benchmark runs on.  They are not
 * part of the MoDA computation; the benchmark prints their rates beside the
 * published peaks it prices against (the roofline's denominators).
 *
 * Conventions: device pointers owned by the caller, 16-byte aligned; work is
 * enqueued on `stream` (a hipStream_t) and the call returns at once; nothing
 * is allocated or synchronised.  Return codes are those of moda.h
 * (MODA_OK, MODA_ERR_NULL, MODA_ERR_SHAPE, MODA_ERR_ALIGN, MODA_ERR_HIP).
 */
#ifndef MODA_PROBE_H
#define MODA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moda_probe_stream_t; /* hipStream_t */

/*
 * bf16 matrix-core rate: `blocks` workgroups of 4 waves; each wave issues
 * 4 * iters v_mfma_f32_32x32x16_bf16 on four independent register
 * accumulators (no memory traffic in the loop), then writes one fp32 per
 * lane to sink[blocks * 256].  random = 1: each chain has its own
 * pseudo-random bf16 operands in [-1, 1), different per lane (switching data,
 * as in real tiles); random = 0: every operand is the constant 1/64.  Where
 * the clock is power limited the two rates differ.
 * Work: blocks * 4 * 4 * iters * 32768 flop.
 * Errors: MODA_ERR_NULL (sink); MODA_ERR_SHAPE (blocks or iters <= 0,
 * random not 0 or 1); MODA_ERR_ALIGN; MODA_ERR_HIP.
 */
int moda_probe_mfma_bf16(float* sink, int blocks, int iters, int random, moda_probe_stream_t stream);

/*
 * HBM copy: dst[0 .. bytes) = src[0 .. bytes) in 16-byte units by `blocks`
 * workgroups of 256 threads, each moving one contiguous span with
 * non-temporal loads and stores.  bytes must be a
 * multiple of 16; src and dst must not overlap.  Traffic: 2 * bytes.
 * Errors: MODA_ERR_NULL; MODA_ERR_SHAPE (bytes not a positive multiple of
 * 16, blocks <= 0); MODA_ERR_ALIGN; MODA_ERR_HIP.
 */
int moda_probe_copy(const void* src, void* dst, size_t bytes, int blocks, moda_probe_stream_t stream);

/*
 * HBM read: every 16-byte unit of src[0 .. bytes) is read once and folded
 * (xor) into one 32-bit value per thread, written to sink[blocks * 256].
 * Traffic: bytes.  Errors as moda_probe_copy.
 */
int moda_probe_read(const void* src, size_t bytes, int blocks, unsigned int* sink, moda_probe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MODA_PROBE_H */
