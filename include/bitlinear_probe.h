/*
 * bitlinear_probe.h -- calibration kernels for the roofline denominators.
 *
 * The contraction kernels are reported against the part's published peaks
 * (8 TB/s HBM, 5.0 POP/s dense int8) and also against what this part
 * sustains on the same two resources, measured by these two probes.  They
 * compute nothing of the BitLinear layer; each leaves a checksum so that its
 * work cannot be elided and its result can be checked on the host.
 *
 * Conventions are those of bitlinear.h: device pointers owned by the
 * caller, 16-byte aligned; calls only enqueue work on `stream` (a
 * hipStream_t, NULL = default stream); 0 = BITLINEAR_OK, negative = error
 * with a message from bitlinear_last_error(); a rejected call enqueues
 * nothing.
 */
#ifndef BITLINEAR_PROBE_H
#define BITLINEAR_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Words of the read probe's sink: 256 per chunk of chunk_bytes (0 on
 * invalid sizes). */
int64_t bitlinear_probe_read_sink_words(int64_t bytes, int64_t chunk_bytes);

/*
 * Streaming read of `bytes` bytes of device memory at `buf` with 16-byte
 * non-temporal loads.  One workgroup of 256 threads per chunk of
 * chunk_bytes (the last chunk may be short); consecutive lanes read
 * consecutive 16-byte words, eight loads in flight per thread.
 *   bytes        > 0 and a multiple of 16        (BITLINEAR_ERR_SHAPE)
 *   chunk_bytes  a multiple of 4096, and at most 2^31 chunks
 *                                                (BITLINEAR_ERR_SHAPE)
 *   sink         uint32[bitlinear_probe_read_sink_words(bytes, chunk_bytes)];
 *                thread t of chunk c writes sink[256 c + t], the XOR of the
 *                32-bit words it read.  The XOR of all sink words is the XOR
 *                of all 32-bit words of the buffer.
 */
int bitlinear_probe_read(const void *buf, int64_t bytes, int64_t chunk_bytes, uint32_t *sink, void *stream);

/*
 * A chain of v_mfma_i32_32x32x32_i8 with no memory traffic: each 256-thread
 * workgroup runs four independent accumulator chains per wave for `iters`
 * rounds, with every A operand byte equal to a and every B byte equal to b.
 * It performs blocks * 4 * iters * 4 * 65536 int8 operations.
 *   iters        >= 1, and 2048 |a b| iters < 2^31 (BITLINEAR_ERR_SHAPE)
 *   a, b         in [-128, 127]                   (BITLINEAR_ERR_ARG)
 *   blocks       >= 1                             (BITLINEAR_ERR_SHAPE)
 *   sink         int32[256 * blocks]; every thread writes 2048 a b iters,
 *                the sum of its 64 accumulator elements.
 */
int bitlinear_probe_mfma(int64_t iters, int32_t a, int32_t b, int32_t blocks, int32_t *sink, void *stream);

/* Workgroups of bitlinear_probe_mfma that are resident on the current
 * device at once (compute units times workgroups per unit), into *blocks.
 * Queries the HIP runtime: BITLINEAR_ERR_HIP if it fails. */
int bitlinear_probe_mfma_blocks(int32_t *blocks);

#ifdef __cplusplus
}
#endif
#endif /* BITLINEAR_PROBE_H */
