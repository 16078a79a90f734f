/*
 * bitlinear_probe.h -- calibration kernels for the roofline denominators.
 *
 * The contraction kernels are reported against the part's published peaks
 * (8 TB/s HBM, 5.0 POP/s dense int8) and also against what this part
 * sustains on the same two resources, measured by the first two probes; the
 * third measures a grid-wide barrier, the cost per dependent stage of a
 * persistent kernel.  They compute nothing of the BitLinear layer; each
 * leaves a checksum so that its work cannot be elided and its result can be
 * checked on the host.
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

/*
 * The chains of bitlinear_probe_mfma with operands from memory, so that the
 * matrix instructions toggle as many bits as a contraction over real data
 * does: `operands` holds four sets of an A and a B fragment, int8
 * [4][2][64 lanes][16 bytes] (set j's A at [j][0], its B at [j][1]); every
 * wave loads them once and chain j multiplies set j for `iters` rounds.
 * It performs blocks * 4 * iters * 4 * 65536 int8 operations.
 *   iters     >= 1, blocks >= 1                     (BITLINEAR_ERR_SHAPE)
 *   sink      int32[256 * blocks]; thread t of workgroup b writes the sum,
 *             wrapped to 32 bits, of its 64 accumulator elements.  Byte i
 *             of lane l of an A fragment and byte i of lane l' of a B
 *             fragment meet in a product exactly when l / 32 = l' / 32, so
 *             the 256 words of a workgroup add up (mod 2^32) to
 *             4 iters sum_j sum_{h<2, i<16} (sum_{r<32} A_j[32h+r][i])
 *             (sum_{r<32} B_j[32h+r][i]).
 *   clocks    uint64[3 * blocks]: per workgroup, read by thread 0, the
 *             shader-clock count (s_memtime) elapsed over its loop, then the
 *             constant-rate reference counter (s_memrealtime) at the loop's
 *             start and at its end.
 */
int bitlinear_probe_mfma_data(int64_t iters, const void *operands, int32_t blocks, int32_t *sink, uint64_t *clocks,
                              void *stream);

/* Workgroups of bitlinear_probe_mfma that are resident on the current
 * device at once (compute units times workgroups per unit), into *blocks.
 * Queries the HIP runtime: BITLINEAR_ERR_HIP if it fails. */
int bitlinear_probe_mfma_blocks(int32_t *blocks);

/*
 * `rounds` grid-wide barriers among `blocks` workgroups of 256 threads: at
 * each, every workgroup publishes one word (round * blocks + its index) with
 * a device-scope store, waits for it to complete, increments a device-scope
 * counter and polls it until every workgroup has arrived, then reads all
 * words of that round with device-scope loads and adds them to its sum.
 * The poll is bounded: a workgroup that polls spin_limit times (each poll
 * about 64 clocks apart) without seeing everyone records a give-up and stops.
 *   rounds      >= 1                              (BITLINEAR_ERR_SHAPE)
 *   blocks      1 .. the device's compute units, so that all are resident
 *               at once                            (BITLINEAR_ERR_SHAPE)
 *   spin_limit  >= 1                              (BITLINEAR_ERR_ARG)
 *   state       uint32[2 + 2 * blocks], ZERO-FILLED by the caller; after the
 *               call state[0] = rounds * blocks and state[1] = 0 (give-ups)
 *               unless a workgroup gave up.
 *   sink        uint32[256 * blocks]; the 256 words of workgroup b add up
 *               (mod 2^32) to the sum over rounds r and workgroups i of
 *               r * blocks + i.
 */
int bitlinear_probe_barrier(int32_t rounds, int32_t blocks, int32_t spin_limit, uint32_t *state, uint32_t *sink,
                            void *stream);

/* Compute units of the current device, into *cus (the most workgroups
 * bitlinear_probe_barrier takes).  BITLINEAR_ERR_HIP if the query fails. */
int bitlinear_probe_compute_units(int32_t *cus);

#ifdef __cplusplus
}
#endif
#endif /* BITLINEAR_PROBE_H */
