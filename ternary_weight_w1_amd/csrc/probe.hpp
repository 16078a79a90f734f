// Launchers of the calibration probes (defined in probes.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

hipError_t launch_probe_read(const void *buf, int64_t bytes, int64_t chunk_bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_probe_mfma(int64_t iters, int a, int b, int blocks, int32_t *sink, hipStream_t s);
hipError_t launch_probe_mfma_data(int64_t iters, const void *ops, int blocks, int32_t *sink, uint64_t *clocks,
                                  hipStream_t s);
hipError_t probe_mfma_resident_blocks(int *blocks);
hipError_t launch_probe_barrier(int rounds, int blocks, int spin_limit, uint32_t *state, uint32_t *sink,
                                hipStream_t s);
hipError_t probe_compute_units(int *cus);

}  // namespace bl
