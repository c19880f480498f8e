// probe_launch.hpp -- host launchers of the machine-peak probes (k_probe.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace sgqa {

hipError_t launch_probe_mfma(int waves, int iters, float *sink, hipStream_t stream);
hipError_t launch_probe_read(const void *buf, int64_t bytes, uint32_t *sink, int blocks,
                             hipStream_t stream);
hipError_t launch_probe_gather(const void *table, int row16, const int32_t *idx, int64_t n,
                               uint32_t *sink, int blocks, hipStream_t stream);

} // namespace sgqa
