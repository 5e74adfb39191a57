// Host-side device queries of the launchers, cached per device.
//
// The CU count, a kernel's occupancy at a block size and LDS size, and the
// raised dynamic-LDS limit of a kernel depend only on the device and the
// kernel, so each is asked of the HIP runtime once per (device, kernel,
// block size, LDS bytes) and kept for the life of the process.  Eager calls
// then pay a thread-local device lookup and a short locked map probe instead
// of several runtime queries.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace aqg {
namespace detail {

// CU count of the current device.
hipError_t device_cus(int& cus);

// hipOccupancyMaxActiveBlocksPerMultiprocessor on the current device.
hipError_t occupancy(int& blocks_per_cu, const void* fn, int threads, size_t lds_bytes);

// Raise fn's dynamic LDS limit to `bytes` on the current device (once).
hipError_t raise_lds_limit(const void* fn, size_t bytes);

}  // namespace detail
}  // namespace aqg
