// device_checks.h -- per-device, run-once checks before the first launches.
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>
#include <unordered_map>

namespace dsa {

// Result of a check per device id.
struct PerDeviceCache {
  std::mutex mu;
  std::unordered_map<int, hipError_t> done;
};

// Runs fn() once on the current device and caches its result.
hipError_t once_per_device(PerDeviceCache& cache, hipError_t (*fn)());

// hipSuccess when `kernel` can be launched with `threads` threads and
// `dyn_lds` bytes of dynamic LDS on the current device (block-size limit,
// static + dynamic LDS against the device's per-workgroup maximum, at most
// 512 registers a lane); hipErrorInvalidConfiguration otherwise.
hipError_t check_launch_limits(const void* kernel, int threads, size_t dyn_lds);

}  // namespace dsa
