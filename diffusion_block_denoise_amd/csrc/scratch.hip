// The library's static device scratch: a file-scope device array that holds the partial results
// of a handle made by dllm_create_static_scratch (split-K partial tiles, attention key-chunk
// partials, lm_head tile partials), for callers that cannot allocate device memory.  Every GPU
// the library runs on gets its own copy when the code object is loaded there and keeps it until
// the process ends.  Handles on one GPU share it: their calls must not overlap in time.
#include "kernels.h"

#include <map>
#include <mutex>

namespace dllm {

static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

// Device address of the current device's copy of `scratch`.  In host code the array's name is a
// host-side stand-in, not a device address: kernels and copies get this address instead.  Looked
// up once per device (with that device current) and kept.
hipError_t static_scratch_address(void **ptr) {
  static std::mutex mu;
  static std::map<int, void *> per_device;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  const auto it = per_device.find(dev);
  if (it != per_device.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  void *p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  per_device[dev] = p;
  *ptr = p;
  return hipSuccess;
}

}  // namespace dllm
