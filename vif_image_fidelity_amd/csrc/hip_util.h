// hip_util.h -- small host-side HIP helpers shared by the library's C-ABI
// translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime_api.h>

namespace vifk {

// Makes a context's device current for the scope of one call and restores
// the caller's device afterwards.
class DeviceScope {
public:
  explicit DeviceScope(int dev) {
    if (hipGetDevice(&prev_) != hipSuccess)
      prev_ = -1;
    if (prev_ != dev)
      err_ = hipSetDevice(dev);
  }
  ~DeviceScope() {
    int cur = -1;
    if (prev_ >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev_)
      (void)hipSetDevice(prev_);
  }
  DeviceScope(const DeviceScope &) = delete;
  DeviceScope &operator=(const DeviceScope &) = delete;
  hipError_t error() const { return err_; }

private:
  int prev_ = -1;
  hipError_t err_ = hipSuccess;
};

// Destroys an event if it exists and clears the handle.
inline void destroy_event(hipEvent_t &e) {
  if (e) {
    (void)hipEventDestroy(e);
    e = nullptr;
  }
}

} // namespace vifk
