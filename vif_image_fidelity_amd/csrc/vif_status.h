// vif_status.h -- thread-local error state of the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include "../../include/vif.h"

namespace vifk {

// Records code (and, for VIF_EHIP, the HIP error) for vif_errno() and
// vif_strerror() on the calling thread; returns code.
int set_status(int code, hipError_t hip = hipSuccess);

// VIF_OK for hipSuccess, VIF_ENOMEM for an allocation failure, VIF_EHIP
// otherwise; recorded as by set_status().
int status_from_hip(hipError_t e);

} // namespace vifk
