// Host-side helpers shared by the C-ABI entry points: the argument checks
// (mha_validate.hpp) and the per-device architecture check.
#pragma once

#include "../../include/mha.h"
#include "mha_validate.hpp"

#include <hip/hip_runtime.h>

namespace mha_host {

// MHA_OK if the current HIP device is a gfx950 (cached per device),
// MHA_ERR_UNSUPPORTED for another architecture, MHA_ERR_DEVICE without one.
mha_status_t check_device();

}  // namespace mha_host
