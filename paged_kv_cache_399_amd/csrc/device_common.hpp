// Helpers shared by the HIP translation units.
#pragma once

#include <cstdint>

#include "pkv.h"

namespace pkv {

// Device address of the current device's error word (PKV_DEVERR_* bits that
// kernels OR in with a vector atomic).  Looked up once per device.
int device_error_word(int32_t** out);

}  // namespace pkv
