// Host-side helpers for the device entry points: alignment checks and the
// status of the last launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

inline bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline pkv_status launch_status() {
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // namespace pkv
