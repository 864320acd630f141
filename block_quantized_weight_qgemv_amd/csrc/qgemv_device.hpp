// Host-side helpers shared by the entry points of every kernel family.
#pragma once

#include <cstdint>

namespace qgl {

// Compute units of the current device, read once per device and cached
// (thread-safe); 0 when there is no usable device or the query fails.
// Defined in qgemv_api.hip.
int device_cu_count();

inline bool aligned_to(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace qgl
