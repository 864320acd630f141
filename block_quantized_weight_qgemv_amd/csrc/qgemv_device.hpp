// Host-side helpers shared by the entry points of every kernel family.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <tuple>
#include <utility>

#include "qgemv.h"

namespace qgl {

// Compute units of the current device, read once per device and cached
// (thread-safe); 0 when there is no usable device or the query fails.
// Defined in qgemv_api.hip.
int device_cu_count();

inline bool aligned_to(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <class... KArgs, size_t... I>
inline hipError_t launch_packed(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                                std::tuple<KArgs...> &vals, std::index_sequence<I...>) {
    void *ptrs[sizeof...(KArgs)] = {static_cast<void *>(&std::get<I>(vals))...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), grid, block, ptrs, lds, stream);
}

// Enqueue kern<<<grid, block, lds, stream>>>(args...) and return the status
// of that launch itself (hipLaunchKernel's result).  The thread's last-error
// state is neither read nor cleared here, so an error an earlier, unrelated
// HIP call left behind is not reported as this launch's failure.
template <class... KArgs, class... Args>
inline qg_status launch_kernel(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                               Args &&...args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count of the kernel");
    std::tuple<KArgs...> vals(std::forward<Args>(args)...);
    const hipError_t e = launch_packed(kern, grid, block, lds, stream, vals, std::index_sequence_for<KArgs...>{});
    return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH;
}

}  // namespace qgl
