// launch.hpp -- host-side entry points of the kernels (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <tuple>
#include <type_traits>
#include <utility>

#include "common.hpp"

namespace ra {

// Launches `kernel` with its arguments converted to the kernel's parameter
// types.  With a start or stop event (profiled calls) the launch goes
// through hipExtLaunchKernel, which records the events at the kernel's own
// start and end, so that the pair brackets the kernel's execution alone;
// otherwise through hipLaunchKernel.
template <typename... P, typename... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop, A &&...args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<std::decay_t<P>...> values(std::forward<A>(args)...);
    void *ptrs[sizeof...(P) ? sizeof...(P) : 1];
    std::apply([&](auto &...v) {
        int i = 0;
        ((ptrs[i++] = (void *)&v), ...);
    }, values);
    if (ev_start || ev_stop)
        return hipExtLaunchKernel((const void *)kernel, grid, block, ptrs, shmem, stream, ev_start, ev_stop, 0);
    return hipLaunchKernel((const void *)kernel, grid, block, ptrs, shmem, stream);
}

// ev_start / ev_stop (may be null): events given to the kernel launch.
hipError_t launch_generic(const Params &p, hipStream_t stream, hipEvent_t ev_start = nullptr,
                          hipEvent_t ev_stop = nullptr);
bool generic_supports(int D);

}  // namespace ra
