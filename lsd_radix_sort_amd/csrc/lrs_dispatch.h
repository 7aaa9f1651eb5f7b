// lrs_dispatch.h -- how the library hands one kernel to the runtime
// (internal header): the stream, and the timer's events when a caller times
// the kernel.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace lrs {

// Where a kernel goes: its stream and, when a caller times it, the events
// that the dispatch itself stamps with the kernel's start and end (no marker
// of their own between kernels; null for an untimed launch).
struct Launch {
    hipStream_t s = nullptr;
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// An untimed kernel goes through the plain launch, which costs the host about
// half as much per launch as the extended launch that carries events.
#ifndef LRS_PLAIN_UNTIMED
#define LRS_PLAIN_UNTIMED 1
#endif
template <typename Kernel, typename... Args>
inline void launch_on(Kernel kernel, dim3 grid, dim3 block, const Launch &L, Args... args) {
    if (LRS_PLAIN_UNTIMED && L.start == nullptr && L.stop == nullptr)
        hipLaunchKernelGGL(kernel, grid, block, 0, L.s, args...);
    else
        hipExtLaunchKernelGGL(kernel, grid, block, 0, L.s, L.start, L.stop, 0, args...);
}

}  // namespace lrs
