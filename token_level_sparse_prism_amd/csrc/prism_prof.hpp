// prism_prof.hpp -- optional per-kernel timing with HIP events (off by default).  When enabled,
// every kernel is launched with a start and a stop event attached to its own dispatch
// (hipExtLaunchKernel), so the elapsed time between them is the kernel's execution on the GPU,
// not the surrounding queue gaps.  Results are aggregated per kernel name on query.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace prism {

bool prof_enabled();
// Per-thread switch that keeps prof_enabled() false (event creation may allocate; the
// allocation-free entry point turns timing off for its own launches).
void prof_suppress(bool on);
// Two timing events registered under `name`; false (and no events) when none can be created.
bool prof_pair(const char* name, hipEvent_t* begin, hipEvent_t* end);

template <typename F, typename... Args>
inline void launch_k(const char* name, F kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
    hipEvent_t b = nullptr, e = nullptr;
    if (prof_enabled() && prof_pair(name, &b, &e))
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, b, e, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

}  // namespace prism
