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

// ---- per-workgroup phase timeline (diagnostics; compiled in only with PRISM_TIMELINE=1) -------
// Thread 0 of each workgroup stores the 100 MHz real-time counter at the kernel's phase points
// into a device array of its translation unit: [kernel slot][workgroup][phase].  Each launch
// overwrites its workgroups' entries; prism_timeline_read merges the translation units' arrays.
// The normal library build compiles every stamp to nothing.
enum TlKernel { kTlScan = 0, kTlCand, kTlCompact, kTlRscore, kTlAttend, kTlSelect, kTlRows, kTlAttendD, kTlKernels };
constexpr int kTlWgs = 8192;
constexpr int kTlPhases = 8;
#ifndef PRISM_TIMELINE
#define PRISM_TIMELINE 0
#endif
#if PRISM_TIMELINE
void tl_register(hipError_t (*copy)(unsigned long long*, size_t), hipError_t (*clear)());
static __device__ unsigned long long g_tl[kTlKernels * kTlWgs * kTlPhases];
static hipError_t tl_copy_tu(unsigned long long* h, size_t n) { return hipMemcpyFromSymbol(h, HIP_SYMBOL(g_tl), n * 8); }
static hipError_t tl_clear_tu() {
    static unsigned long long zeros[kTlKernels * kTlWgs * kTlPhases];
    return hipMemcpyToSymbol(HIP_SYMBOL(g_tl), zeros, sizeof(zeros));
}
static const bool g_tl_registered = (tl_register(&tl_copy_tu, &tl_clear_tu), true);
__device__ __forceinline__ void tl_stamp(int k, int phase) {
    if (threadIdx.x == 0) {
        const unsigned wg = blockIdx.x + blockIdx.y * gridDim.x;
        if (wg < unsigned(kTlWgs)) g_tl[(size_t(k) * kTlWgs + wg) * kTlPhases + phase] = __builtin_amdgcn_s_memrealtime();
    }
}
#define PRISM_TL(k, ph) ::prism::tl_stamp((k), (ph))
#else
#define PRISM_TL(k, ph) ((void)0)
#endif

template <typename F, typename... Args>
inline void launch_k(const char* name, F kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
    hipEvent_t b = nullptr, e = nullptr;
    if (prof_enabled() && prof_pair(name, &b, &e))
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, b, e, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

}  // namespace prism
