// prism_prof.hpp -- optional per-kernel timing with HIP events (off by default).  When enabled,
// every kernel launch is bracketed by two events recorded on the launch stream; results are
// aggregated per kernel name on query.
#pragma once

#include <hip/hip_runtime.h>

namespace prism {

bool prof_enabled();
void prof_mark(const char* name, hipStream_t st, bool begin);

struct ProfScope {
    const char* name;
    hipStream_t st;
    bool on;
    ProfScope(const char* n, hipStream_t s) : name(n), st(s), on(prof_enabled()) {
        if (on) prof_mark(name, st, true);
    }
    ~ProfScope() {
        if (on) prof_mark(name, st, false);
    }
};

}  // namespace prism
