// k_scan2.hip -- the proposal scan over 2-bit (INT2) keys; the kernel is in scan_kernel.hpp.
#include "scan_kernel.hpp"

namespace prism {

hipError_t launch_scan2(const ProposeArgs& a, int agg_max, hipStream_t st) { return launch_scan_kb<2>(a, agg_max, st); }

}  // namespace prism
