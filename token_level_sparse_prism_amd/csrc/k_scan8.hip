// k_scan8.hip -- the proposal scan over int8 keys; the kernel is in scan_kernel.hpp.
#include "scan_kernel.hpp"

namespace prism {

hipError_t launch_scan8(const ProposeArgs& a, int agg_max, hipStream_t st) { return launch_scan_kb<8>(a, agg_max, st); }

}  // namespace prism
