// k_refine_f32.hip -- refined layer, fp32 instantiations; the kernels are in refine_kernels.hpp.
#include "refine_kernels.hpp"

namespace prism {

hipError_t launch_refine_f32(const RefineArgs& a, int agg_max, hipStream_t st) { return refine_d<float>(a, agg_max, st); }

}  // namespace prism
