// k_refine.hip -- refined layer (bf16 instantiations and the dtype dispatch); the kernels are in
// refine_kernels.hpp.
#include "refine_kernels.hpp"

namespace prism {

hipError_t launch_refine_f32(const RefineArgs& a, int agg_max, hipStream_t st);

hipError_t launch_refine(const RefineArgs& a, int bf16, int agg_max, hipStream_t st) {
    return bf16 ? refine_d<uint16_t>(a, agg_max, st) : launch_refine_f32(a, agg_max, st);
}

}  // namespace prism
