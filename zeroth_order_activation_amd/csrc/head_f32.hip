// Head-estimator variants for f32 cached logits.
#include "head_impl.hpp"

namespace dust {
hipError_t launch_head_f32(const HeadPlan& plan, const HeadArgs& args, hipStream_t stream) {
    return dispatch_head<0>(plan, args, stream);
}
}  // namespace dust
