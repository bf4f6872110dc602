// Head-estimator variants for bf16 cached logits.
#include "head_impl.hpp"

namespace dust {
hipError_t launch_head_bf16(const HeadPlan& plan, const HeadArgs& args, hipStream_t stream) {
    return dispatch_head<1>(plan, args, stream);
}
}  // namespace dust
