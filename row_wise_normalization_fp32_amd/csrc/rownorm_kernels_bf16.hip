// Kernel instances for bf16 I/O: grid-per-row launches, the element, split-row and general kernels (see
// rownorm_kernels.hpp). One translation unit per dtype and mode so they compile in parallel.
#include "rownorm_kernels.hpp"

namespace rn {

hipError_t launch_bf16(int op, const Plan& plan, const Params& p, hipStream_t stream) {
    return launch_dtype<DT_BF16, false>(op, plan, p, stream);
}

hipError_t launch_wide_bf16(int op, const Plan& plan, const Params& p, const WideArgs& wa, hipStream_t stream) {
    return launch_wide<DT_BF16>(op, plan, p, wa, stream);
}

}  // namespace rn
