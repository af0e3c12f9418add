// Kernel instances for f16 I/O: grid-per-row launches and the general kernel (see
// rownorm_kernels.hpp). One translation unit per dtype and mode so they compile in parallel.
#include "rownorm_kernels.hpp"

namespace rn {

hipError_t launch_f16(int op, const Plan& plan, const Params& p, hipStream_t stream) {
    return launch_dtype<DT_F16, false>(op, plan, p, stream);
}

}  // namespace rn
