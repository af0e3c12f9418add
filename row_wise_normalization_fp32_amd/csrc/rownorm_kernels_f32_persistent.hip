// Kernel instances for f32 I/O: persistent launches (see rownorm_kernels.hpp).
#include "rownorm_kernels.hpp"

namespace rn {

hipError_t launch_f32_persistent(int op, const Plan& plan, const Params& p, hipStream_t stream) {
    return launch_dtype<DT_F32, true>(op, plan, p, stream);
}

}  // namespace rn
