// Kernel instances for bf16 I/O: persistent launches (see rownorm_kernels.hpp).
#include "rownorm_kernels.hpp"

namespace rn {

hipError_t launch_bf16_persistent(int op, const Plan& plan, const Params& p, hipStream_t stream) {
    return launch_dtype<DT_BF16, true>(op, plan, p, stream);
}

}  // namespace rn
