// Backward kernel instances for bf16 I/O (see rownorm_backward.hpp).
#include "rownorm_backward.hpp"

namespace rn {

hipError_t launch_bwd_bf16(int op, const Plan& plan, const BwdParams& p, const BwdColParams& cp, hipStream_t stream) {
    return launch_bwd_dtype<DT_BF16>(op, plan, p, cp, stream);
}

}  // namespace rn
