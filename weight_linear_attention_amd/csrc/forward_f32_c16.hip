// Instantiates the chunked forward kernel for f32 inputs and chunks of 16 rows.
#include "forward_kernel.h"

namespace fwa {
hipError_t launch_fwd_f32_c16(const FwdPlan& p, int BH, hipStream_t s) {
    return launch_fwd_dispatch<false, 16>(p, BH, s);
}
}  // namespace fwa
