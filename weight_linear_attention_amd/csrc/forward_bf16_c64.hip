// Instantiates the chunked forward kernel for bf16 inputs and chunks of 64 rows.
#include "forward_kernel.h"

namespace fwa {
hipError_t launch_fwd_bf16_c64(const FwdPlan& p, int BH, hipStream_t s) {
    return launch_fwd_dispatch<true, 64>(p, BH, s);
}
}  // namespace fwa
