// Instantiates the chunked forward for bf16 inputs and chunks of 64 rows.
#include "chunked_kernels.h"

namespace fwa {
hipError_t launch_chunked_bf16_c64(const ChunkPlan& p, hipStream_t s) {
    return launch_chunked_t<true, 64>(p, s);
}
}  // namespace fwa
