// Instantiates the chunked forward for f32 inputs and chunks of 32 rows.
#include "chunked_kernels.h"

namespace fwa {
hipError_t launch_chunked_f32_c32(const ChunkPlan& p, hipStream_t s) {
    return launch_chunked_t<false, 32>(p, s);
}
}  // namespace fwa
