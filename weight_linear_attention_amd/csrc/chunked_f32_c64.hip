// Instantiates the chunked forward for f32 inputs and chunks of 64 rows.
#include "chunked_kernels.h"

namespace fwa {
hipError_t launch_chunked_f32_c64(const ChunkPlan& p, hipStream_t s) {
    return launch_chunked_t<false, 64>(p, s);
}
}  // namespace fwa
