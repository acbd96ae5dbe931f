// chunk_mfma.hip -- placeholder until the MFMA path lands.
#include "kernels.h"

namespace gdn2 {

bool chunk_mfma_supported(const ChunkArgs &) { return false; }

hipError_t launch_chunk_mfma(const ChunkArgs &, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace gdn2
