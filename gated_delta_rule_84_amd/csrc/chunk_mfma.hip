// chunk_mfma.hip -- bf16 matrix-core prefill kernel (gfx950).  Not enabled yet:
// every shape currently runs the fp32 vector-ALU kernel.
#include "gdr_internal.hpp"

namespace gdr {
bool chunk_mfma_supported(const ChunkParams &) { return false; }
size_t chunk_mfma_workspace(const ChunkParams &) { return 0; }
hipError_t launch_chunk_mfma(const ChunkParams &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gdr
