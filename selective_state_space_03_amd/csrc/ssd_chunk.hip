// Chunked SSD scan (placeholder until the MFMA kernel lands).
#include "ssm_internal.h"

namespace ssm {

size_t chunk_workspace_bytes(int, int, int, int, int) { return 0; }

hipError_t launch_chunk(const ChunkLaunch&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ssm
