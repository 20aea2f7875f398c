// lion_chunk.hip -- chunkwise form (in progress).
#include "lion_device.h"
#include "lion_internal.h"

namespace lion {
size_t chunk_workspace_bytes(int, int, int, int, int) { return 0; }
hipError_t launch_chunk(const AttnArgs &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace lion
