// lion_birnn.hip -- bidirectional RNN form (in progress).
#include "lion_device.h"
#include "lion_internal.h"

namespace lion {
size_t birnn_workspace_bytes(int, int, int, int) { return 0; }
hipError_t launch_birnn(const AttnArgs &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace lion
