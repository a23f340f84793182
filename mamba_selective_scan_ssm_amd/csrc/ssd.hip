// Mamba-2 SSD chunked scan (placeholder until the matrix-core kernels land).
#include "launch.h"

namespace ssm {

int64_t ssd_ws_bytes(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_ssd(const SSDArgs &, void *, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ssm
