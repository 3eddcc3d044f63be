// temporary: entry points whose kernels are not written yet
#include "launch.h"
namespace sa {
hipError_t launch_indexer(const uint16_t*, const uint16_t*, const float*, int, int, int64_t, int64_t, float*, hipStream_t) { return hipErrorNotSupported; }
size_t vs_workspace_bytes(int64_t, int64_t) { return 0; }
hipError_t launch_vs_estimate(const uint16_t*, const uint16_t*, int, int, int, int64_t, int, int, float, float*, float*, void*, hipStream_t) { return hipErrorNotSupported; }
}
