// placeholder until the large-chunk linear kernels land
#include "kernels.h"
namespace ttt {
bool large_chunk_linear_supported(int64_t, int64_t, int64_t, int) { return false; }
size_t large_chunk_linear_workspace(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t) { return 0; }
hipError_t launch_large_chunk_linear(const LargeChunkArgs&, hipStream_t) { return hipErrorNotSupported; }
bool large_chunk_swiglu_supported(int64_t, int64_t, int64_t, int) { return false; }
size_t large_chunk_swiglu_workspace(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t) { return 0; }
hipError_t launch_large_chunk_swiglu(const LargeChunkArgs&, hipStream_t) { return hipErrorNotSupported; }
}
