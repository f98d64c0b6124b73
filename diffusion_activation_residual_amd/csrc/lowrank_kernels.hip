// lowrank_kernels.hip -- placeholder until the subspace-iteration kernels land.
#include "cfz_internal.h"

namespace cfz {

size_t lowrank_workspace_bytes(int64_t batch, int64_t m, int64_t n, int r)
{
    return 256;
}

hipError_t launch_lowrank(const LowrankArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace cfz
