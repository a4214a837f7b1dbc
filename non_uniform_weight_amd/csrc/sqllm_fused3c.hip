// sqllm_fused3c.hip -- instantiations of the 3-bit fused kernels with the
// compact pair table (matrix-core form, batch 2 to 8).
#include "sqllm_device.h"

namespace sqllm {

hipError_t launch_fused3_compact(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_batch<3, kFused, 2, kMaxDotBatch, true>(a, batch, ls, stream);
}

hipError_t launch_group_fused3_compact(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_group_batch<3, kFused, 2, kMaxDotBatch, true>(g, batch, ls, stream);
}

} // namespace sqllm
