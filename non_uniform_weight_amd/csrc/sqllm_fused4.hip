// sqllm_fused4.hip -- instantiations of the 4-bit fused kernels (y = (D + S) x).
#include "sqllm_device.h"

namespace sqllm {

hipError_t launch_fused4(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_batch<4, kFused, 1, kMaxDotBatch>(a, batch, ls, stream);
}

hipError_t launch_group_fused4(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_group_batch<4, kFused, 1, kMaxDotBatch>(g, batch, ls, stream);
}

} // namespace sqllm
