// sqllm_wide2.hip -- instantiations of the 2-bit kernels at batch 9 to 16
// (matrix-core form only).
#include "sqllm_device.h"

namespace sqllm {

hipError_t launch_fused2_wide(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_batch<2, kFused, kMaxDotBatch + 1, kMaxBatch>(a, batch, ls, stream);
}

hipError_t launch_gemv2_wide(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_batch<2, kDenseOnly, kMaxDotBatch + 1, kMaxBatch>(a, batch, ls, stream);
}

hipError_t launch_group_fused2_wide(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_group_batch<2, kFused, kMaxDotBatch + 1, kMaxBatch>(g, batch, ls, stream);
}

hipError_t launch_group_gemv2_wide(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_group_batch<2, kDenseOnly, kMaxDotBatch + 1, kMaxBatch>(g, batch, ls, stream);
}

} // namespace sqllm
