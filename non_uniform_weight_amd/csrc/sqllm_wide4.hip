// sqllm_wide4.hip -- instantiations of the 4-bit kernels at batch 9 to 16
// (matrix-core form only).
#include "sqllm_device.h"

namespace sqllm {

hipError_t launch_fused4_wide(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_batch<4, kFused, kMaxDotBatch + 1, kMaxBatch>(a, batch, ls, stream);
}

hipError_t launch_gemv4_wide(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_batch<4, kDenseOnly, kMaxDotBatch + 1, kMaxBatch>(a, batch, ls, stream);
}

hipError_t launch_group_fused4_wide(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_group_batch<4, kFused, kMaxDotBatch + 1, kMaxBatch>(g, batch, ls, stream);
}

hipError_t launch_group_gemv4_wide(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_group_batch<4, kDenseOnly, kMaxDotBatch + 1, kMaxBatch>(g, batch, ls, stream);
}

} // namespace sqllm
