// sqllm_wide3.hip -- instantiations of the 3-bit kernels at batch 9 to 16
// (matrix-core form only) and of the outlier-only kernel at those batches.
#include "sqllm_device.h"

namespace sqllm {

hipError_t launch_fused3_wide(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_batch<3, kFused, kMaxDotBatch + 1, kMaxBatch>(a, batch, ls, stream);
}

hipError_t launch_gemv3_wide(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_batch<3, kDenseOnly, kMaxDotBatch + 1, kMaxBatch>(a, batch, ls, stream);
}

hipError_t launch_group_fused3_wide(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_group_batch<3, kFused, kMaxDotBatch + 1, kMaxBatch>(g, batch, ls, stream);
}

hipError_t launch_group_gemv3_wide(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_group_batch<3, kDenseOnly, kMaxDotBatch + 1, kMaxBatch>(g, batch, ls, stream);
}

hipError_t launch_spmv_add_wide(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_batch<3, kSparseAdd, kMaxDotBatch + 1, kMaxBatch>(a, batch, ls, stream);
}

} // namespace sqllm
