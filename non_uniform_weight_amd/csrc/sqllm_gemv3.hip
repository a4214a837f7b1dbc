// sqllm_gemv3.hip -- instantiations of the 3-bit gemv kernels (y = D x).
#include "sqllm_device.h"

namespace sqllm {

hipError_t launch_gemv3(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_batch<3, kDenseOnly, 1, kMaxDotBatch>(a, batch, ls, stream);
}

hipError_t launch_group_gemv3(const GroupArgs &g, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_group_batch<3, kDenseOnly, 1, kMaxDotBatch>(g, batch, ls, stream);
}

} // namespace sqllm
