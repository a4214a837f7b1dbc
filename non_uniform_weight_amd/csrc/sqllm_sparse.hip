// sqllm_sparse.hip -- instantiations of the outlier-only kernel (y += S x).
#include "sqllm_device.h"

namespace sqllm {

hipError_t launch_spmv_add(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    return dev::launch_batch<3, kSparseAdd, 1, kMaxDotBatch>(a, batch, ls, stream);
}

} // namespace sqllm
