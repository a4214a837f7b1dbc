// sqllm_sparse.hip -- instantiations of the outlier-only kernel (y += S x).
#include "sqllm_device.h"

namespace sqllm {

hipError_t launch_spmv_add(const KernelArgs &a, int batch, const LaunchShape &ls, hipStream_t stream)
{
    LaunchShape one = ls;
    one.gw = 1; // no code groups in this mode
    return dev::launch_gw<3, kSparseAdd>(a, batch, one, stream);
}

} // namespace sqllm
