// sqllm_noalloc.hip -- sqllm_dense_sparse_gemv_noalloc: the fused product
// for callers that may not allocate device memory.  Its workspace (the
// split-combine words and the transposed x) is a file-scope device array of
// fixed size, of which each GPU holds its own copy from the library's load
// until the process ends.  The product itself is sqllm_dense_sparse_gemv's:
// same checks, launch choice and kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "sqllm.h"
#include "sqllm_internal.h"

namespace {

constexpr size_t kScratchBytes = SQLLM_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch must hold whole 256-byte blocks");

// In host code this name stands for the symbol only; the array's device
// address on a GPU comes from hipGetSymbolAddress with that GPU current.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    void *ptr = nullptr;   // device address of `scratch` on this GPU
    bool clean = false;    // every byte known to be zero (set by the first call's clear)
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

__global__ void __launch_bounds__(256) clear_scratch(uint4 *p, size_t n)
{
    const uint4 z = {0u, 0u, 0u, 0u};
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = z;
}

// The device address of this GPU's array for a call on `stream`; on the
// first call on a GPU (and after a failed launch) the array is zero-filled
// on `stream`, ahead of the call's kernels.
sqllm_status device_scratch(hipStream_t stream, DeviceScratch **out)
{
    int dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SQLLM_ERR_HIP;
    DeviceScratch &d = g_dev[dev];
    if (!d.ptr) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return SQLLM_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return SQLLM_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return SQLLM_ERR_HIP;
        if (e != hipSuccess || !p || ((uintptr_t)p & 255) != 0) return SQLLM_ERR_HIP;
        d.ptr = p;
    }
    if (!d.clean) {
        hipLaunchKernelGGL(clear_scratch, dim3(1024), dim3(256), 0, stream, (uint4 *)d.ptr, kScratchBytes / 16);
        if (hipGetLastError() != hipSuccess) return SQLLM_ERR_HIP;
        d.clean = true;
    }
    *out = &d;
    return SQLLM_OK;
}

} // namespace

extern "C" sqllm_status sqllm_dense_sparse_gemv_noalloc(const void *packed, const uint16_t *lut, int bits,
                                                        const int32_t *row_ptr, const uint16_t *col_idx,
                                                        const uint16_t *val, int64_t nnz, int64_t rows, int64_t cols,
                                                        const uint16_t *x, int batch, uint16_t *y,
                                                        hipStream_t stream)
{
    // Argument errors first, without touching the device (a call without a
    // workspace reports them before its workspace check).
    if (sqllm_workspace_bytes(rows, cols, batch) == 0)
        return sqllm_dense_sparse_gemv(packed, lut, bits, row_ptr, col_idx, val, nnz, rows, cols, x, batch, y,
                                       nullptr, 0, stream);
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch *d = nullptr;
    sqllm_status st = device_scratch(stream, &d);
    if (st != SQLLM_OK) return st;
    st = sqllm_dense_sparse_gemv(packed, lut, bits, row_ptr, col_idx, val, nnz, rows, cols, x, batch, y, d->ptr,
                                 kScratchBytes, stream);
    if (st == SQLLM_ERR_WORKSPACE) return SQLLM_ERR_SCRATCH; // the launch's words exceed the array
    if (st == SQLLM_ERR_HIP) d->clean = false;                // a launch may have stopped half way
    return st;
}
