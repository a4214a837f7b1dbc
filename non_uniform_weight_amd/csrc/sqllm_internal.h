// sqllm_internal.h -- declarations shared by the C-ABI layer and the kernels
// (plain C++, no HIP types except the runtime's status and stream handles).
#ifndef SQLLM_INTERNAL_H
#define SQLLM_INTERNAL_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace sqllm {

constexpr int kTileRows = 64;     // rows per tile = lanes per wave
constexpr int kGroupCols = 256;   // codes per group
constexpr int kMaxBatch = 8;
constexpr int kMaxWaves = 8;      // waves per workgroup
constexpr int kSplitCap = 16;     // most workgroups sharing one row tile

struct KernelArgs {
    const void *packed;       // packed codes (16-byte aligned)
    const uint16_t *lut;      // fp16 [rows][2^bits]
    const int32_t *row_ptr;   // [rows + 1]
    const uint16_t *col;      // [nnz]
    const uint16_t *val;      // fp16 [nnz]
    const uint16_t *x;        // fp16 [batch][cols]
    uint16_t *y;              // fp16 [batch][rows]
    float *part;              // workspace: fp32 partials [tiles][split][batch][64]
    uint32_t *counters;       // workspace: one arrival counter per tile
    int rows, cols, tiles, groups;
    int split;                // workgroups per row tile
    int gps;                  // column groups per split
};

hipError_t launch_dense_sparse(const KernelArgs &a, int bits, int batch, bool dense, bool sparse, bool add_y,
                               int waves, hipStream_t stream);
hipError_t launch_pack(const uint8_t *codes, int rows, int cols, int bits, void *packed, int *bad, hipStream_t stream);
hipError_t launch_unpack(const void *packed, const uint16_t *lut, int rows, int cols, int bits, uint8_t *codes,
                         uint16_t *w, hipStream_t stream);

} // namespace sqllm

#endif
