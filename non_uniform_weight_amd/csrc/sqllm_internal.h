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
constexpr int kMaxWaves = 16;     // waves per workgroup
constexpr int kMaxSplit = 64;     // workgroups sharing one row tile
constexpr int kTableBytes = 256 * 64 * 4;           // pair table: 256 entries x 64 lanes x half2
constexpr int kLdsBudget = 160 * 1024;              // LDS per compute unit on gfx950
constexpr int kSparseBatch = 4;   // 64-nonzero chunks a wave loads at once

enum Mode { kFused = 0, kDenseOnly = 1, kSparseAdd = 2 };

struct KernelArgs {
    const void *packed;       // packed codes (16-byte aligned)
    const uint16_t *lut;      // fp16 [rows][2^bits]
    const int32_t *row_ptr;   // [rows + 1]
    const uint16_t *col;      // [nnz]
    const uint16_t *val;      // fp16 [nnz]
    const uint16_t *x;        // fp16 [batch][cols]
    uint16_t *y;              // fp16 [batch][rows]
    unsigned long long *slots;  // workspace: one (fp32 sum, count) word per (tile, batch, row)
    int rows, cols, tiles, groups;
    int split;                // workgroups per row tile
    int gps;                  // column groups per workgroup (the last one may have fewer)
    int gpw;                  // column groups per wave
    int x_full;               // 1: every column of x is staged in LDS (outlier gathers read LDS)
};

// One launch configuration, chosen on the host.
struct LaunchShape {
    int waves;                // waves per workgroup
    int gw;                   // compiled groups-per-wave capacity (1..4)
    size_t dyn_lds;           // dynamic LDS bytes
};

// Most waves per workgroup a kernel holding gw groups of codes per wave and
// `batch` accumulators is compiled for: 16 (128 VGPRs each) while codes plus
// ~8 registers per batch column stay under 96 dwords, else 8.
constexpr int max_waves(int bits, int batch, int gw) { return gw * 8 * bits + 8 * batch >= 96 ? 8 : 16; }

hipError_t launch_dense_sparse(const KernelArgs &a, int bits, int batch, Mode mode, const LaunchShape &ls,
                               hipStream_t stream);
hipError_t launch_pack(const uint8_t *codes, int rows, int cols, int bits, void *packed, int *bad, hipStream_t stream);
hipError_t launch_unpack(const void *packed, const uint16_t *lut, int rows, int cols, int bits, uint8_t *codes,
                         uint16_t *w, hipStream_t stream);

// dynamic LDS of one workgroup: staged x (xgroups column groups of every
// batch column), the tile's row pointers, per-wave outlier row sums
inline size_t dynamic_lds_bytes(int xgroups, int batch, int waves, bool sparse)
{
    size_t b = (size_t)xgroups * kGroupCols * 2 * batch;
    if (sparse) b += 68 * 4 + (size_t)waves * batch * kTileRows * 4;
    return b;
}

} // namespace sqllm

#endif
